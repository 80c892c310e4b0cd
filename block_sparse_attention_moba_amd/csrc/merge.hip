// Online-softmax merge of a query row's partial outputs (write-up "MoBA:
// Mixture of Block Attention", implementation step five: a query attends its
// own block and several history blocks, so the per-block results are combined
// with the softmax renormalisation).  Each partial o_j is normalised within
// its block and carries its base-2 log-sum-exp l_j; the row's output is
//     sum_j 2^(l_j - L) o_j,  L = log2 sum_j 2^l_j,
// taken against the largest l_j for range.  The row's own log-sum-exp L (as a
// natural log) is also written when the caller asks for it.  Slots 0 .. npast-1 hold the past
// blocks, slot topk-1 the own block; rows without past blocks were written
// by the own-block pass directly and are skipped here.
//
// Bandwidth-bound: D/8 lanes per row, one 8-element piece each, every slot
// read once with whole-row coalesced loads; small register use keeps many
// waves resident to cover the load latency.
#include "moba_internal.hpp"

namespace moba {

namespace {

__device__ inline void load8(const __bf16 *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

__device__ inline void load8(const float *p, float *f) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ inline void store8(__bf16 *p, const float *f) {
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
    *reinterpret_cast<bf16x8_t *>(p) = v;
}

__device__ inline void store8(float *p, const float *f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// grid ceil(rows / (256 / (D / 8))), 256 threads; rows ordered (batch, head,
// token of the chunk [r0, r0 + R)), partial buffers chunk-local.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(const T *__restrict__ part_o,
                                                    const float *__restrict__ part_lse,
                                                    T *__restrict__ out,
                                                    float *__restrict__ lse_out, int S, int Hq,
                                                    int B, int topk, int nslot, long long rows,
                                                    int r0, int R) {
    constexpr int LPR = D / 8;
    constexpr int RPW = 256 / LPR;
    const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
    const int ch = threadIdx.x % LPR;
    if (row >= rows) return;
    const int t = r0 + (int)(row % R);
    const long long bh = row / R;
    const int h = (int)(bh % Hq), b = (int)(bh / Hq);
    const int npast = min(topk - 1, t / B);
    if (npast == 0) return;
    const float *ls = part_lse + row * nslot;
    const T *po = part_o + row * nslot * D + ch * 8;
    const float l_own = ls[nslot - 1];
    float mx = l_own;
    for (int s = 0; s < npast; ++s) mx = fmaxf(mx, ls[s]);
    float o[8];
    load8(po + (size_t)(nslot - 1) * D, o);
    const float w_own = exp2f(l_own - mx);
    float wsum = w_own;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= w_own;
    for (int s = 0; s < npast; ++s) {
        const float w = exp2f(ls[s] - mx);
        wsum += w;
        float f[8];
        load8(po + (size_t)s * D, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w, f[e], o[e]);
    }
    const float iw = 1.f / wsum;
    if (lse_out && ch == 0) lse_out[((size_t)b * Hq + h) * S + t] = (mx + log2f(wsum)) * kLn2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= iw;
    store8(out + (((size_t)b * S + t) * Hq + h) * D + ch * 8, o);
}

template <typename T, int D>
hipError_t merge_impl(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    constexpr int RPW = 256 / (D / 8);
    const long long rows = (long long)p.batch * p.Hq * p.R;
    merge_kernel<T, D><<<(unsigned)((rows + RPW - 1) / RPW), 256, 0, st>>>(
        static_cast<const T *>(bf.part_o), bf.part_lse, static_cast<T *>(bf.out), bf.lse_out, p.S,
        p.Hq, p.B,
        p.topk, part_slots(p), rows, p.r0, p.R);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    if (p.dtype == kBF16)
        return p.D == 64 ? merge_impl<__bf16, 64>(bf, p, st) : merge_impl<__bf16, 128>(bf, p, st);
    return p.D == 64 ? merge_impl<float, 64>(bf, p, st) : merge_impl<float, 128>(bf, p, st);
}

}  // namespace moba
