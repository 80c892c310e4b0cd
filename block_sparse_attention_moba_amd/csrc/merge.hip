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

// raw 8-element pieces, loaded first and widened when used
template <typename T> struct Piece;
template <> struct Piece<__bf16> { uint4 u; };
template <> struct Piece<float> { float4 a, b; };
__device__ inline void loadp(const __bf16 *p, Piece<__bf16> &x) { x.u = *reinterpret_cast<const uint4 *>(p); }
__device__ inline void loadp(const float *p, Piece<float> &x) {
    x.a = *reinterpret_cast<const float4 *>(p);
    x.b = *reinterpret_cast<const float4 *>(p + 4);
}
__device__ inline void widen(const Piece<__bf16> &x, float *f) {
    const uint32_t w[4] = {x.u.x, x.u.y, x.u.z, x.u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ inline void widen(const Piece<float> &x, float *f) {
    f[0] = x.a.x; f[1] = x.a.y; f[2] = x.a.z; f[3] = x.a.w;
    f[4] = x.b.x; f[5] = x.b.y; f[6] = x.b.z; f[7] = x.b.w;
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
// token of the chunk [r0, r0 + R)), partial buffers chunk-local.  NS > 0: at
// most NS past slots, all loads issued before any is used (slots past the
// row's count read its last past slot again and get weight 0); NS = 0: a loop
// over any count.
template <typename T, int D, int NS>
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
    float o[8];
    float wsum;
    if constexpr (NS > 0) {
        float lv[NS];
        Piece<T> pc[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int sc = min(s, npast - 1);
            lv[s] = ls[sc];
            loadp(po + (size_t)sc * D, pc[s]);
        }
        load8(po + (size_t)(nslot - 1) * D, o);
#pragma unroll
        for (int s = 0; s < NS; ++s) mx = fmaxf(mx, lv[s]);     // repeats of a slot change nothing
        const float w_own = exp2f(l_own - mx);
        wsum = w_own;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= w_own;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float w = s < npast ? exp2f(lv[s] - mx) : 0.f;
            wsum += w;
            float f[8];
            widen(pc[s], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(w, f[e], o[e]);
        }
    } else {
        for (int s = 0; s < npast; ++s) mx = fmaxf(mx, ls[s]);
        load8(po + (size_t)(nslot - 1) * D, o);
        const float w_own = exp2f(l_own - mx);
        wsum = w_own;
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
    }
    const float iw = 1.f / wsum;
    if (lse_out && ch == 0) lse_out[((size_t)b * Hq + h) * S + t] = (mx + log2f(wsum)) * kLn2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= iw;
    store8(out + (((size_t)b * S + t) * Hq + h) * D + ch * 8, o);
}

template <typename T, int D, int NS>
hipError_t merge_ns(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    constexpr int RPW = 256 / (D / 8);
    const long long rows = (long long)p.batch * p.Hq * p.R;
    merge_kernel<T, D, NS><<<(unsigned)((rows + RPW - 1) / RPW), 256, 0, st>>>(
        static_cast<const T *>(bf.part_o), bf.part_lse, static_cast<T *>(bf.out), bf.lse_out, p.S,
        p.Hq, p.B,
        p.topk, part_slots(p), rows, p.r0, p.R);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t merge_impl(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    if (p.npast <= 4) return merge_ns<T, D, 4>(bf, p, st);
    if (p.npast <= 8) return merge_ns<T, D, 8>(bf, p, st);
    if (p.npast <= 12) return merge_ns<T, D, 12>(bf, p, st);
    return merge_ns<T, D, 0>(bf, p, st);
}

}  // namespace

hipError_t launch_merge(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    if (p.dtype == kBF16)
        return p.D == 64 ? merge_impl<__bf16, 64>(bf, p, st) : merge_impl<__bf16, 128>(bf, p, st);
    return p.D == 64 ? merge_impl<float, 64>(bf, p, st) : merge_impl<float, 128>(bf, p, st);
}

}  // namespace moba
