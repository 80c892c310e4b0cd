// Parameter-free gate and causal top-k (write-up "MoBA: Mixture of Block
// Attention", the first implementation step: assign each query token to KV
// blocks from the gate and the causal mask; Taiwan AI overview, section
// "技術細節與優勢": the own block is always kept, future blocks never).
//
// One thread owns one query row (b, h, t).  The fp32 block means of the
// row's KV head are staged through LDS in chunks of JC blocks and read as
// broadcasts; the score is an fp32 inner product of the decoded query with
// the block mean.  The row keeps its best KP candidates in registers, sorted
// by score: the first KP - npast slots hold +inf sentinels that are never
// displaced, so the live list is exactly npast long and its last entry is the
// admission threshold.  Blocks are scanned in ascending order and a candidate
// must beat an entry strictly, so equal scores keep the smaller block index.
#include <limits.h>
#include <math.h>

#include "moba_internal.hpp"

namespace moba {

constexpr int kGateJC = 32;   // block means per LDS chunk

__device__ inline float to_f32(__bf16 x) { return (float)x; }
__device__ inline float to_f32(float x) { return x; }

// grid (ceil(S / 256), Hq, batch), 256 threads.
template <typename T, int D, int KP>
__global__ __launch_bounds__(256) void gate_kernel(const T *__restrict__ q,
                                                   const float *__restrict__ kbar,
                                                   int32_t *__restrict__ idx, int S, int Hq,
                                                   int Hkv, int G, int B, int n, int topk) {
    __shared__ float kb[kGateJC][D];
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / G;
    const int t = blockIdx.x * 256 + threadIdx.x;
    const bool valid = t < S;
    const int own = valid ? t / B : 0;
    const int npast = min(topk - 1, own);
    const int t_last = min((int)blockIdx.x * 256 + 255, S - 1);
    // rows of this workgroup need past blocks j < t_last / B at most
    const int jend = (topk > 1) ? t_last / B : 0;

    float qv[D];
    if (valid) {
        const T *src = q + (((size_t)b * S + t) * Hq + h) * D;
#pragma unroll
        for (int i = 0; i < D; ++i) qv[i] = to_f32(src[i]);
    } else {
#pragma unroll
        for (int i = 0; i < D; ++i) qv[i] = 0.f;
    }
    float val[KP];
    int ix[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
        val[p] = (p < KP - npast) ? INFINITY : -INFINITY;
        ix[p] = INT_MAX;
    }

    const float *kbase = kbar + ((size_t)b * Hkv + g) * n * D;
    for (int jc = 0; jc < jend; jc += kGateJC) {
        const int cnt = min(kGateJC, jend - jc);
        __syncthreads();
        for (int e = threadIdx.x; e < cnt * D; e += 256) kb[e / D][e % D] = kbase[(size_t)jc * D + e];
        __syncthreads();
        for (int jj = 0; jj < cnt; ++jj) {
            const int j = jc + jj;
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int i = 0; i < D; i += 4) {
                const float4 kv = *reinterpret_cast<const float4 *>(&kb[jj][i]);
                a0 = fmaf(qv[i], kv.x, a0);
                a1 = fmaf(qv[i + 1], kv.y, a1);
                a2 = fmaf(qv[i + 2], kv.z, a2);
                a3 = fmaf(qv[i + 3], kv.w, a3);
            }
            const float s = (a0 + a1) + (a2 + a3);
            if (j < own && s > val[KP - 1]) {
                float cs = s;
                int cj = j;
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    const bool c = cs > val[p];
                    const float tv = val[p];
                    const int ti = ix[p];
                    val[p] = c ? cs : tv;
                    ix[p] = c ? cj : ti;
                    cs = c ? tv : cs;
                    cj = c ? ti : cj;
                }
            }
        }
    }
    if (!valid) return;
    int32_t *dst = idx + (((size_t)b * Hq + h) * S + t) * topk;
    // write the live entries in ascending block order (rank by block index)
#pragma unroll
    for (int p = 0; p < KP; ++p) {
        if (p >= KP - npast) {
            int r = 0;
#pragma unroll
            for (int o = 0; o < KP; ++o) r += (o >= KP - npast && ix[o] < ix[p]) ? 1 : 0;
            dst[r] = ix[p];
        }
    }
    dst[npast] = own;
    for (int c = npast + 1; c < topk; ++c) dst[c] = -1;
}

// Every causal block is selected (topk >= number of blocks): no scoring needed.
// grid (ceil(S / 256), Hq, batch), 256 threads.
__global__ __launch_bounds__(256) void gate_all_kernel(int32_t *__restrict__ idx, int S, int Hq,
                                                       int B, int topk) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= S) return;
    const int own = t / B;
    int32_t *dst = idx + (((size_t)blockIdx.z * Hq + blockIdx.y) * S + t) * topk;
    for (int c = 0; c < topk; ++c) dst[c] = (c <= own) ? c : -1;
}

template <typename T, int D, int KP>
static hipError_t gate_impl(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                            hipStream_t st) {
    dim3 grid((p.S + 255) / 256, p.Hq, p.batch);
    gate_kernel<T, D, KP><<<grid, 256, 0, st>>>(static_cast<const T *>(q), kbar, idx, p.S, p.Hq,
                                                p.Hkv, p.G, p.B, p.n, p.topk);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t gate_kp(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                          hipStream_t st) {
    const int np = p.npast;
    if (np <= 1) return gate_impl<T, D, 1>(q, kbar, idx, p, st);
    if (np <= 2) return gate_impl<T, D, 2>(q, kbar, idx, p, st);
    if (np <= 4) return gate_impl<T, D, 4>(q, kbar, idx, p, st);
    if (np <= 8) return gate_impl<T, D, 8>(q, kbar, idx, p, st);
    if (np <= 16) return gate_impl<T, D, 16>(q, kbar, idx, p, st);
    return gate_impl<T, D, 32>(q, kbar, idx, p, st);
}

hipError_t launch_gate(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                       hipStream_t st) {
    if (p.dense) {
        dim3 grid((p.S + 255) / 256, p.Hq, p.batch);
        gate_all_kernel<<<grid, 256, 0, st>>>(idx, p.S, p.Hq, p.B, p.topk);
        return hipGetLastError();
    }
    if (p.dtype == kBF16)
        return p.D == 64 ? gate_kp<__bf16, 64>(q, kbar, idx, p, st)
                         : gate_kp<__bf16, 128>(q, kbar, idx, p, st);
    return p.D == 64 ? gate_kp<float, 64>(q, kbar, idx, p, st)
                     : gate_kp<float, 128>(q, kbar, idx, p, st);
}

}  // namespace moba
