// Parameter-free gate and causal top-k (write-up "MoBA: Mixture of Block
// Attention", the first implementation step: assign each query token to KV
// blocks from the gate and the causal mask; Taiwan AI overview, section
// "技術細節與優勢": the own block is always kept, future blocks never).
//
// Selection rule shared by both kernels: a row keeps its best npast =
// min(topk - 1, own) past blocks by score, equal scores resolved toward the
// smaller block index, and writes them in ascending block order followed by
// its own block (then -1 up to topk).  Each row keeps its best KP candidates
// in registers, sorted by score: the first KP - npast slots hold +inf
// sentinels that are never displaced, so the live list is exactly npast long
// and its last entry is the admission threshold.
//
// bf16 inputs (gate_mfma_kernel): the scores come from the matrix cores.
// A workgroup owns one (batch, KV head) and 32 TW consecutive tokens of all
// G query heads of that KV head (one wave per 32 rows of one head), so every
// chunk of 32 block means staged in LDS serves all of them.  The fp32 means
// are split into bf16 hi + lo parts (hi = rne(x), lo = rne(x - hi)), so two
// MFMAs per 16 dims give q.kbar with a relative error near 2^-17.  The 32x32
// result leaves each row's scores in two lanes (16 blocks each per chunk);
// each lane keeps its own best list over ascending block indices, then the
// two lists merge with an explicit (score, smaller index) order.
//
// fp32 inputs (gate_kernel): one thread owns one query row and takes fp32
// inner products with the block means broadcast from LDS.
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

// ---- bf16: matrix-core scores ----

constexpr int kGateMaxWaves = 8;

// Insert (cs, cj) into the sorted list: strictly higher scores displace.
template <int KP>
__device__ __forceinline__ void list_insert(float (&val)[KP], int (&ix)[KP], float cs, int cj) {
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

// grid (ceil(S / (32 TW)), Hkv, batch), 64 G TW threads: wave w holds head
// g G + w % G, tokens t0 .. t0 + 31 with t0 = 32 (blockIdx.x TW + w / G).
template <int D, int KP>
__global__ __launch_bounds__(64 * kGateMaxWaves) void gate_mfma_kernel(
    const __bf16 *__restrict__ q, const float *__restrict__ kbar, int32_t *__restrict__ idx, int S,
    int Hq, int Hkv, int G, int B, int n, int topk, int TW) {
    constexpr int CPR = D / 8;                      // 16-byte chunks per row
    __shared__ __attribute__((aligned(16))) __bf16 khi[2][32 * D];
    __shared__ __attribute__((aligned(16))) __bf16 klo[2][32 * D];
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int g = blockIdx.y, b = blockIdx.z;
    const int h = g * G + wave % G;
    const int t0 = (blockIdx.x * TW + wave / G) * 32;
    const int t = t0 + col;
    const bool valid = t < S;
    // all 32 rows of the wave share one block (B is a multiple of 64)
    const int own = min(t0, S - 1) / B;
    const int npast = min(topk - 1, own);
    const int t_last = min((int)(blockIdx.x * TW + TW) * 32 - 1, S - 1);
    const int jend = (topk > 1) ? t_last / B : 0;   // past blocks any row here can use

    bf16x8_t qf[D / 16];
    {
        const __bf16 *src = q + (((size_t)b * S + (valid ? t : 0)) * Hq + h) * D + half * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            qf[kk] = *reinterpret_cast<const bf16x8_t *>(src + kk * 16);
            if (!valid)
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.f;
        }
    }
    float val[KP];
    int ix[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
        val[p] = (p < KP - npast) ? INFINITY : -INFINITY;
        ix[p] = INT_MAX;
    }
    const float *kb = kbar + ((size_t)b * Hkv + g) * n * D;
    const f32x16_t zero16 = {};
    for (int c = 0; c * 32 < jend; ++c) {
        const int buf = c & 1;
        // stage block means c*32 .. c*32+31 as bf16 hi / lo, chunk-swizzled rows
        for (int it = tid; it < 32 * CPR; it += nthreads) {
            const int r = it / CPR, ch = it % CPR;
            const int j = c * 32 + r;
            bf16x8_t hi, lo;
            if (j < n) {
                const float4 x0 = *reinterpret_cast<const float4 *>(kb + (size_t)j * D + ch * 8);
                const float4 x1 = *reinterpret_cast<const float4 *>(kb + (size_t)j * D + ch * 8 + 4);
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi[e] = (__bf16)x[e];
                    lo[e] = (__bf16)(x[e] - (float)hi[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) hi[e] = lo[e] = (__bf16)0.f;
            }
            const int off = r * D + ((ch ^ (r & (CPR - 1))) << 3);
            *reinterpret_cast<bf16x8_t *>(&khi[buf][off]) = hi;
            *reinterpret_cast<bf16x8_t *>(&klo[buf][off]) = lo;
        }
        __syncthreads();
        if (c * 32 < own) {
            // S^T of 32 blocks x 32 rows: rows = blocks, columns = queries
            f32x16_t sa = zero16;
            const int sw = col & (CPR - 1);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int off = col * D + (((kk * 2 + half) ^ sw) << 3);
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&khi[buf][off]);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(&klo[buf][off]);
                sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[kk], sa, 0, 0, 0);
                sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[kk], sa, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                if (j < own && sa[i] > val[KP - 1]) list_insert<KP>(val, ix, sa[i], j);
            }
        }
    }
    // merge the partner lane's live entries: higher score first, then smaller
    // index.  Both lanes merge at once, so the partner's list is copied whole
    // before either list changes.
    float pv[KP];
    int pj[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
        pv[p] = __shfl_xor(val[p], 32, 64);
        pj[p] = __shfl_xor(ix[p], 32, 64);
    }
#pragma unroll
    for (int p = 0; p < KP; ++p) {
        float cs = pv[p];
        int cj = pj[p];
        if (p >= KP - npast) {
#pragma unroll
            for (int o = 0; o < KP; ++o) {
                const bool cc = cs > val[o] || (cs == val[o] && cj < ix[o]);
                const float tv = val[o];
                const int ti = ix[o];
                val[o] = cc ? cs : tv;
                ix[o] = cc ? cj : ti;
                cs = cc ? tv : cs;
                cj = cc ? ti : cj;
            }
        }
    }
    if (!valid || half) return;
    int32_t *dst = idx + (((size_t)b * Hq + h) * S + t) * topk;
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
    for (int cc = npast + 1; cc < topk; ++cc) dst[cc] = -1;
}

// Token chunks of 32 per workgroup: G TW waves, at most kGateMaxWaves.
inline int gate_tw(int G) { return G >= kGateMaxWaves ? 1 : (kGateMaxWaves / G >= 2 ? 2 : 1); }

template <int D, int KP>
static hipError_t gate_mfma_impl(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                                 hipStream_t st) {
    const int TW = gate_tw(p.G);
    dim3 grid((p.S + 32 * TW - 1) / (32 * TW), p.Hkv, p.batch);
    gate_mfma_kernel<D, KP><<<grid, 64 * p.G * TW, 0, st>>>(
        static_cast<const __bf16 *>(q), kbar, idx, p.S, p.Hq, p.Hkv, p.G, p.B, p.n, p.topk, TW);
    return hipGetLastError();
}

template <int D>
static hipError_t gate_mfma_kp(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                               hipStream_t st) {
    const int np = p.npast;
    if (np <= 1) return gate_mfma_impl<D, 1>(q, kbar, idx, p, st);
    if (np <= 2) return gate_mfma_impl<D, 2>(q, kbar, idx, p, st);
    if (np <= 4) return gate_mfma_impl<D, 4>(q, kbar, idx, p, st);
    if (np <= 8) return gate_mfma_impl<D, 8>(q, kbar, idx, p, st);
    if (np <= 12) return gate_mfma_impl<D, 12>(q, kbar, idx, p, st);
    if (np <= 16) return gate_mfma_impl<D, 16>(q, kbar, idx, p, st);
    if (np <= 24) return gate_mfma_impl<D, 24>(q, kbar, idx, p, st);
    return gate_mfma_impl<D, 32>(q, kbar, idx, p, st);
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
    if (p.dtype == kBF16 && p.G <= kGateMaxWaves)
        return p.D == 64 ? gate_mfma_kp<64>(q, kbar, idx, p, st) : gate_mfma_kp<128>(q, kbar, idx, p, st);
    if (p.dtype == kBF16)
        return p.D == 64 ? gate_kp<__bf16, 64>(q, kbar, idx, p, st)
                         : gate_kp<__bf16, 128>(q, kbar, idx, p, st);
    return p.D == 64 ? gate_kp<float, 64>(q, kbar, idx, p, st)
                     : gate_kp<float, 128>(q, kbar, idx, p, st);
}

}  // namespace moba
