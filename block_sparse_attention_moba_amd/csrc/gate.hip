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
// chunk of 32 block means staged in LDS serves all of them.  The means come
// split into bf16 hi + lo parts by the pool pass (hi = rne(x), lo = rne(x -
// hi)), so two MFMAs per 16 dims give q.kbar with a relative error near 2^-17.  The 32x32
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
                                                   int Hkv, int G, int B, int n, int topk, int r0,
                                                   int R) {
    __shared__ float kb[kGateJC][D];
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / G;
    const int t = r0 + blockIdx.x * 256 + threadIdx.x;
    const bool valid = t < r0 + R;
    const int own = valid ? t / B : 0;
    const int npast = min(topk - 1, own);
    const int t_last = min(r0 + (int)blockIdx.x * 256 + 255, r0 + R - 1);
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
    int32_t *dst = idx + (((size_t)b * Hq + h) * R + (t - r0)) * topk;
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

// Spread the 4 nibbles of a 16-bit value to the even nibbles of a 32-bit word.
__device__ inline uint32_t spread_nibbles(uint32_t x) {
    x &= 0xffffu;
    x = (x | (x << 8)) & 0x00ff00ffu;
    return (x | (x << 4)) & 0x0f0f0f0fu;
}

// Sorted descending value list: insert x (the smallest value falls off).
// Slot p becomes the median of (old slot p-1, x, old slot p).
template <int KP>
__device__ __forceinline__ void value_insert(float (&val)[KP], float x) {
#pragma unroll
    for (int p = KP - 1; p > 0; --p) val[p] = __builtin_amdgcn_fmed3f(val[p - 1], x, val[p]);
    val[0] = fmaxf(val[0], x);
}

// grid (ceil(S / (32 TW)), Hkv, batch), 64 G TW threads: wave w holds head
// g G + w % G, tokens t0 .. t0 + 31 with t0 = 32 (blockIdx.x TW + w / G).
//
// Two passes over the blocks, no index lists.  Pass 1 keeps only values (a
// branch-free median-of-three network) and yields T, the row's npast-th best
// score, and how many scores lie strictly above it.  Pass 2 recomputes the
// same scores (bitwise identical: same instructions on the same data) and,
// chunk by chunk in ascending block order, selects the blocks with s > T and
// the first of those with s == T that complete the list (ties go to the
// smallest indices), so the output comes out ascending as it is written.
// (Keeping pass 1's scores in registers instead halves the occupancy and
// measured slower.)
template <int D, int KP>
__global__ __launch_bounds__(64 * kGateMaxWaves) void gate_mfma_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ khl, int32_t *__restrict__ idx, int S,
    int Hq, int Hkv, int G, int B, int n, int topk, int TW, int r0, int R) {
    constexpr int CPR = D / 8;                      // 16-byte chunks per row
    __shared__ __attribute__((aligned(16))) __bf16 khi[2][32 * D];
    __shared__ __attribute__((aligned(16))) __bf16 klo[2][32 * D];
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int g = blockIdx.y, b = blockIdx.z;
    const int h = g * G + wave % G;
    const int t0 = r0 + (blockIdx.x * TW + wave / G) * 32;
    const int t = t0 + col;
    const bool valid = t < r0 + R;
    // all 32 rows of the wave share one block (B is a multiple of 64)
    const int own = min(t0, r0 + R - 1) / B;
    const int npast = min(topk - 1, own);
    const int t_last = min(r0 + (int)(blockIdx.x * TW + TW) * 32 - 1, r0 + R - 1);
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
    const __bf16 *kb = khl + ((size_t)b * Hkv + g) * n * 2 * D;
    const f32x16_t zero16 = {};
    // stage the hi / lo parts of block means c*32 .. c*32+31, chunk-swizzled rows
    auto stage = [&](int c) {
        const int buf = c & 1;
        for (int it = tid; it < 32 * CPR; it += nthreads) {
            const int r = it / CPR, ch = it % CPR;
            const int j = c * 32 + r;
            bf16x8_t hi, lo;
            if (j < n) {
                hi = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)j * 2 * D + ch * 8);
                lo = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)j * 2 * D + D + ch * 8);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) hi[e] = lo[e] = (__bf16)0.f;
            }
            const int off = r * D + ((ch ^ (r & (CPR - 1))) << 3);
            *reinterpret_cast<bf16x8_t *>(&khi[buf][off]) = hi;
            *reinterpret_cast<bf16x8_t *>(&klo[buf][off]) = lo;
        }
    };
    // S^T of 32 blocks x 32 rows: rows = blocks, columns = queries; lane
    // (col, half) gets blocks c*32 + 8 (i / 4) + 4 half + i % 4 of row col
    auto scores = [&](int c) {
        const int buf = c & 1;
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
        return sa;
    };
    int32_t *dst = idx + (((size_t)b * Hq + h) * R + (t - r0)) * topk;

    // pass 1: the npast best values of the lane's blocks, then of the row
    float val[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) val[p] = (p < KP - npast) ? INFINITY : -INFINITY;
    for (int c = 0; c * 32 < jend; ++c) {
        stage(c);
        __syncthreads();
        if (c * 32 < own) {
            const f32x16_t sa = scores(c);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                value_insert<KP>(val, j < own ? sa[i] : -INFINITY);
            }
        }
    }
    float pv[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) pv[p] = __shfl_xor(val[p], 32, 64);
#pragma unroll
    for (int p = 0; p < KP; ++p)
        if (p >= KP - npast) value_insert<KP>(val, pv[p]);
    const float T = val[KP - 1];
    int ngt = 0;                   // scores strictly above T: all of them are in the list
#pragma unroll
    for (int p = 0; p < KP; ++p) ngt += (p >= KP - npast && val[p] > T) ? 1 : 0;
    int need = npast - ngt;        // ties at T, smallest indices first
    int r = 0;
    __syncthreads();               // every wave is done with the staging buffers of pass 1

    // pass 2: per chunk, this lane's blocks above T and equal to T as 16-bit
    // masks; the half-0 lane interleaves them with its partner's (it holds
    // blocks 8m .. 8m+3 of the chunk, the partner 8m+4 .. 8m+7) and writes
    for (int c = 0; c * 32 < jend; ++c) {
        stage(c);
        __syncthreads();
        uint32_t gt = 0u, ti = 0u;
        if (c * 32 < own) {
            const f32x16_t sa = scores(c);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                if (j < own && sa[i] > T) gt |= 1u << i;
                if (j < own && sa[i] == T) ti |= 1u << i;
            }
        }
        const uint32_t pg = __shfl_xor(gt, 32, 64), pt = __shfl_xor(ti, 32, 64);
        if (valid && !half) {
            const uint32_t fg = spread_nibbles(gt) | (spread_nibbles(pg) << 4);
            uint32_t w = spread_nibbles(ti) | (spread_nibbles(pt) << 4), keep = 0u;
            while (need > 0 && w) {
                const uint32_t low = w & (0u - w);
                keep |= low;
                w ^= low;
                --need;
            }
            uint32_t f = fg | keep;
            while (f) {
                if (r < npast) dst[r] = c * 32 + __builtin_ctz(f);   // npast exactly, unless a score is NaN
                ++r;
                f &= f - 1;
            }
        }
    }
    if (!valid || half) return;
    dst[npast] = own;
    for (int cc = npast + 1; cc < topk; ++cc) dst[cc] = -1;
}

// Token chunks of 32 per workgroup: G TW waves, at most kGateMaxWaves.
inline int gate_tw(int G) { return G >= kGateMaxWaves ? 1 : (kGateMaxWaves / G >= 2 ? 2 : 1); }

template <int D, int KP>
static hipError_t gate_mfma_impl(const void *q, const __bf16 *khl, int32_t *idx, const Problem &p,
                                 hipStream_t st) {
    const int TW = gate_tw(p.G);
    dim3 grid((p.R + 32 * TW - 1) / (32 * TW), p.Hkv, p.batch);
    gate_mfma_kernel<D, KP><<<grid, 64 * p.G * TW, 0, st>>>(
        static_cast<const __bf16 *>(q), khl, idx, p.S, p.Hq, p.Hkv, p.G, p.B, p.n, p.topk, TW,
        p.r0, p.R);
    return hipGetLastError();
}

template <int D>
static hipError_t gate_mfma_kp(const void *q, const __bf16 *khl, int32_t *idx, const Problem &p,
                               hipStream_t st) {
    const int np = p.npast;
    if (np <= 1) return gate_mfma_impl<D, 1>(q, khl, idx, p, st);
    if (np <= 2) return gate_mfma_impl<D, 2>(q, khl, idx, p, st);
    if (np <= 4) return gate_mfma_impl<D, 4>(q, khl, idx, p, st);
    if (np <= 8) return gate_mfma_impl<D, 8>(q, khl, idx, p, st);
    if (np <= 12) return gate_mfma_impl<D, 12>(q, khl, idx, p, st);
    if (np <= 16) return gate_mfma_impl<D, 16>(q, khl, idx, p, st);
    if (np <= 24) return gate_mfma_impl<D, 24>(q, khl, idx, p, st);
    return gate_mfma_impl<D, 32>(q, khl, idx, p, st);
}

// Every causal block is selected (topk >= number of blocks): no scoring needed.
// grid (ceil(R / 256), Hq, batch), 256 threads.
__global__ __launch_bounds__(256) void gate_all_kernel(int32_t *__restrict__ idx, int Hq, int B,
                                                       int topk, int r0, int R) {
    const int tl = blockIdx.x * 256 + threadIdx.x;
    if (tl >= R) return;
    const int own = (r0 + tl) / B;
    int32_t *dst = idx + (((size_t)blockIdx.z * Hq + blockIdx.y) * R + tl) * topk;
    for (int c = 0; c < topk; ++c) dst[c] = (c <= own) ? c : -1;
}

template <typename T, int D, int KP>
static hipError_t gate_impl(const void *q, const float *kbar, int32_t *idx, const Problem &p,
                            hipStream_t st) {
    dim3 grid((p.R + 255) / 256, p.Hq, p.batch);
    gate_kernel<T, D, KP><<<grid, 256, 0, st>>>(static_cast<const T *>(q), kbar, idx, p.S, p.Hq,
                                                p.Hkv, p.G, p.B, p.n, p.topk, p.r0, p.R);
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

hipError_t launch_gate(const void *q, const float *kbar, const __bf16 *khl, int32_t *idx,
                       const Problem &p, hipStream_t st) {
    if (p.dense) {
        dim3 grid((p.R + 255) / 256, p.Hq, p.batch);
        gate_all_kernel<<<grid, 256, 0, st>>>(idx, p.Hq, p.B, p.topk, p.r0, p.R);
        return hipGetLastError();
    }
    if (p.dtype == kBF16 && p.G <= kGateMaxWaves)
        return p.D == 64 ? gate_mfma_kp<64>(q, khl, idx, p, st) : gate_mfma_kp<128>(q, khl, idx, p, st);
    if (p.dtype == kBF16)
        return p.D == 64 ? gate_kp<__bf16, 64>(q, kbar, idx, p, st)
                         : gate_kp<__bf16, 128>(q, kbar, idx, p, st);
    return p.D == 64 ? gate_kp<float, 64>(q, kbar, idx, p, st)
                     : gate_kp<float, 128>(q, kbar, idx, p, st);
}

}  // namespace moba
