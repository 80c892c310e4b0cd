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

#include <algorithm>

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

// ---- bf16, d = 128, n <= 257 blocks: one pass, persistent ----
//
// The kernel above computes every score twice (pass 1 finds the threshold,
// pass 2 recomputes the scores to select against it), and its top-k network
// is as long as the largest list it supports.  Here every score is computed
// once and stays in registers (16 per lane and chunk of 32 blocks, at most 8
// chunks), the value list is exactly npast = topk - 1 long, and rows whose
// own block is at most topk - 1 (all their past blocks are selected) read no
// query at all.  Per row:
//   1. each of the row's two lanes keeps the npast best of its own scores (a
//      median-of-three insertion network, npast operations per score);
//   2. the two lists meet through a lane swap: the npast best of the union
//      are max(A[i], B[npast-1-i]) (A, B sorted descending), so the row's
//      npast-th best score is T = min_i max(A[i], B[npast-1-i]);
//   3. the stored scores give the row's blocks with s >= T as bit masks; if
//      there are exactly npast of them (no tie at T) they are the selection,
//      otherwise the blocks with s > T plus the smallest-index blocks with
//      s == T (ties toward the smaller block, as in the rule above).
// The workgroup is persistent: it walks tiles (one (batch, KV head) pair, 32
// TW tokens, all G heads) in a static order, heaviest (latest) tiles of each
// pair first, keeps the pair's block means in LDS while it stays on that
// pair.  Selected indices are staged per wave in LDS and stored as
// contiguous rows.
constexpr int kSpMaxKP = 16;       // npast handled here (topk <= 17)

struct GateSpArgs {
    const __bf16 *q;
    const __bf16 *khl;     // [batch][Hkv][n][2][D]
    int32_t *idx;
    int S, Hq, Hkv, G, B, n, topk, r0, R;
    int TW;                // token groups of 32 rows per workgroup (G waves each)
    int npairs;            // batch * Hkv
};

// Waves per SIMD: 4 (two 8-wave workgroups per CU, 128 registers) for one
// chunk, else 2 (256 registers: the scores of up to 8 chunks and the next
// chunk's accumulators).  The other waves of the SIMD cover a tile's query
// loads; a next-tile prefetch would cost 32 registers and spill.
template <int KP, int NCH>
constexpr int gate_sp_waves() { return NCH == 1 ? 4 : 2; }

template <int KP, int NCH>
__global__ __launch_bounds__(64 * kGateMaxWaves, (gate_sp_waves<KP, NCH>())) void gate_sp_kernel(
    GateSpArgs a) {
    constexpr int D = 128, CPR = D / 8, KD = D / 16;
    constexpr int TOPK = KP + 1;
    __shared__ __attribute__((aligned(16))) __bf16 khi[NCH * 32 * D];
    __shared__ __attribute__((aligned(16))) __bf16 klo[NCH * 32 * D];
    __shared__ int32_t orow[kGateMaxWaves][32 * TOPK];
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int hh = wave % a.G, tg = wave / a.G;
    int32_t *stage_row = orow[wave];
    const int nstage = min(a.n, NCH * 32);        // blocks held in LDS

    // per-lane LDS offsets of the A operand (block col of a chunk, 16-byte chunk 2 kk + half)
    int aoff[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) aoff[kk] = col * D + (((kk * 2 + half) ^ (col & (CPR - 1))) << 3);

    // Items: (pair, 32-token group), pair-major, the latest (heaviest) token
    // groups of a pair first.  Workgroup w owns items w, w + grid, w + 2 grid,
    // ...; its TW token groups (G waves each, one per head) take them in turn
    // and run independently, so the two waves of a SIMD (different groups)
    // drift apart and overlap each other's loads, matrix-core and vector work.
    // They meet only where the pair changes and the block means are restaged.
    const int n32 = a.R / 32;                          // R is a multiple of 64
    const long long nitems = (long long)a.npairs * n32;
    const long long w = blockIdx.x, grid = gridDim.x;
    auto stage = [&](int pair) {
        __syncthreads();                               // every wave is done with the last pair
        const __bf16 *kb = a.khl + (size_t)pair * a.n * 2 * D;
        for (int it = tid; it < NCH * 32 * CPR; it += nthreads) {
            const int j = it / CPR, ch = it % CPR;
            bf16x8_t hi, lo;
            if (j < nstage) {
                hi = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)j * 2 * D + ch * 8);
                lo = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)j * 2 * D + D + ch * 8);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) hi[e] = lo[e] = (__bf16)0.f;
            }
            const int off = j * D + ((ch ^ (j & (CPR - 1))) << 3);
            *reinterpret_cast<bf16x8_t *>(&khi[off]) = hi;
            *reinterpret_cast<bf16x8_t *>(&klo[off]) = lo;
        }
        __syncthreads();
    };
    // S^T of chunk c (32 blocks x this wave's 32 rows): lane (col, half) gets
    // blocks 32 c + 8 (i / 4) + 4 half + i % 4 of row col
    auto chunk_scores = [&](int c, const bf16x8_t (&qf)[KD]) {
        f32x16_t acc = {};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&khi[c * 32 * D + aoff[kk]]);
            const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(&klo[c * 32 * D + aoff[kk]]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[kk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[kk], acc, 0, 0, 0);
        }
        return acc;
    };

    for (long long k0 = 0;;) {
        const long long first = w + k0 * grid;
        if (first >= nitems) break;
        const int pair = (int)(first / n32);
        // this workgroup's items of the pair: k0 <= k < k1
        const long long k1 = ((long long)(pair + 1) * n32 - w + grid - 1) / grid;
        stage(pair);
        const int b = pair / a.Hkv, g = pair % a.Hkv, h = g * a.G + hh;
        // first token of item k of this pair (k0 <= k < k1: item w + k grid lies in the pair)
        auto item_t0 = [&](long long k) {
            return a.r0 + (n32 - 1 - (int)(w + k * grid - (long long)pair * n32)) * 32;
        };
        // Q of the item's 32 rows; the next item's is loaded as soon as this
        // item's last product has been issued, so that its latency overlaps the
        // rest of this item (the last insertions, the merge, the emission)
        bf16x8_t qf[KD];
        auto load_q = [&](long long k) {
            const __bf16 *src = a.q + (((size_t)b * a.S + item_t0(k) + col) * a.Hq + h) * D + half * 8;
    #pragma unroll
            for (int kk = 0; kk < KD; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t *>(src + kk * 16);
        };
        auto needs_q = [&](long long k) { return k < k1 && item_t0(k) / a.B > a.topk - 1; };
        if (needs_q(k0 + tg)) load_q(k0 + tg);
        for (long long k = k0 + tg; k < k1; k += a.TW) {
            const int t0 = item_t0(k);
            const int own = t0 / a.B;                      // all 32 rows share a block
            const bool pref = needs_q(k + a.TW);
            if (own <= a.topk - 1) {
                if (pref) load_q(k + a.TW);
                // every past block is selected: blocks 0 .. own - 1, the own block, then -1
                for (int e = lane; e < 32 * a.topk; e += 64) {
                    const int c = e % a.topk;
                    stage_row[e] = c < own ? c : (c == own ? own : -1);
                }
            } else {
                const int nchw = (own + 31) / 32;          // chunks of past blocks (wave-uniform)
                f32x16_t sc[NCH];
                float lst[KP];
    #pragma unroll
                for (int p = 0; p < KP; ++p) lst[p] = -INFINITY;
                // the matrix cores compute chunk c + 1 while the vector unit inserts chunk c
                sc[0] = chunk_scores(0, qf);
                if (nchw == 1 && pref) load_q(k + a.TW);
    #pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (c + 1 < NCH && c + 1 < nchw) {
                        sc[c + 1] = chunk_scores(c + 1, qf);
                        if (c + 2 == nchw && pref) load_q(k + a.TW);
    #pragma unroll
                        for (int i = 0; i < 16; ++i) value_insert<KP>(lst, sc[c][i]);
                    } else if (c + 1 == nchw) {
                        if (c * 32 + 32 > own) {           // the last chunk holds the own block
    #pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int j = c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                                if (j >= own) sc[c][i] = -INFINITY;
                            }
                        }
    #pragma unroll
                        for (int i = 0; i < 16; ++i) value_insert<KP>(lst, sc[c][i]);
                    }
                }
                // T: the row's KP-th best score, from this lane's list and its partner's
                float T = INFINITY;
    #pragma unroll
                for (int p = 0; p < KP; ++p) {
                    const float other = __shfl_xor(lst[KP - 1 - p], 32, 64);
                    T = fminf(T, fmaxf(lst[p], other));
                }
                // the row's blocks with s >= T, one 32-bit mask per chunk (bit j - 32 c)
                uint32_t m[NCH];
                int cnt = 0;
    #pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    m[c] = 0u;
                    if (c < nchw) {
                        uint32_t b16 = 0u;
    #pragma unroll
                        for (int i = 0; i < 16; ++i) b16 |= (sc[c][i] >= T ? 1u : 0u) << i;
                        cnt += __builtin_popcount(b16);
                        const uint32_t mine = spread_nibbles(b16) << (4 * half);
                        m[c] = mine | __shfl_xor(mine, 32, 64);
                    }
                }
                cnt += __shfl_xor(cnt, 32, 64);
                if (__any(cnt != KP)) {
                    // ties at T: the blocks above T, then the smallest blocks equal to T
                    int need = KP;
                    uint32_t eq[NCH];
    #pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        eq[c] = 0u;
                        if (c < nchw) {
                            uint32_t g16 = 0u, e16 = 0u;
    #pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                g16 |= (sc[c][i] > T ? 1u : 0u) << i;
                                e16 |= (sc[c][i] == T ? 1u : 0u) << i;
                            }
                            const uint32_t gm = spread_nibbles(g16) << (4 * half);
                            const uint32_t em = spread_nibbles(e16) << (4 * half);
                            m[c] = gm | __shfl_xor(gm, 32, 64);
                            eq[c] = em | __shfl_xor(em, 32, 64);
                            need -= __builtin_popcount(m[c]);
                        }
                    }
    #pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        if (c < nchw) {
                            uint32_t ew = eq[c];
                            while (need > 0 && ew) {
                                const uint32_t low = ew & (0u - ew);
                                m[c] |= low;
                                ew ^= low;
                                --need;
                            }
                        }
                    }
                }
                // ascending block indices of the row (half 0 lanes), then the own block
                if (half == 0) {
                    int rr = 0;
    #pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        if (c < nchw) {
                            uint32_t f = m[c];
                            while (f) {
                                if (rr < KP) stage_row[col * TOPK + rr] = c * 32 + __builtin_ctz(f);
                                ++rr;
                                f &= f - 1;
                            }
                        }
                    }
                    for (; rr < KP; ++rr) stage_row[col * TOPK + rr] = -1;   // only with NaN scores
                    stage_row[col * TOPK + KP] = own;
                }
            }
            // the wave's 32 rows are contiguous in idx: [b][h][t - r0][topk]
            int32_t *dst = a.idx + (((size_t)b * a.Hq + h) * a.R + (t0 - a.r0)) * a.topk;
            for (int e = lane; e < 32 * a.topk; e += 64) dst[e] = stage_row[e];
        }
        k0 = k1;
    }
}

static int device_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

template <int KP, int NCH>
static hipError_t gate_sp_launch(const void *q, const __bf16 *khl, int32_t *idx, const Problem &p,
                                 hipStream_t st) {
    GateSpArgs a;
    a.q = static_cast<const __bf16 *>(q);
    a.khl = khl;
    a.idx = idx;
    a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.B = p.B; a.n = p.n; a.topk = p.topk;
    a.TW = p.G >= kGateMaxWaves ? 1 : kGateMaxWaves / p.G;
    a.r0 = p.r0; a.R = p.R;
    a.npairs = p.batch * p.Hkv;
    const long long items = (long long)a.npairs * (p.R / 32);
    // workgroups per CU: waves per SIMD x 4 SIMDs / waves per workgroup
    const int wgpc = std::max(1, gate_sp_waves<KP, NCH>() * 4 / (p.G * a.TW));
    const int grid = (int)std::min<long long>((items + a.TW - 1) / a.TW, (long long)device_cus() * wgpc);
    if (grid <= 0) return hipSuccess;
    gate_sp_kernel<KP, NCH><<<grid, 64 * p.G * a.TW, 0, st>>>(a);
    return hipGetLastError();
}

template <int KP>
static hipError_t gate_sp_nch(const void *q, const __bf16 *khl, int32_t *idx, const Problem &p,
                              hipStream_t st) {
    const int own_max = (p.r0 + p.R - 1) / p.B;
    const int nch = (own_max + 31) / 32;
    if (nch <= 1) return gate_sp_launch<KP, 1>(q, khl, idx, p, st);
    if (nch <= 2) return gate_sp_launch<KP, 2>(q, khl, idx, p, st);
    if (nch <= 4) return gate_sp_launch<KP, 4>(q, khl, idx, p, st);
    return gate_sp_launch<KP, 8>(q, khl, idx, p, st);
}

static hipError_t gate_sp(const void *q, const __bf16 *khl, int32_t *idx, const Problem &p,
                          hipStream_t st) {
    switch (p.npast) {
    case 1: return gate_sp_nch<1>(q, khl, idx, p, st);
    case 2: return gate_sp_nch<2>(q, khl, idx, p, st);
    case 3: return gate_sp_nch<3>(q, khl, idx, p, st);
    case 4: return gate_sp_nch<4>(q, khl, idx, p, st);
    case 5: return gate_sp_nch<5>(q, khl, idx, p, st);
    case 6: return gate_sp_nch<6>(q, khl, idx, p, st);
    case 7: return gate_sp_nch<7>(q, khl, idx, p, st);
    case 8: return gate_sp_nch<8>(q, khl, idx, p, st);
    case 9: return gate_sp_nch<9>(q, khl, idx, p, st);
    case 10: return gate_sp_nch<10>(q, khl, idx, p, st);
    case 11: return gate_sp_nch<11>(q, khl, idx, p, st);
    case 12: return gate_sp_nch<12>(q, khl, idx, p, st);
    case 13: return gate_sp_nch<13>(q, khl, idx, p, st);
    case 14: return gate_sp_nch<14>(q, khl, idx, p, st);
    case 15: return gate_sp_nch<15>(q, khl, idx, p, st);
    case 16: return gate_sp_nch<16>(q, khl, idx, p, st);
    default: return hipErrorInvalidValue;       // excluded by launch_gate's dispatch
    }
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

// The gate scores themselves (for tests of the gate's arithmetic): s_j =
// q_t . K-bar_j for every past block j < t / B, computed as the bf16 gate
// kernels compute them (per 16 dimensions the hi product, then the lo
// product, into one fp32 accumulator); NaN for j >= t / B.  One wave per 32
// tokens of one head; the block means are read straight from global memory.
// grid (S / 32, Hq, batch), 64 threads; scores [batch][Hq][S][n].
template <int D>
__global__ __launch_bounds__(64) void gate_scores_kernel(const __bf16 *__restrict__ q,
                                                         const __bf16 *__restrict__ khl,
                                                         float *__restrict__ scores, int S, int Hq,
                                                         int Hkv, int G, int B, int n) {
    constexpr int KD = D / 16;
    const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
    const int t0 = blockIdx.x * 32, h = blockIdx.y, b = blockIdx.z, g = h / G;
    const int t = t0 + col;                          // this lane's query row (S % 64 == 0)
    bf16x8_t qf[KD];
    const __bf16 *src = q + (((size_t)b * S + t) * Hq + h) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t *>(src + kk * 16);
    const __bf16 *kb = khl + ((size_t)b * Hkv + g) * n * 2 * D;
    const int own = t / B, nch = ((t0 + 31) / B + 31) / 32;
    // stored as bit patterns: this file is built with NaNs ruled out of its
    // floating-point arithmetic, so the quiet NaN is never a float value here
    constexpr uint32_t kNaN = 0x7fc00000u;
    uint32_t *row = reinterpret_cast<uint32_t *>(scores) + (((size_t)b * Hq + h) * S + t) * n;
    for (int c = 0; c < nch; ++c) {
        const int blk = c * 32 + col;                // this lane's A-operand block
        f32x16_t acc = {};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            bf16x8_t ah, al;
            if (blk < n) {
                ah = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)blk * 2 * D + kk * 16 + half * 8);
                al = *reinterpret_cast<const bf16x8_t *>(kb + (size_t)blk * 2 * D + D + kk * 16 + half * 8);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ah[e] = al[e] = (__bf16)0.f;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[kk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[kk], acc, 0, 0, 0);
        }
        // lane (col, half) holds blocks 32 c + 8 (i / 4) + 4 half + i % 4 of row col
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (j < n) row[j] = j < own ? __float_as_uint(acc[i]) : kNaN;
        }
    }
    // blocks past the tile's last own block
    for (int j = nch * 32 + half; j < n; j += 2) row[j] = kNaN;
}

hipError_t launch_gate_scores(const void *q, const __bf16 *khl, float *scores, const Problem &p,
                              hipStream_t st) {
    dim3 grid(p.S / 32, p.Hq, p.batch);
    if (p.D == 64)
        gate_scores_kernel<64><<<grid, 64, 0, st>>>(static_cast<const __bf16 *>(q), khl, scores, p.S,
                                                    p.Hq, p.Hkv, p.G, p.B, p.n);
    else
        gate_scores_kernel<128><<<grid, 64, 0, st>>>(static_cast<const __bf16 *>(q), khl, scores, p.S,
                                                     p.Hq, p.Hkv, p.G, p.B, p.n);
    return hipGetLastError();
}

hipError_t launch_gate(const void *q, const float *kbar, const __bf16 *khl, int32_t *idx,
                       const Problem &p, hipStream_t st) {
    if (p.dense) {
        dim3 grid((p.R + 255) / 256, p.Hq, p.batch);
        gate_all_kernel<<<grid, 256, 0, st>>>(idx, p.Hq, p.B, p.topk, p.r0, p.R);
        return hipGetLastError();
    }
    // one pass: bf16, d = 128, topk - 1 == npast <= 16 (not capped by the block count),
    // past blocks of the chunk's rows in at most 8 chunks of 32
    if (p.dtype == kBF16 && p.D == 128 && p.G <= kGateMaxWaves && p.npast == p.topk - 1 &&
        p.npast >= 1 && p.npast <= kSpMaxKP && (p.r0 + p.R - 1) / p.B <= 256)
        return gate_sp(q, khl, idx, p, st);
    if (p.dtype == kBF16 && p.G <= kGateMaxWaves)
        return p.D == 64 ? gate_mfma_kp<64>(q, khl, idx, p, st) : gate_mfma_kp<128>(q, khl, idx, p, st);
    if (p.dtype == kBF16)
        return p.D == 64 ? gate_kp<__bf16, 64>(q, kbar, idx, p, st)
                         : gate_kp<__bf16, 128>(q, kbar, idx, p, st);
    return p.D == 64 ? gate_kp<float, 64>(q, kbar, idx, p, st)
                     : gate_kp<float, 128>(q, kbar, idx, p, st);
}

}  // namespace moba
