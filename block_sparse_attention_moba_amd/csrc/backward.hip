// Backward pass of the MoBA attention: dq, dk, dv under the forward's block
// selection.  The write-up trains with MoBA (continual pre-training and
// fine-tuning, section "MoBA：將MoE原理應用于注意力機制" and its experiments),
// so the attention needs gradients; the selection gets none (a hard top-k is
// piecewise constant and the gate has no parameters of its own).
//
// With z = q.k / sqrt(d) the scaled logit, P = softmax over the row's
// selected keys, the forward output O and the upstream gradient dO:
//   dV_s = sum_t P_ts dO_t,   dP_ts = dO_t . v_s,   delta_t = dO_t . O_t,
//   dS_ts = P_ts (dP_ts - delta_t),
//   dQ_t = sum_s dS_ts k_s / sqrt(d),   dK_s = sum_t dS_ts q_t / sqrt(d).
// P is recomputed from the forward's per-row log-sum-exp: P = 2^(z log2 e - L2).
//
// Kernels (bf16 inputs, bf16 matrix-core products, fp32 accumulation):
//   bwd_prep_kernel   delta_t and L2_t per row (bandwidth-bound).
//   bwd_dq_kernel     the forward's gathered-row tiles (PAST: a list's rows
//                     against one past block; OWN: consecutive rows against
//                     their own block, causal); each tile accumulates dQ of its
//                     256 rows over the block's keys and writes one partial
//                     slot per (row, block), like the forward's partial outputs.
//   bwd_dq_sum_kernel the row's partial slots added up (fixed order) into dq.
//   bwd_kv_kernel     one workgroup per (batch, KV head, block, 256 keys): it
//                     walks every query row that attends these keys (the
//                     block's list, then the block's own rows, causal) and owns
//                     dV (first pass) or dK (second pass) of its keys, so no
//                     atomics and no reduction.
#include <type_traits>

#include "moba_internal.hpp"

namespace moba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
enum BwdTile { kPastTile = 0, kOwnTile = 1 };
constexpr int kBS = 32;   // keys per dq slice, rows per dk/dv chunk

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

struct BwdArgs {
    const __bf16 *q, *k, *v, *dout;
    const float *l2;       // [batch][Hq][S] base-2 log-sum-exp of z log2 e
    const float *delta;    // [batch][Hq][S] dO . O
    __bf16 *dk, *dv;       // [batch][S][Hkv][D]
    __bf16 *part_dq;       // [batch][Hq][S][nslot][D]
    const uint64_t *lists, *list_off;
    const uint32_t *tile_off, *tile_list;
    int batch, S, Hq, Hkv, G, B, n, topk, nslot, M;
    long long L;
    unsigned ntiles;
    float scale_log2, scale;
};

// LDS rows of D bf16 with their 16-byte chunks XOR-swizzled by the row index,
// so that both kinds of read spread over the banks:
//   row reads, one 16-byte chunk per lane: the rows that share banks in one
//   pass (16 consecutive rows of 256 bytes; the even or the odd ones of 16
//   rows of 128 bytes) get distinct chunks;
//   transposing reads, 32 lanes over rows r0 .. r0 + 3 (r0 a multiple of 4)
//   and four adjacent chunks 4c .. 4c + 3: the rows that share banks land in
//   different aligned groups of four chunks.
// (XOR with r mod 16 alone satisfies the first but puts rows r0 .. r0 + 3 of
// a transposing read on the same four chunks.)
template <int D>
__device__ inline int lds_swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D>
__device__ inline int lds_off(int r, int chunk) {
    return r * D + ((chunk ^ lds_swz<D>(r)) << 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const char lds_char_t;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x4v_t lds_f32x4_t;

// Byte offsets of a lane's reads of a block of 32 LDS rows laid out by lds_off.
//   ro[kk]: the row operand of slice kk -- lane (row = lane % 32, half) gets
//     chunk 2 kk + half of its row.
//   lo[dt], hi[dt]: the transposed operand of the products that sum over the
//     32 rows -- lane (dim = lane % 32, half) receives rows {16 h2 + 4 half + e,
//     16 h2 + 8 + 4 half + e} (e = 0..3) of dimension dt * 32 + lane % 32, in
//     the order the matrix-core result registers hold those rows, by two
//     ds_read_b64_tr_b16 (within 16 lanes, lane j receives element j mod 4 of
//     the 8 bytes lane 4 e + j / 4 addresses).  Offsets for h2 = 0; rows 16 on
//     (h2 = 1) are 32 D bytes further, with the same swizzle.
// In a loop over a ring of LDS slots, refresh() redefines the offsets in place
// at each step through empty asm statements (no instruction): every read then adds
// its slot's address as an immediate offset, instead of each (slot, offset)
// sum being formed once outside the loop and held in a register of its own.
template <int D>
struct ReadOffsets {
    int ro[D / 16], lo[D / 32], hi[D / 32];
    __device__ void init(int lane) {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) ro[kk] = 2 * lds_off<D>(col, 2 * kk + half);
        const int g = lane >> 4, j = lane & 15;
        const int r = 4 * (g >> 1) + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int d = dt * 32 + 16 * (g & 1) + 4 * (j & 3);
            lo[dt] = 2 * (lds_off<D>(r, d >> 3) + (d & 7));
            hi[dt] = 2 * (lds_off<D>(r + 8, d >> 3) + (d & 7));
        }
    }
    __device__ void refresh() {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(ro[kk]));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            asm volatile("" : "+v"(lo[dt]));
            asm volatile("" : "+v"(hi[dt]));
        }
    }
};

// 16 bytes at byte offset off of an LDS block
__device__ inline bf16x8_t lds_rd16(const __bf16 *s, int off) {
    return *reinterpret_cast<const lds_bf16x8_t *>((lds_char_t *)s + off);
}

// the transposed operand (see ReadOffsets) of rows 16 h2 .. 16 h2 + 15
template <int D>
__device__ inline bf16x8_t lds_rd_tr(const __bf16 *s, const ReadOffsets<D> &o, int h2, int dt) {
    lds_char_t *b = (lds_char_t *)s + h2 * 32 * D;
    const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(b + o.lo[dt]));
    const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(b + o.hi[dt]));
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// End of a pipeline step: this wave's memory operations other than the newest
// n have completed and its LDS accesses too, then the workgroup meets (the
// workgroup fence of __syncthreads would wait for every load in flight).
template <int n>
__device__ __forceinline__ void ring_barrier() {
    static_assert(n < 16, "vmcnt immediate");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(n | 0x70);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ inline void pack16(const float (&x)[16], bf16x8_t (&o)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i >> 3][i & 7] = (__bf16)x[i];
}

// ---------------------------------------------------------------- prep

// grid ceil(rows / (256 / (D / 8))), 256 threads; rows in (batch, head, token) order.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16 *__restrict__ out,
                                                       const __bf16 *__restrict__ dout,
                                                       const float *__restrict__ lse,
                                                       float *__restrict__ l2,
                                                       float *__restrict__ delta, int S, int Hq,
                                                       long long rows) {
    constexpr int LPR = D / 8;
    constexpr int RPW = 256 / LPR;
    const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
    const int ch = threadIdx.x % LPR;
    if (row >= rows) return;        // whole rows leave together
    const int t = (int)(row % S);
    const long long bh = row / S;
    const int h = (int)(bh % Hq);
    const long long b = bh / Hq;
    const size_t off = (((size_t)b * S + t) * Hq + h) * D + ch * 8;
    const bf16x8_t o = *reinterpret_cast<const bf16x8_t *>(out + off);
    const bf16x8_t g = *reinterpret_cast<const bf16x8_t *>(dout + off);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, LPR);
    if (ch == 0) {
        delta[row] = acc;
        l2[row] = lse[row] * kLog2e;
    }
}

// ---------------------------------------------------------------- dq

struct DqTile {
    int b, g, h, key_begin, nslice, t0, tend, nrows;
    uint64_t row_begin;
};

template <int MODE>
__device__ inline bool dq_tile(const BwdArgs &a, unsigned tile, DqTile &tl) {
    if (MODE == kPastTile) {
        if (tile >= a.tile_off[a.L]) return false;
        const long long lid = a.tile_list[tile];
        const int j = (int)(lid % a.n);
        tl.g = (int)((lid / a.n) % a.Hkv);
        tl.b = (int)(lid / ((long long)a.n * a.Hkv));
        tl.row_begin = a.list_off[lid] + (uint64_t)(tile - a.tile_off[lid]) * a.M;
        tl.nrows = (int)min((uint64_t)a.M, a.list_off[lid + 1] - tl.row_begin);
        tl.key_begin = j * a.B;
        tl.nslice = a.B / kBS;
        return true;
    }
    if (tile >= a.ntiles) return false;
    const int tpb = (a.B + a.M - 1) / a.M;
    unsigned rest = tile;
    const int tt = rest % tpb; rest /= tpb;
    const int hh = rest % a.G; rest /= a.G;
    const int i = rest % a.n; rest /= a.n;
    tl.g = rest % a.Hkv;
    tl.b = rest / a.Hkv;
    tl.h = tl.g * a.G + hh;
    tl.t0 = i * a.B + tt * a.M;
    tl.tend = min(i * a.B + a.B, a.S);
    if (tl.t0 >= tl.tend) return false;
    tl.key_begin = i * a.B;
    const int tmax = min(tl.t0 + a.M, tl.tend) - 1;
    tl.nslice = (tmax - tl.key_begin) / kBS + 1;
    return true;
}

// 256 rows, 8 waves of 32.  The block's keys come in slices of 32 (K and V)
// through a ring of 4 LDS slots filled straight from global memory
// (global_load_lds), like the kv passes: slices s + 1 .. s + 3 are in flight
// while slice s is worked on.  Every wave issues the same loads per slice
// (D = 128: 4 rows of K and 4 of V; D = 64: 8 rows of K or of V).
template <int D, int MODE>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a) {
    constexpr int SLOT = 2 * kBS * D;      // K slice, V slice
    __shared__ __attribute__((aligned(16))) __bf16 sS0[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sS1[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sS2[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sS3[SLOT];
    DqTile tl;
    // past-block tiles: the grid bounds the count from above (see xcd_tile_counted)
    const unsigned tile = MODE == kPastTile ? xcd_tile_counted(blockIdx.x, a.tile_off[a.L])
                                            : xcd_tile(blockIdx.x, gridDim.x);
    if (!dq_tile<MODE>(a, tile, tl)) return;
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;          // rows per 1 KB load
    constexpr int NV = D == 128 ? 2 : 1;   // loads per slice and wave
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // this lane's query row
    const int r = wave * 32 + col;
    bool valid;
    int t, h, slot;
    if (MODE == kPastTile) {
        valid = r < tl.nrows;
        const uint64_t rec = valid ? a.lists[tl.row_begin + r] : 0ull;
        t = (int)row_t(rec);
        h = tl.g * a.G + (int)row_hh(rec);
        slot = (int)row_slot(rec);
    } else {
        t = tl.t0 + r;
        valid = t < tl.tend;
        h = tl.h;
        slot = a.nslot - 1;
    }
    const int tq = valid ? t : -1;   // OWN: keys after the row are masked
    const size_t qoff = (((size_t)tl.b * a.S + (valid ? t : 0)) * a.Hq + h) * D + half * 8;
    bf16x8_t qf[D / 16], gf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        qf[kk] = *reinterpret_cast<const bf16x8_t *>(a.q + qoff + kk * 16);
        gf[kk] = *reinterpret_cast<const bf16x8_t *>(a.dout + qoff + kk * 16);
        if (!valid)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[kk][e] = gf[kk][e] = (__bf16)0.f;
    }
    const size_t rowid = ((size_t)tl.b * a.Hq + h) * a.S + (valid ? t : 0);
    const float l2r = valid ? a.l2[rowid] : INFINITY;
    const float dr = valid ? a.delta[rowid] : 0.f;

    // staging: this lane's 16-byte piece of key row rq of a slice.  Every key
    // row loaded lies before S: past blocks are whole, and an own tile's last
    // slice ends at its last row rounded up to 32 (S is a multiple of 64).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int rq = (D == 128 ? wave : (wave & 3)) * RPI + lane / CPR;
    const int pc = ((lane % CPR) ^ lds_swz<D>(rq)) << 3;
    const size_t rstride = (size_t)a.Hkv * D;
    const size_t kvoff = ((size_t)tl.b * a.S + tl.key_begin + rq) * rstride + (size_t)tl.g * D + pc;
    const __bf16 *srcA = (D == 128 || wave < 4 ? a.k : a.v) + kvoff;   // K (D = 64: K or V)
    const __bf16 *srcB = a.v + kvoff;                                   // V (D = 128)
    // slices past the last are the last again (loaded, never used)
    auto issue = [&](int hs, __bf16 *dst) {
        const size_t o = (size_t)min(hs, tl.nslice - 1) * kBS * rstride;
        if constexpr (D == 128) {
            __bf16 *d0 = dst + wave_s * RPI * D;
            __builtin_amdgcn_global_load_lds(srcA + o, (lds_void_t *)d0, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(srcB + o, (lds_void_t *)(d0 + kBS * D), 16, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds(
                srcA + o, (lds_void_t *)(dst + (wave_s >> 2) * kBS * D + (wave_s & 3) * RPI * D), 16, 0, 0);
        }
    };

    ReadOffsets<D> offs;
    offs.init(lane);
    f32x16_t dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[dt][i] = 0.f;
    const f32x16_t zero16 = {};

    // The products of slice hs, from slot sl (K, then V).
    auto compute = [&](int hs, const __bf16 *sl) {
        offs.refresh();
        const ReadOffsets<D> &o = offs;
        const __bf16 *k_s = sl, *v_s = sl + kBS * D;
        // S^T = K Q^T and dP^T = V dO^T: rows = 32 keys, columns = query rows
        f32x16_t s = zero16, dp = zero16;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd16(k_s, o.ro[kk]), qf[kk], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd16(v_s, o.ro[kk]), gf[kk], dp, 0, 0, 0);
        }
        // dS^T = P^T (dP^T - delta), P recomputed from the row's log-sum-exp;
        // steps past the last slice weigh nothing
        float ds[16];
        if (hs >= tl.nslice) {
#pragma unroll
            for (int i = 0; i < 16; ++i) ds[i] = 0.f;
        } else {
            const int kbase = tl.key_begin + hs * kBS + 4 * half;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kbase + 8 * (i >> 2) + (i & 3);
                float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -l2r));
                if (MODE != kPastTile && key > tq) p = 0.f;
                ds[i] = p * (dp[i] - dr);
            }
        }
        bf16x8_t db[2];
        pack16(ds, db);
        // dQ^T += K^T dS^T
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd_tr<D>(k_s, o, h2, dt), db[h2],
                                                                 dq[dt], 0, 0, 0);
    };

    issue(0, sS0);
    issue(1, sS1);
    issue(2, sS2);
    // the query rows and the first slices have landed (without this wait the
    // compiler, unsure of the row loads on the path that skips the loop,
    // would wait for them inside it, and so for every slice in flight)
    __builtin_amdgcn_s_waitcnt(0);
    // Step hs: slice hs has landed (after it: slices hs + 1, hs + 2, 2 NV
    // loads), the workgroup meets (every wave is done with slice hs - 1,
    // whose slot takes slice hs + 3), then slice hs is worked on.
    auto step = [&](int hs, const __bf16 *cur, __bf16 *nxt) {
        ring_barrier<2 * NV>();
        issue(hs + 3, nxt);
        compute(hs, cur);
    };
    // a multiple of 4 steps (the loop has one exit)
    const int ns4 = (tl.nslice + 3) & ~3;
    for (int h4 = 0; h4 < ns4; h4 += 4) {
        step(h4, sS0, sS3);
        step(h4 + 1, sS1, sS0);
        step(h4 + 2, sS2, sS1);
        step(h4 + 3, sS3, sS2);
    }
    __builtin_amdgcn_s_waitcnt(0);     // the slices loaded past the last have landed
    if (!valid) return;
    // lane (row, half) holds dims dt * 32 + 8 (i / 4) + 4 half + i % 4
    __bf16 *dst = a.part_dq + (rowid * a.nslot + slot) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(dq[dt][4 * i4 + e] * a.scale);
            *reinterpret_cast<bf16x4_t *>(dst + dt * 32 + 8 * i4 + 4 * half) = w;
        }
}

// grid ceil(rows / (256 / (D / 8))), 256 threads; rows in (batch, head, token) order.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_sum_kernel(const __bf16 *__restrict__ part,
                                                         __bf16 *__restrict__ dq, int S, int Hq,
                                                         int B, int topk, int nslot,
                                                         long long rows) {
    constexpr int LPR = D / 8;
    constexpr int RPW = 256 / LPR;
    const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
    const int ch = threadIdx.x % LPR;
    if (row >= rows) return;
    const int t = (int)(row % S);
    const long long bh = row / S;
    const int h = (int)(bh % Hq);
    const long long b = bh / Hq;
    const int npast = min(topk - 1, t / B);
    const __bf16 *src = part + (size_t)row * nslot * D + ch * 8;
    float acc[8];
    bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(src + (size_t)(nslot - 1) * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = (float)x[e];
    for (int c = 0; c < npast; ++c) {
        x = *reinterpret_cast<const bf16x8_t *>(src + (size_t)c * D);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
    }
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x8_t *>(dq + (((size_t)b * S + t) * Hq + h) * D + ch * 8) = o;
}

// ---------------------------------------------------------------- dk, dv

constexpr int kKeysPerWG = 256;   // 8 waves x 32 keys
enum KvPass { kPassDV = 0, kPassDK = 1 };

// One chunk slot of the kv staging ring: the chunk's 32 Q rows, its 32 dO rows
// (both [row][D], 16-byte chunks swizzled as lds_off), then 8 x 64 floats of
// per-row log-sum-exp and delta.
template <int D>
constexpr int kv_slot_elems() { return 2 * kBS * D + 2 * 8 * 64; }

// The last part of a slot, per row r of the chunk: D = 128: wave r / 4 moves
// rows 4 (r / 4) .. + 3, its 64 floats hold their four log-sum-exps, then
// their four deltas.  D = 64: wave r / 8 moves the log-sum-exps of rows
// 8 (r / 8) .. + 7, wave r / 8 + 4 their deltas.  Four consecutive rows
// r0 .. r0 + 3 (r0 a multiple of 4) are contiguous in both.

// One pass over the query rows that attend a workgroup's 256 keys: the
// block's list (past rows, every key visible), then the block's own rows
// t >= k0 of every head of the group (causal).  PASS dV: S, P, dV^T += dO^T P.
// PASS dK: S, dP, dS, dK^T += Q^T dS.  Two passes instead of one keep each
// under 256 registers, so two waves share a SIMD (one pass holding both
// accumulators and both operands needs one SIMD per wave); S is computed twice.
//
// The rows arrive in chunks of 32 through a ring of 4 LDS slots, moved
// straight from global memory into LDS (global_load_lds: no registers, no
// stores): while chunk c is worked on, chunks c + 1 .. c + 3 are in flight.
// Every wave issues the same four memory operations per chunk (D = 128: its
// 4 rows of Q, its 4 rows of dO, their log-sum-exps and deltas; D = 64: 8
// rows of Q or of dO and their log-sum-exps or deltas; plus the list record of
// its rows 6 chunks ahead, into a register), so one vector-memory count bounds
// what is still in flight.  A list record is loaded 3 chunks before the rows
// it addresses, so it has landed when they are issued.  Rows past the list's
// end reuse its last record and get weight 0; chunks past the last reuse it.
// grid: (ceil(B / 256) key groups x n blocks x batch * Hkv, rounded up to a
// multiple of 8), 512 threads.  Consecutive workgroups -- the key groups of one
// block's list, which read the same query rows -- run on the same XCD.
template <int D, int PASS>
__global__ __launch_bounds__(512) void bwd_kv_kernel(BwdArgs a, int nsub, unsigned nwg) {
    constexpr int SLOT = kv_slot_elems<D>();
    __shared__ __attribute__((aligned(16))) __bf16 sR0[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sR1[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sR2[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 sR3[SLOT];
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;     // rows per 1 KB load
    constexpr int NV = D == 128 ? 4 : 3;   // vector-memory operations per chunk and wave
    const unsigned wg = xcd_tile(blockIdx.x, gridDim.x);
    if (wg >= nwg) return;
    const int sub = (int)(wg % nsub);
    const int j = (int)((wg / nsub) % a.n);
    const int bg = (int)(wg / ((unsigned)nsub * a.n));
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int blk_end = min((j + 1) * a.B, a.S);
    const int k0 = j * a.B + sub * kKeysPerWG;
    if (k0 >= blk_end) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // this lane's key (matrix-core column) and its K (and V) operands
    const int key = k0 + wave * 32 + col;
    const bool kvalid = key < blk_end;
    const size_t rstride = (size_t)a.Hkv * D;
    const size_t koff = ((size_t)b * a.S + (kvalid ? key : k0)) * rstride + (size_t)g * D + half * 8;
    bf16x8_t kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        kf[kk] = *reinterpret_cast<const bf16x8_t *>(a.k + koff + kk * 16);
        if (PASS == kPassDK) vf[kk] = *reinterpret_cast<const bf16x8_t *>(a.v + koff + kk * 16);
    }

    const long long lid = ((long long)b * a.Hkv + g) * a.n + j;
    const uint64_t lbeg = a.list_off[lid];
    const long long nlist = (long long)(a.list_off[lid + 1] - lbeg);
    const int nc1 = (int)((nlist + kBS - 1) / kBS);
    const int own_rows = blk_end - k0;               // a multiple of 64: B and S are
    const int cph = own_rows / kBS;                   // own chunks per head
    const int nc = nc1 + cph * a.G;

    // ---- loads.  The chunk row whose 16-byte piece this lane moves, the
    // piece's place in the row, and the lane's constant part of its addresses.
    // Row, log-sum-exp and list indices fit in 32 bits: the dq partial
    // workspace holds nslot x D values for every (batch, head, token) row.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);     // scalar copy, for the LDS bases
    const int rq = (D == 128 ? wave : (wave & 3)) * RPI + lane / CPR;
    const int pc = ((lane % CPR) ^ lds_swz<D>(rq)) << 3;
    const __bf16 *rowA = (D == 128 || wave < 4 ? a.q : a.dout) + pc;   // Q (D = 64: Q or dO)
    const __bf16 *rowB = a.dout + pc;                                  // dO (D = 128)
    const unsigned rqHq = (unsigned)rq * (unsigned)a.Hq;
    // the row whose log-sum-exp (or delta) this lane moves, within the chunk,
    // and the lane that holds that row's record: D = 128 rows 4 wave + lane % 4,
    // D = 64 rows 8 (wave % 4) + lane % 8 (lanes beyond those repeat them)
    const int ld_row = D == 128 ? 4 * wave + (lane & 3) : 8 * (wave & 3) + (lane & 7);
    const int ld_src = D == 128 ? 16 * (lane & 3) : 8 * (lane & 7);
    const float *ld_base = (D == 128 ? (lane & 4) != 0 : wave >= 4) ? a.delta : a.l2;
    const unsigned bSHq = (unsigned)b * a.S * a.Hq, bHq = (unsigned)b * a.Hq, gG = (unsigned)g * a.G;

    // the list record of row rq of chunk x (clamped into the list; a list with
    // no rows reads a word of the delta array instead, never used)
    const uint64_t *recp = nlist > 0 ? a.lists + lbeg : reinterpret_cast<const uint64_t *>(a.delta);
    const long long rlast = nlist > 0 ? nlist - 1 : 0;
    auto load_rec = [&](int x) -> uint64_t { return recp[min((long long)x * kBS + rq, rlast)]; };
    int iss_c = 0, iss_h = 0;         // odometer of the next own chunk to issue
    // Issue the loads of chunk x into slot dst.
    auto issue = [&](int x, uint64_t rec, __bf16 *dst) {
        unsigned R, rid;              // this lane's row (token-major) and its log-sum-exp row
        if (x < nc1) {
            const unsigned t = row_t(rec), hq = gG + row_hh(rec);
            R = bSHq + t * (unsigned)a.Hq + hq;
            rid = __shfl((bHq + hq) * (unsigned)a.S + t, ld_src, 64);
        } else {
            int c = cph - 1, h = a.G - 1;     // chunks past the last: the last one again
            if (x < nc) {
                c = iss_c;
                h = iss_h;
                if (++iss_c == cph) {
                    iss_c = 0;
                    ++iss_h;
                }
            }
            const unsigned t0 = (unsigned)(k0 + c * kBS), hq = gG + (unsigned)h;
            R = bSHq + t0 * (unsigned)a.Hq + hq + rqHq;
            rid = (bHq + hq) * (unsigned)a.S + t0 + (unsigned)ld_row;
        }
        __bf16 *d0 = dst + wave_s * RPI * D;
        if constexpr (D == 128) {
            __builtin_amdgcn_global_load_lds(rowA + (size_t)R * D, (lds_void_t *)d0, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(rowB + (size_t)R * D, (lds_void_t *)(d0 + kBS * D), 16, 0, 0);
        } else {
            __bf16 *d1 = dst + (wave_s >> 2) * kBS * D + (wave_s & 3) * RPI * D;
            __builtin_amdgcn_global_load_lds(rowA + (size_t)R * D, (lds_void_t *)d1, 16, 0, 0);
        }
        __builtin_amdgcn_global_load_lds(ld_base + rid, (lds_void_t *)(dst + 2 * kBS * D + wave_s * 128),
                                         4, 0, 0);
    };

    // ---- products
    ReadOffsets<D> offs;
    offs.init(lane);
    // byte offsets of the log-sum-exps of rows r0 .. r0 + 3 (r0 = 8 i4 + 4 half)
    // in a slot: LDB + lb + i4 LI4; their deltas LDL further on
    int lb = D == 128 ? 256 * half : 16 * half;
    constexpr int LI4 = D == 128 ? 512 : 256, LDL = D == 128 ? 16 : 1024;
    constexpr int LDB = 2 * kBS * D * 2;

    f32x16_t acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    const f32x16_t zero16 = {};
    int cmp_c = 0;                    // own chunk index within its head, for the next own chunk

    // The products of chunk ci, from slot sl.
    auto compute = [&](int ci, const __bf16 *sl) {
        offs.refresh();
        const ReadOffsets<D> &o = offs;
        asm volatile("" : "+v"(lb));
        const lds_char_t *base = (lds_char_t *)sl;
        // S = Q K^T (and dP = dO V^T): rows = 32 query rows, columns = this wave's keys
        f32x16_t s = zero16, dp = zero16;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd16(sl, o.ro[kk]), kf[kk], s, 0, 0, 0);
            if (PASS == kPassDK)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd16(sl + kBS * D, o.ro[kk]), vf[kk], dp,
                                                             0, 0, 0);
        }
        // register i holds row 8 (i / 4) + 4 half + i % 4.  Keys past the
        // block's end (a short block) are not masked: they only reach their own
        // result columns, which are never stored.  Past-list rows see every key
        // (rows past the list's end none); own rows are masked causally.
        // lim: weight 0 where the row index within the chunk is >= lim (past),
        // or < lim (own: row base + r sees key only if r >= key - base).
        float w[16];
        auto form_w = [&](auto kind_c, int lim) {
            constexpr int kind = decltype(kind_c)::value;   // 0 all rows, 1 rows < lim, 2 rows >= lim
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int r0 = 8 * i4 + 4 * half;
                const f32x4v_t l4 = *reinterpret_cast<const lds_f32x4_t *>(base + LDB + lb + i4 * LI4);
                const float lv[4] = {l4[0], l4[1], l4[2], l4[3]};
                float dvv[4] = {0.f, 0.f, 0.f, 0.f};
                if (PASS == kPassDK) {
                    const f32x4v_t d4 = *reinterpret_cast<const lds_f32x4_t *>(base + LDB + LDL + lb + i4 * LI4);
                    dvv[0] = d4[0]; dvv[1] = d4[1]; dvv[2] = d4[2]; dvv[3] = d4[3];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * i4 + e;
                    float pe = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -lv[e]));
                    if constexpr (kind == 1) {
                        if (r0 + e >= lim) pe = 0.f;
                    } else if constexpr (kind == 2) {
                        if (r0 + e < lim) pe = 0.f;
                    }
                    w[i] = PASS == kPassDV ? pe : pe * (dp[i] - dvv[e]);
                }
            }
        };
        if (ci >= nc) {
            form_w(std::integral_constant<int, 1>(), 0);
        } else if (ci >= nc1) {
            form_w(std::integral_constant<int, 2>(), key - (k0 + cmp_c * kBS));
            if (++cmp_c == cph) cmp_c = 0;
        } else if ((ci + 1) * kBS > nlist) {
            form_w(std::integral_constant<int, 1>(), (int)(nlist - (long long)ci * kBS));
        } else {
            form_w(std::integral_constant<int, 0>(), 0);
        }
        bf16x8_t wb[2];
        pack16(w, wb);
        // dV^T += dO^T P, or dK^T += Q^T dS, over the chunk's 32 rows
        const __bf16 *src = PASS == kPassDV ? sl + kBS * D : sl;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_rd_tr<D>(src, o, h2, dt), wb[h2],
                                                                  acc[dt], 0, 0, 0);
    };

    // Prologue: the records of chunks 0 .. 2 (waited for, with the K / V
    // operands: without this wait the compiler, unsure of them on the path
    // where the loop is skipped, would wait for them inside the loop, and so
    // for every load in flight), then chunks 0 .. 2 issued, each after the
    // record 6 chunks ahead of the one being worked on at that point.
    uint64_t r3 = load_rec(0), r4 = load_rec(1), r5 = load_rec(2);
    __builtin_amdgcn_s_waitcnt(0);
    {
        uint64_t r6 = load_rec(3);
        issue(0, r3, sR0);
        r3 = r4; r4 = r5; r5 = r6;
        r6 = load_rec(4);
        issue(1, r3, sR1);
        r3 = r4; r4 = r5; r5 = r6;
        r6 = load_rec(5);
        issue(2, r3, sR2);
        r3 = r4; r4 = r5; r5 = r6;
    }
    // Step ci: chunk ci has landed (after it: the loads of chunks ci + 1 and
    // ci + 2 and two records, 2 NV operations), the workgroup meets (so every
    // wave is done with chunk ci - 1, whose slot now takes chunk ci + 3),
    // then chunk ci is worked on.
    auto step = [&](int ci, const __bf16 *cur, __bf16 *nxt) {
        ring_barrier<2 * NV>();
        const uint64_t r6 = load_rec(ci + 6);
        issue(ci + 3, r3, nxt);
        r3 = r4; r4 = r5; r5 = r6;
        compute(ci, cur);
    };
    // a multiple of 4 steps (the loop has one exit): steps past the last
    // chunk work on a reloaded copy of it with every weight 0
    const int nc4 = (nc + 3) & ~3;
    for (int c4 = 0; c4 < nc4; c4 += 4) {
        step(c4, sR0, sR3);
        step(c4 + 1, sR1, sR0);
        step(c4 + 2, sR2, sR1);
        step(c4 + 3, sR3, sR2);
    }
    __builtin_amdgcn_s_waitcnt(0);     // the chunks loaded past the last have landed
    if (!kvalid) return;
    // lane (key, half) holds dims dt * 32 + 8 (i / 4) + 4 half + i % 4
    __bf16 *dst = (PASS == kPassDV ? a.dv : a.dk) + ((size_t)b * a.S + key) * rstride +
                  (size_t)g * D;
    const float f = PASS == kPassDV ? 1.f : a.scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[dt][4 * i4 + e] * f);
            *reinterpret_cast<bf16x4_t *>(dst + dt * 32 + 8 * i4 + 4 * half) = o;
        }
}

template <int D>
hipError_t backward_impl(const BwdBuffers &bb, const Problem &p, uint64_t tiles_upper,
                         hipStream_t st) {
    constexpr int RPW = 256 / (D / 8);
    const long long rows = (long long)p.batch * p.Hq * p.S;
    const unsigned rgrid = (unsigned)((rows + RPW - 1) / RPW);
    bwd_prep_kernel<D><<<rgrid, 256, 0, st>>>(static_cast<const __bf16 *>(bb.out),
                                              static_cast<const __bf16 *>(bb.dout), bb.lse,
                                              bb.l2, bb.delta, p.S, p.Hq, rows);
    BwdArgs a;
    a.q = static_cast<const __bf16 *>(bb.q);
    a.k = static_cast<const __bf16 *>(bb.k);
    a.v = static_cast<const __bf16 *>(bb.v);
    a.dout = static_cast<const __bf16 *>(bb.dout);
    a.l2 = bb.l2;
    a.delta = bb.delta;
    a.dk = static_cast<__bf16 *>(bb.dk);
    a.dv = static_cast<__bf16 *>(bb.dv);
    a.part_dq = static_cast<__bf16 *>(bb.part_dq);
    a.lists = bb.lists; a.list_off = bb.list_off; a.tile_off = bb.tile_off;
    a.tile_list = bb.tile_list;
    a.batch = p.batch; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.B = p.B; a.n = p.n;
    a.topk = p.topk;
    a.nslot = bwd_slots(p);
    a.M = tile_rows(p);
    a.L = (long long)p.batch * p.Hkv * p.n;
    a.scale = (float)(1.0 / sqrt((double)p.D));
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
    if (tiles_upper > 0) {
        a.ntiles = 0;
        const unsigned g = (unsigned)((tiles_upper + 7) / 8 * 8);
        bwd_dq_kernel<D, kPastTile><<<g, 512, 0, st>>>(a);
    }
    a.ntiles = (unsigned)(p.batch * p.Hkv * p.n * p.G * ((p.B + a.M - 1) / a.M));
    bwd_dq_kernel<D, kOwnTile><<<(a.ntiles + 7) / 8 * 8, 512, 0, st>>>(a);
    bwd_dq_sum_kernel<D><<<rgrid, 256, 0, st>>>(a.part_dq, static_cast<__bf16 *>(bb.dq), p.S,
                                                p.Hq, p.B, p.topk, a.nslot, rows);
    const int nsub = (p.B + kKeysPerWG - 1) / kKeysPerWG;
    const unsigned nwg = (unsigned)(nsub * p.n * p.batch * p.Hkv);
    bwd_kv_kernel<D, kPassDV><<<(nwg + 7) / 8 * 8, 512, 0, st>>>(a, nsub, nwg);
    bwd_kv_kernel<D, kPassDK><<<(nwg + 7) / 8 * 8, 512, 0, st>>>(a, nsub, nwg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdBuffers &bb, const Problem &p, uint64_t tiles_upper,
                           hipStream_t st) {
    return p.D == 64 ? backward_impl<64>(bb, p, tiles_upper, st)
                     : backward_impl<128>(bb, p, tiles_upper, st);
}

}  // namespace moba
