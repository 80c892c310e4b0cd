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
// so that both the row reads (one 16-byte chunk per lane, 32 rows) and the
// transposing reads (4 rows x 4 dims per 16 lanes) spread over the banks.
template <int D>
__device__ inline int lds_off(int r, int chunk) {
    return r * D + ((chunk ^ (r & (D / 8 - 1))) << 3);
}

// Row operand: lane (row = lane % 32, half) gets chunk 2 kk + half of its row.
template <int D>
__device__ inline bf16x8_t read_row(const __bf16 *s, int r, int kk, int half) {
    return *reinterpret_cast<const bf16x8_t *>(s + lds_off<D>(r, 2 * kk + half));
}

// Transposed operand for the products that sum over the 32 staged rows: lane
// (dim = lane % 32, half) receives rows {16 h2 + 4 half + e, 16 h2 + 8 + 4 half + e}
// (e = 0..3) of dimension dt * 32 + lane % 32, in the order the matrix-core
// result registers hold those rows.  Two ds_read_b64_tr_b16: within 16 lanes,
// lane j receives element j mod 4 of the 8 bytes lane 4 e + j / 4 addresses.
template <int D>
__device__ inline bf16x8_t read_tr(const __bf16 *s, int h2, int dt, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int r = 16 * h2 + 4 * (g >> 1) + (j >> 2);
    const int d = dt * 32 + 16 * (g & 1) + 4 * (j & 3);
    const __bf16 *lo = s + lds_off<D>(r, d >> 3) + (d & 7);
    const __bf16 *hi = s + lds_off<D>(r + 8, d >> 3) + (d & 7);
    const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t *)(lo));
    const bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t *)(hi));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
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

// 256 rows, 8 waves of 32; keys in slices of 32 staged through two LDS buffers.
template <int D, int MODE>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 sK[2][kBS * D];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][kBS * D];
    DqTile tl;
    // past-block tiles: the grid bounds the count from above (see xcd_tile_counted)
    const unsigned tile = MODE == kPastTile ? xcd_tile_counted(blockIdx.x, a.tile_off[a.L])
                                            : xcd_tile(blockIdx.x, gridDim.x);
    if (!dq_tile<MODE>(a, tile, tl)) return;
    constexpr int CPR = D / 8;
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

    // staging: thread -> (key row, chunk) of a slice
    const size_t rstride = (size_t)a.Hkv * D;
    const __bf16 *kb = a.k + ((size_t)tl.b * a.S + tl.key_begin) * rstride + (size_t)tl.g * D;
    const __bf16 *vb = a.v + ((size_t)tl.b * a.S + tl.key_begin) * rstride + (size_t)tl.g * D;
    const int sr = tid / CPR, sc = tid % CPR;
    const bool stager = tid < kBS * CPR;
    uint4 kn = {}, vn = {};
    auto fetch = [&](int hs) {
        if (stager) {
            const size_t o = (size_t)(hs * kBS + sr) * rstride + sc * 8;
            kn = *reinterpret_cast<const uint4 *>(kb + o);
            vn = *reinterpret_cast<const uint4 *>(vb + o);
        }
    };
    auto store = [&](int buf) {
        if (stager) {
            *reinterpret_cast<uint4 *>(&sK[buf][lds_off<D>(sr, sc)]) = kn;
            *reinterpret_cast<uint4 *>(&sV[buf][lds_off<D>(sr, sc)]) = vn;
        }
    };

    f32x16_t dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[dt][i] = 0.f;
    const f32x16_t zero16 = {};
    fetch(0);
    store(0);
    __syncthreads();
    for (int hs = 0; hs < tl.nslice; ++hs) {
        const int buf = hs & 1;
        if (hs + 1 < tl.nslice) fetch(hs + 1);
        const __bf16 *k_s = sK[buf], *v_s = sV[buf];
        // S^T = K Q^T and dP^T = V dO^T: rows = 32 keys, columns = query rows
        f32x16_t s = zero16, dp = zero16;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(k_s, col, kk, half), qf[kk], s,
                                                        0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(v_s, col, kk, half), gf[kk],
                                                         dp, 0, 0, 0);
        }
        // dS^T = P^T (dP^T - delta), P recomputed from the row's log-sum-exp
        float ds[16];
        const int kbase = tl.key_begin + hs * kBS + 4 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + (i & 3);
            float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -l2r));
            if (MODE != kPastTile && key > tq) p = 0.f;
            ds[i] = p * (dp[i] - dr);
        }
        bf16x8_t db[2];
        pack16(ds, db);
        // dQ^T += K^T dS^T
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(k_s, h2, dt, lane),
                                                                 db[h2], dq[dt], 0, 0, 0);
        if (hs + 1 < tl.nslice) store(buf ^ 1);
        __syncthreads();
    }
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

// One pass over the query rows that attend a workgroup's 256 keys: the
// block's list (past rows, every key visible), then the block's own rows
// t >= k0 of every head of the group (causal).  PASS dV: S, P, dV^T += dO^T P.
// PASS dK: S, dP, dS, dK^T += Q^T dS.  Two passes instead of one keep each
// under 256 registers, so two waves share a SIMD (one pass holding both
// accumulators and both operands needs one SIMD per wave); S is computed twice.
// grid: (ceil(B / 256) key groups x n blocks x batch * Hkv, rounded up to a
// multiple of 8), 512 threads.  Consecutive workgroups -- the key groups of one
// block's list, which read the same query rows -- run on the same XCD.
template <int D, int PASS>
__global__ __launch_bounds__(512) void bwd_kv_kernel(BwdArgs a, int nsub, unsigned nwg) {
    // two chunk buffers: chunk c + 1 is stored while others still read chunk c
    __shared__ __attribute__((aligned(16))) __bf16 sQ[2][kBS * D];
    __shared__ __attribute__((aligned(16))) __bf16 sG[2][kBS * D];
    __shared__ __attribute__((aligned(16))) float sL[2][kBS];
    __shared__ __attribute__((aligned(16))) float sD[2][kBS];
    __shared__ __attribute__((aligned(16))) int sT[2][kBS];
    constexpr int CPR = D / 8;
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
    const int own_rows = blk_end - k0;
    const int cph = (own_rows + kBS - 1) / kBS;      // own chunks per head
    const int nc = nc1 + cph * a.G;

    // staging: thread -> one (row, chunk) piece of the Q and dO rows of a chunk
    const int srr = tid / CPR, scc = tid % CPR;
    const bool stager = tid < kBS * CPR;
    uint4 qn = {}, gn = {};
    float ln = INFINITY, dn = 0.f;
    int tn = -1;
    // Rows of chunk ci.  Past-list chunks: the list records, loaded one chunk
    // ahead of the Q / dO loads that need them.  Own chunks: an odometer over
    // (32-row chunk, head of the group), advanced once per fetch (chunks are
    // fetched in order).  Every load reads a valid row (rows past the end are
    // clamped to the last one) and nothing selects on a loaded value before
    // the chunk's products, so no load is waited for early.  A row past the
    // end gets t = -1 and log-sum-exp +inf, hence P = 0.
    auto rec_of = [&](int ci, int rr) -> uint64_t {
        const long long e = min((long long)ci * kBS + rr, nlist - 1);
        return a.lists[lbeg + e];
    };
    uint64_t rec_s = 0, rec_l = 0;     // records of the next chunk to fetch (staging row, row tid)
    int own_c = 0, own_h = 0;          // odometer of the next own chunk
    auto fetch = [&](int ci) {
        int ts, hs, tl, hl;
        bool okl;
        if (ci < nc1) {
            ts = (int)row_t(rec_s);
            hs = g * a.G + (int)row_hh(rec_s);
            tl = (int)row_t(rec_l);
            hl = g * a.G + (int)row_hh(rec_l);
            okl = (long long)ci * kBS + tid < nlist;
        } else {
            const int base = k0 + own_c * kBS;
            ts = min(base + srr, blk_end - 1);
            hs = hl = g * a.G + own_h;
            tl = min(base + tid, blk_end - 1);
            okl = base + tid < blk_end;
            if (++own_c == cph) {
                own_c = 0;
                ++own_h;
            }
        }
        if (stager) {
            const size_t o = (((size_t)b * a.S + ts) * a.Hq + hs) * D + scc * 8;
            qn = *reinterpret_cast<const uint4 *>(a.q + o);
            gn = *reinterpret_cast<const uint4 *>(a.dout + o);
        }
        if (tid < kBS) {
            const size_t rid = ((size_t)b * a.Hq + hl) * a.S + tl;
            ln = a.l2[rid];
            dn = a.delta[rid];
            tn = !okl ? -1 : ci < nc1 ? 0x7fffffff : tl;      // past rows see every key
        }
        // the records of chunk ci + 1
        if (nlist > 0) {
            if (stager) rec_s = rec_of(ci + 1, srr);
            if (tid < kBS) rec_l = rec_of(ci + 1, tid);
        }
    };
    auto store = [&](int buf) {
        if (stager) {
            *reinterpret_cast<uint4 *>(&sQ[buf][lds_off<D>(srr, scc)]) = qn;
            *reinterpret_cast<uint4 *>(&sG[buf][lds_off<D>(srr, scc)]) = gn;
        }
        if (tid < kBS) {
            sL[buf][tid] = tn < 0 ? INFINITY : ln;
            sD[buf][tid] = dn;
            sT[buf][tid] = tn;
        }
    };

    f32x16_t acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    const f32x16_t zero16 = {};
    if (nc > 0) {
        if (nlist > 0) {
            if (stager) rec_s = rec_of(0, srr);
            if (tid < kBS) rec_l = rec_of(0, tid);
        }
        fetch(0);
        store(0);
    }
    // The K (and V) operands have landed before the loop.  Without this wait the
    // compiler, unsure of them on the path where the loop is skipped, waits for
    // them inside the loop, and so for the next chunk's loads as well: that
    // would expose the whole gathered-load latency on every chunk.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int c2 = 0; c2 < nc; c2 += 2)
#pragma unroll
    for (int buf = 0; buf < 2; ++buf) {
        const int ci = c2 + buf;
        if (ci >= nc) break;
        if (ci + 1 < nc) fetch(ci + 1);
        const __bf16 *sq = sQ[buf], *sg = sG[buf];
        // S = Q K^T (and dP = dO V^T): rows = 32 query rows, columns = this wave's keys
        f32x16_t s = zero16, dp = zero16;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(sq, col, kk, half), kf[kk], s,
                                                        0, 0, 0);
            if (PASS == kPassDK)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(sg, col, kk, half),
                                                             vf[kk], dp, 0, 0, 0);
        }
        // register i holds row 8 (i / 4) + 4 half + i % 4.  Keys past the
        // block's end (a short block) are not masked: they only reach their own
        // result columns, which are never stored.  Past-list rows see every key;
        // own rows are masked causally.
        float w[16];
        auto form_w = [&](auto causal_c) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int r0 = 8 * i4 + 4 * half;
                const float4 l4 = *reinterpret_cast<const float4 *>(&sL[buf][r0]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                float dvv[4] = {0.f, 0.f, 0.f, 0.f};
                if (PASS == kPassDK) {
                    const float4 d4 = *reinterpret_cast<const float4 *>(&sD[buf][r0]);
                    dvv[0] = d4.x; dvv[1] = d4.y; dvv[2] = d4.z; dvv[3] = d4.w;
                }
                int tv[4] = {0, 0, 0, 0};
                if constexpr (decltype(causal_c)::value) {
                    const int4 t4 = *reinterpret_cast<const int4 *>(&sT[buf][r0]);
                    tv[0] = t4.x; tv[1] = t4.y; tv[2] = t4.z; tv[3] = t4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * i4 + e;
                    float pe = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -lv[e]));
                    if constexpr (decltype(causal_c)::value) {
                        if (key > tv[e]) pe = 0.f;
                    }
                    w[i] = PASS == kPassDV ? pe : pe * (dp[i] - dvv[e]);
                }
            }
        };
        if (ci >= nc1) form_w(std::true_type());
        else form_w(std::false_type());
        bf16x8_t wb[2];
        pack16(w, wb);
        // dV^T += dO^T P, or dK^T += Q^T dS, over the chunk's 32 rows
        const __bf16 *src = PASS == kPassDV ? sg : sq;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(src, h2, dt, lane),
                                                                  wb[h2], acc[dt], 0, 0, 0);
        // the other buffer was last read before the previous barrier
        if (ci + 1 < nc) store(buf ^ 1);
        __syncthreads();
    }
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
