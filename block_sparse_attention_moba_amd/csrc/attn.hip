// Block-sparse attention over the selected KV blocks, and the online-softmax
// merge of the partial outputs (write-up "MoBA: Mixture of Block Attention",
// implementation steps three to five: per-KV-block attention of the queries
// assigned to it, outputs put back in query order, and an online-softmax
// merge because a query attends its current block plus several history
// blocks; Taiwan AI overview, section "技術細節與優勢": the own block is
// always attended, causally).
//
// Three tile kinds share one kernel body:
//   PAST  : up to 128 listed query rows of one (batch, KV head, past block j)
//           attend all B keys of block j (fully visible, no mask) and write a
//           normalised partial output plus its base-2 log-sum-exp to the
//           row's slot of the partial buffer;
//   OWN   : 128 consecutive query rows of one head attend their own block
//           causally (mask only on the sub-tiles that cross the diagonal) and
//           write the own slot;
//   DENSE : 128 consecutive query rows attend every key <= t and write the
//           final output (full causal attention, used when every causal block
//           is selected).
// Four waves each own 32 query rows.  Keys stream through LDS in sub-tiles of
// 64, double-buffered through registers.  S^T = K Q^T and O^T += V^T P^T run
// on v_mfma_f32_32x32x16_bf16 with fp32 accumulation: a lane holds one query
// column and 16 keys of each 32-key S^T tile, so the softmax row reductions
// are in-lane plus one exchange with lane ^ 32.  The A-operand rows of S^T are
// read from K rows whose index has bits 2 and 3 swapped, which makes the 8
// P values each lane feeds to the PV product 8 consecutive keys; V is stored
// transposed in LDS (register transpose on the way in) so that the V^T
// operand is one 16-byte LDS read.
#include <math.h>

#include "moba_internal.hpp"

namespace moba {

enum Mode { kPast = 0, kOwn = 1, kDense = 2 };

constexpr int kN = 64;      // keys per sub-tile
constexpr int kPad = 8;     // LDS row padding (elements) against bank conflicts

struct AttnArgs {
    const void *q, *k, *v;
    void *out;
    void *part_o;
    float *part_lse;
    const uint64_t *lists, *list_off;
    const uint32_t *tile_off;
    int batch, S, Hq, Hkv, G, B, n, topk;
    long long L;           // number of lists
    unsigned ntiles;       // tiles of OWN / DENSE launches
    float scale_log2;      // log2(e) / sqrt(D)
};

// Rows of one tile, as seen by one thread (row index r inside the tile).
struct Tile {
    int b, g;
    int key_begin;   // first key of the range
    int nsub;        // sub-tiles of kN keys to visit
    int tmin, tmax;  // token range of the tile's rows (OWN / DENSE)
    // PAST
    uint64_t row_begin;
    int nrows;
    // OWN / DENSE
    int t0, h, slot, tend;   // rows t0 + r for t0 + r < tend
};

__device__ inline bool decode_tile(const AttnArgs &a, int mode, Tile &tl) {
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);
    if (mode == kPast) {
        const long long L = a.L;
        if (tile >= a.tile_off[L]) return false;
        long long lo = 0, hi = L;
        while (hi - lo > 1) {
            const long long mid = (lo + hi) >> 1;
            if (a.tile_off[mid] <= tile) lo = mid;
            else hi = mid;
        }
        const long long lid = lo;
        const int j = (int)(lid % a.n);
        tl.g = (int)((lid / a.n) % a.Hkv);
        tl.b = (int)(lid / ((long long)a.n * a.Hkv));
        tl.row_begin = a.list_off[lid] + (uint64_t)(tile - a.tile_off[lid]) * kTileRows;
        const uint64_t rend = a.list_off[lid + 1];
        tl.nrows = (int)min((uint64_t)kTileRows, rend - tl.row_begin);
        tl.key_begin = j * a.B;
        tl.nsub = a.B / kN;
        tl.tmin = 0x7fffffff;
        tl.tmax = 0x7fffffff;
        return true;
    }
    if (tile >= a.ntiles) return false;
    if (mode == kOwn) {
        const int tpb = (a.B + kTileRows - 1) / kTileRows;
        unsigned rest = tile;
        const int tt = rest % tpb; rest /= tpb;
        const int hh = rest % a.G; rest /= a.G;
        const int i = rest % a.n; rest /= a.n;
        tl.g = rest % a.Hkv;
        tl.b = rest / a.Hkv;
        tl.h = tl.g * a.G + hh;
        tl.t0 = i * a.B + tt * kTileRows;
        tl.tend = i * a.B + a.B;
        tl.key_begin = i * a.B;
        tl.slot = min(a.topk, i + 1) - 1;
    } else {
        const int ntt = (a.S + kTileRows - 1) / kTileRows;
        const int bh = tile % (a.batch * a.Hq);
        const int tt = ntt - 1 - (int)(tile / (a.batch * a.Hq));
        tl.b = bh / a.Hq;
        tl.h = bh % a.Hq;
        tl.g = tl.h / a.G;
        tl.t0 = tt * kTileRows;
        tl.tend = a.S;
        tl.key_begin = 0;
        tl.slot = 0;
    }
    tl.tmin = tl.t0;
    tl.tmax = min(tl.t0 + kTileRows, tl.tend) - 1;
    tl.nsub = (tl.tmax - tl.key_begin) / kN + 1;
    return true;
}

// ------------------------------------------------------------------ bf16 MFMA path

template <int D>
struct SmemBF16 {
    __bf16 k[2][kN][D + kPad];
    __bf16 vt[2][D][kN + kPad];
};

template <int D>
struct KVRegs {
    static constexpr int KCH = kN * D / 8 / 256;                // 16-byte K chunks per thread
    static constexpr int VUNITS = (kN / 4) * (D / 8);           // 4 keys x 8 dims units
    static constexpr int VPT = (VUNITS + 255) / 256;            // units per thread
    uint4 k[KCH];
    uint4 v[VPT][4];
};

template <int D>
__device__ inline void kv_load(const __bf16 *__restrict__ kp, const __bf16 *__restrict__ vp,
                               size_t row0, size_t rstride, KVRegs<D> &r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < KVRegs<D>::KCH; ++u) {
        const int c = tid + 256 * u;
        const int key = c / (D / 8), col = c % (D / 8);
        r.k[u] = *reinterpret_cast<const uint4 *>(kp + row0 + key * rstride + col * 8);
    }
#pragma unroll
    for (int u = 0; u < KVRegs<D>::VPT; ++u) {
        const int unit = tid + 256 * u;
        if (unit < KVRegs<D>::VUNITS) {
            const int kg = unit / (D / 8), col = unit % (D / 8);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r.v[u][e] = *reinterpret_cast<const uint4 *>(vp + row0 + (kg * 4 + e) * rstride +
                                                            col * 8);
        }
    }
}

template <int D>
__device__ inline void kv_store(SmemBF16<D> &sm, int buf, const KVRegs<D> &r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < KVRegs<D>::KCH; ++u) {
        const int c = tid + 256 * u;
        const int key = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<uint4 *>(&sm.k[buf][key][col * 8]) = r.k[u];
    }
#pragma unroll
    for (int u = 0; u < KVRegs<D>::VPT; ++u) {
        const int unit = tid + 256 * u;
        if (unit < KVRegs<D>::VUNITS) {
            const int kg = unit / (D / 8), col = unit % (D / 8);
            const uint32_t w0[4] = {r.v[u][0].x, r.v[u][0].y, r.v[u][0].z, r.v[u][0].w};
            const uint32_t w1[4] = {r.v[u][1].x, r.v[u][1].y, r.v[u][1].z, r.v[u][1].w};
            const uint32_t w2[4] = {r.v[u][2].x, r.v[u][2].y, r.v[u][2].z, r.v[u][2].w};
            const uint32_t w3[4] = {r.v[u][3].x, r.v[u][3].y, r.v[u][3].z, r.v[u][3].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // dims col*8 + 2p (low halves) and col*8 + 2p + 1 (high halves), keys kg*4 .. +3
                uint2 lo, hi;
                lo.x = (w0[p] & 0xffffu) | (w1[p] << 16);
                lo.y = (w2[p] & 0xffffu) | (w3[p] << 16);
                hi.x = (w0[p] >> 16) | (w1[p] & 0xffff0000u);
                hi.y = (w2[p] >> 16) | (w3[p] & 0xffff0000u);
                *reinterpret_cast<uint2 *>(&sm.vt[buf][col * 8 + 2 * p][kg * 4]) = lo;
                *reinterpret_cast<uint2 *>(&sm.vt[buf][col * 8 + 2 * p + 1][kg * 4]) = hi;
            }
        }
    }
}

// K row read as A-operand row m of a 32-key S^T tile: bits 2 and 3 of m swapped.
__device__ inline int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    __shared__ SmemBF16<D> sm;
    Tile tl;
    if (!decode_tile(a, MODE, tl)) return;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int r = wave * 32 + col;
    const __bf16 *__restrict__ qp = static_cast<const __bf16 *>(a.q);
    const __bf16 *__restrict__ kp = static_cast<const __bf16 *>(a.k);
    const __bf16 *__restrict__ vp = static_cast<const __bf16 *>(a.v);

    // this lane's query row
    bool rvalid;
    int t, h, slot;
    if (MODE == kPast) {
        rvalid = r < tl.nrows;
        const uint64_t rec = rvalid ? a.lists[tl.row_begin + r] : 0ull;
        t = (int)row_t(rec);
        h = tl.g * a.G + (int)row_hh(rec);
        slot = (int)row_slot(rec);
    } else {
        t = tl.t0 + r;
        rvalid = t < tl.tend;
        h = tl.h;
        slot = tl.slot;
    }
    const int tq = rvalid ? t : 0x7fffffff;    // padding rows never mask anything
    // wave-uniform token range of the wave's rows (OWN / DENSE)
    const int wtmin = (MODE == kPast) ? 0 : tl.t0 + wave * 32;
    const int wtmax = (MODE == kPast) ? 0x7fffffff : min(tl.t0 + wave * 32 + 32, tl.tend) - 1;

    bf16x8_t qf[D / 16];
    if (rvalid) {
        const __bf16 *src = qp + (((size_t)tl.b * a.S + t) * a.Hq + h) * D + half * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t *>(src + kk * 16);
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.f;
    }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale_log2;

    const size_t rstride = (size_t)a.Hkv * D;
    const size_t kvbase = ((size_t)tl.b * a.S) * rstride + (size_t)tl.g * D;
    KVRegs<D> regs;
    kv_load<D>(kp, vp, kvbase + (size_t)tl.key_begin * rstride, rstride, regs);
    kv_store<D>(sm, 0, regs);
    __syncthreads();

    const int krow = key_of_row(col);
    for (int s = 0; s < tl.nsub; ++s) {
        const int buf = s & 1;
        const int kb = tl.key_begin + s * kN;
        const bool more = s + 1 < tl.nsub;
        if (more) kv_load<D>(kp, vp, kvbase + (size_t)(kb + kN) * rstride, rstride, regs);

        if (MODE == kPast || kb <= wtmax) {
            // S^T tiles: rows = keys, columns = this wave's 32 queries
            f32x16_t sacc[kN / 32];
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(
                        &sm.k[buf][kt * 32 + krow][kk * 16 + half * 8]);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[kk], sacc[kt], 0, 0, 0);
                }
            }
            // causal mask on sub-tiles that cross the diagonal
            if (MODE != kPast && kb + kN - 1 > wtmin) {
#pragma unroll
                for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + kt * 32 + 16 * (i >> 3) + 8 * half + 4 * ((i >> 2) & 1) + (i & 3);
                        if (key > tq) sacc[kt][i] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx * sl2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            float psum = 0.f;
            bf16x8_t pb[kN / 32][2];
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], sl2, -m_use));
                    psum += pv;
                    pb[kt][i >> 3][i & 7] = (__bf16)pv;
                }
            l_run = fmaf(l_run, alpha, psum);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(
                            &sm.vt[buf][dt * 32 + col][kt * 32 + 16 * h2 + 8 * half]);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kt][h2], oacc[dt], 0, 0, 0);
                    }
        }
        if (more) kv_store<D>(sm, buf ^ 1, regs);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!rvalid) return;
    const float inv = 1.f / l_tot;
    __bf16 *dst;
    if (MODE == kDense) {
        dst = static_cast<__bf16 *>(a.out) + (((size_t)tl.b * a.S + t) * a.Hq + h) * D;
    } else {
        const size_t row_id = ((size_t)tl.b * a.Hq + h) * a.S + t;
        dst = static_cast<__bf16 *>(a.part_o) + (row_id * a.topk + slot) * D;
        if (half == 0) a.part_lse[row_id * a.topk + slot] = m_run + __log2f(l_tot);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = dt * 32 + 8 * g4 + 4 * half;
            union { __bf16 hv[4]; uint2 u; } pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk.hv[e] = (__bf16)(oacc[dt][4 * g4 + e] * inv);
            *reinterpret_cast<uint2 *>(dst + d0) = pk.u;
        }
}

// ------------------------------------------------------------------ fp32 VALU path
//
// fp32 inputs keep fp32 end to end (no matrix-core rounding).  Two threads
// share a query row, each holding half of the head dimensions; the partial
// dot products meet through one lane exchange.  Keys stream through LDS in
// sub-tiles of 32.

constexpr int kNF = 32;

template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
    __shared__ float ks[kNF][D + 4];
    __shared__ float vs[kNF][D + 4];
    Tile tl;
    if (!decode_tile(a, MODE, tl)) return;
    constexpr int DH = D / 2;
    const int r = threadIdx.x >> 1, dh = threadIdx.x & 1;
    const float *__restrict__ qp = static_cast<const float *>(a.q);
    const float *__restrict__ kp = static_cast<const float *>(a.k);
    const float *__restrict__ vp = static_cast<const float *>(a.v);

    bool rvalid;
    int t, h, slot;
    if (MODE == kPast) {
        rvalid = r < tl.nrows;
        const uint64_t rec = rvalid ? a.lists[tl.row_begin + r] : 0ull;
        t = (int)row_t(rec);
        h = tl.g * a.G + (int)row_hh(rec);
        slot = (int)row_slot(rec);
    } else {
        t = tl.t0 + r;
        rvalid = t < tl.tend;
        h = tl.h;
        slot = tl.slot;
    }
    const int tq = rvalid ? t : 0x7fffffff;
    float qv[DH], o[DH];
#pragma unroll
    for (int i = 0; i < DH; ++i) {
        qv[i] = rvalid ? qp[(((size_t)tl.b * a.S + t) * a.Hq + h) * D + dh * DH + i] : 0.f;
        o[i] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale_log2;
    const size_t rstride = (size_t)a.Hkv * D;
    const size_t kvbase = ((size_t)tl.b * a.S) * rstride + (size_t)tl.g * D;
    const int nsub = (MODE == kPast) ? a.B / kNF : (tl.tmax - tl.key_begin) / kNF + 1;
    for (int s = 0; s < nsub; ++s) {
        const int kb = tl.key_begin + s * kNF;
        __syncthreads();
        for (int e = threadIdx.x; e < kNF * D / 4; e += 256) {
            const int key = e / (D / 4), c4 = e % (D / 4);
            const size_t off = kvbase + (size_t)(kb + key) * rstride + c4 * 4;
            *reinterpret_cast<float4 *>(&ks[key][c4 * 4]) = *reinterpret_cast<const float4 *>(kp + off);
            *reinterpret_cast<float4 *>(&vs[key][c4 * 4]) = *reinterpret_cast<const float4 *>(vp + off);
        }
        __syncthreads();
        float sc[kNF];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kNF; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < DH; ++i) acc = fmaf(qv[i], ks[j][dh * DH + i], acc);
            acc += __shfl_xor(acc, 1, 64);
            sc[j] = (kb + j > tq) ? -INFINITY : acc;
            mx = fmaxf(mx, sc[j]);
        }
        const float m_new = fmaxf(m_run, mx * sl2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DH; ++i) o[i] *= alpha;
#pragma unroll
        for (int j = 0; j < kNF; ++j) {
            const float p = exp2f(fmaf(sc[j], sl2, -m_use));
            l_run += p;
#pragma unroll
            for (int i = 0; i < DH; ++i) o[i] = fmaf(p, vs[j][dh * DH + i], o[i]);
        }
    }
    if (!rvalid) return;
    const float inv = 1.f / l_run;
    float *dst;
    if (MODE == kDense) {
        dst = static_cast<float *>(a.out) + (((size_t)tl.b * a.S + t) * a.Hq + h) * D;
    } else {
        const size_t row_id = ((size_t)tl.b * a.Hq + h) * a.S + t;
        dst = static_cast<float *>(a.part_o) + (row_id * a.topk + slot) * D;
        if (dh == 0) a.part_lse[row_id * a.topk + slot] = m_run + log2f(l_run);
    }
#pragma unroll
    for (int i = 0; i < DH; ++i) dst[dh * DH + i] = o[i] * inv;
}

// ------------------------------------------------------------------ merge
//
// out = sum_s w_s O_s / sum_s w_s with w_s = 2^(lse_s - max lse): the exact
// combination of softmaxes over disjoint key sets.  D/8 threads per row, 8
// dimensions each.

__device__ inline void ld8(const __bf16 *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
__device__ inline void ld8(const float *p, float *f) {
    const float4 x = *reinterpret_cast<const float4 *>(p);
    const float4 y = *reinterpret_cast<const float4 *>(p + 4);
    f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
    f[4] = y.x; f[5] = y.y; f[6] = y.z; f[7] = y.w;
}
__device__ inline void st8(__bf16 *p, const float *f) {
    union { __bf16 h[8]; uint4 u; } pk;
#pragma unroll
    for (int e = 0; e < 8; ++e) pk.h[e] = (__bf16)f[e];
    *reinterpret_cast<uint4 *>(p) = pk.u;
}
__device__ inline void st8(float *p, const float *f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, long long rows) {
    constexpr int TPR = D / 8;
    constexpr int RPW = 256 / TPR;
    const long long row_id = (long long)blockIdx.x * RPW + threadIdx.x / TPR;
    if (row_id >= rows) return;
    const int d0 = (threadIdx.x % TPR) * 8;
    const int t = (int)(row_id % a.S);
    const long long bh = row_id / a.S;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    const int nsel = min(a.topk, t / a.B + 1);
    const float *ls = a.part_lse + row_id * a.topk;
    float mx = -INFINITY;
    for (int s = 0; s < nsel; ++s) mx = fmaxf(mx, ls[s]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    const T *po = static_cast<const T *>(a.part_o) + (size_t)row_id * a.topk * D + d0;
    for (int s = 0; s < nsel; ++s) {
        const float w = exp2f(ls[s] - mx);
        wsum += w;
        float f[8];
        ld8(po + (size_t)s * D, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, f[e], acc[e]);
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    st8(static_cast<T *>(a.out) + (((size_t)b * a.S + t) * a.Hq + h) * D + d0, acc);
}

// ------------------------------------------------------------------ launchers

static AttnArgs make_args(const AttnBuffers &bf, const Problem &p) {
    AttnArgs a;
    a.q = bf.q; a.k = bf.k; a.v = bf.v; a.out = bf.out;
    a.part_o = bf.part_o; a.part_lse = bf.part_lse;
    a.lists = bf.lists; a.list_off = bf.list_off; a.tile_off = bf.tile_off;
    a.batch = p.batch; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.B = p.B; a.n = p.n;
    a.topk = p.topk;
    a.L = (long long)p.batch * p.Hkv * p.n;
    a.ntiles = 0;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
    return a;
}

static unsigned round8(unsigned long long x) { return (unsigned)((x + 7) / 8 * 8); }

template <int MODE>
static hipError_t attn_launch(AttnArgs a, const Problem &p, unsigned grid, hipStream_t st) {
    if (grid == 0) return hipSuccess;
    if (p.dtype == kBF16) {
        if (p.D == 64) attn_bf16_kernel<64, MODE><<<grid, 256, 0, st>>>(a);
        else attn_bf16_kernel<128, MODE><<<grid, 256, 0, st>>>(a);
    } else {
        if (p.D == 64) attn_f32_kernel<64, MODE><<<grid, 256, 0, st>>>(a);
        else attn_f32_kernel<128, MODE><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_attn_past(const AttnBuffers &bf, const Problem &p, uint64_t tiles_upper,
                            hipStream_t st) {
    AttnArgs a = make_args(bf, p);
    return attn_launch<kPast>(a, p, round8(tiles_upper), st);
}

hipError_t launch_attn_own(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    AttnArgs a = make_args(bf, p);
    const unsigned long long tpb = (p.B + kTileRows - 1) / kTileRows;
    a.ntiles = (unsigned)((unsigned long long)p.batch * p.Hkv * p.n * p.G * tpb);
    return attn_launch<kOwn>(a, p, round8(a.ntiles), st);
}

hipError_t launch_attn_dense(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    AttnArgs a = make_args(bf, p);
    const unsigned long long ntt = (p.S + kTileRows - 1) / kTileRows;
    a.ntiles = (unsigned)(ntt * p.batch * p.Hq);
    return attn_launch<kDense>(a, p, round8(a.ntiles), st);
}

hipError_t launch_merge(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    AttnArgs a = make_args(bf, p);
    const long long rows = (long long)p.batch * p.Hq * p.S;
    const int rpw = 256 / (p.D / 8);
    const unsigned grid = (unsigned)((rows + rpw - 1) / rpw);
    if (p.dtype == kBF16) {
        if (p.D == 64) merge_kernel<__bf16, 64><<<grid, 256, 0, st>>>(a, rows);
        else merge_kernel<__bf16, 128><<<grid, 256, 0, st>>>(a, rows);
    } else {
        if (p.D == 64) merge_kernel<float, 64><<<grid, 256, 0, st>>>(a, rows);
        else merge_kernel<float, 128><<<grid, 256, 0, st>>>(a, rows);
    }
    return hipGetLastError();
}

}  // namespace moba
