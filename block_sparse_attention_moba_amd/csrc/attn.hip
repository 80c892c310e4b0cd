// Block-sparse attention over the selected KV blocks, with the online-softmax
// merge of the partial outputs fused into the own-block pass (write-up "MoBA:
// Mixture of Block Attention", implementation steps three to five: per-KV-
// block attention of the queries assigned to it, outputs put back in query
// order, and an online-softmax merge because a query attends its current
// block plus several history blocks; Taiwan AI overview, section
// "技術細節與優勢": the own block is always attended, causally).
//
// Three tile kinds share one kernel body:
//   PAST  : up to 128 listed query rows of one (batch, KV head, past block j)
//           attend all B keys of block j (fully visible, no mask) and write a
//           normalised partial output plus its base-2 log-sum-exp to the
//           row's slot of the partial buffer;
//   OWN   : 128 consecutive query rows of one head attend their own block
//           causally (mask only on the sub-tiles that cross the diagonal),
//           then merge with the row's past-block partials and write the
//           final output;
//   DENSE : 128 consecutive query rows attend every key <= t and write the
//           final output (full causal attention, used when every causal block
//           is selected).
// Four waves each own 32 query rows.  Keys stream through LDS in sub-tiles of
// 64, double-buffered through registers.  S^T = K Q^T and O^T += V^T P^T run
// on v_mfma_f32_32x32x16_bf16 with fp32 accumulation: a lane holds one query
// column and 16 keys of each 32-key S^T tile, so the softmax row reductions
// are in-lane plus one exchange with lane ^ 32.  V is stored transposed in
// LDS (register transpose on the way in) with the key columns of every
// 16-key group in bit-2/bit-3-swapped order: the 8 P values a lane feeds to
// the PV product then sit at 8 consecutive columns, so the V^T operand is one
// 16-byte LDS read, and the K operand rows stay in natural order.  The running maximum is only moved (and O
// rescaled) when a row's new maximum exceeds it by more than 2^8, which
// keeps every exponent <= 2^8 and skips almost all rescales.  Results leave
// through LDS so that every global store writes whole 16-byte pieces of
// contiguous 256-byte rows.
#include <math.h>

#include "moba_internal.hpp"

namespace moba {

enum Mode { kPast = 0, kOwn = 1, kDense = 2 };

constexpr int kN = 64;                // keys per sub-tile
constexpr int kPad = 8;               // LDS row padding (elements) against bank conflicts
constexpr float kRescaleSlack = 8.f;  // log2 units a row max may exceed the running max

struct AttnArgs {
    const void *q, *k, *v;
    void *out;
    void *part_o;
    float *part_lse;
    const uint64_t *lists, *list_off;
    const uint32_t *tile_off;
    int batch, S, Hq, Hkv, G, B, n, topk, nslot;
    long long L;           // number of lists
    unsigned ntiles;       // tiles of OWN / DENSE launches
    float scale_log2;      // log2(e) / sqrt(D)
};

struct Tile {
    int b, g;
    int key_begin;   // first key of the range
    int nsub;        // sub-tiles of kN keys to visit
    int tmax;        // last token of the tile's rows (OWN / DENSE)
    // PAST
    uint64_t row_begin;
    int nrows;
    // OWN / DENSE: rows t0 + r for t0 + r < tend
    int t0, h, tend, npast;
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
        tl.npast = min(a.topk - 1, i);
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
        tl.npast = 0;
    }
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

// LDS column of key k in the transposed V tile: bits 2 and 3 of k swapped.
__host__ __device__ constexpr int vt_col(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ inline void unpack8(const uint4 u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ inline uint4 pack8(const float *f) {
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
    return __builtin_bit_cast(uint4, v);
}

__device__ inline uint2 pack4(float a, float b, float c, float d) {
    bf16x4_t v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    return __builtin_bit_cast(uint2, v);
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(SmemBF16<D>)];
    SmemBF16<D> &sm = *reinterpret_cast<SmemBF16<D> *>(smem_raw);
    Tile tl;
    if (!decode_tile(a, MODE, tl)) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;
    const int r = wave * 32 + col;
    const __bf16 *__restrict__ qp = static_cast<const __bf16 *>(a.q);
    const __bf16 *__restrict__ kp = static_cast<const __bf16 *>(a.k);
    const __bf16 *__restrict__ vp = static_cast<const __bf16 *>(a.v);

    // this lane's query row
    bool rvalid;
    int t, h, slot = 0;
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

    // ---- K / V staging: global -> registers -> LDS (V transposed on the way)
    constexpr int KCH = kN * D / 8 / 256;          // 16-byte K chunks per thread
    constexpr int VUN = (kN / 4) * (D / 8);        // units of 4 keys x 8 dims
    static_assert(VUN <= 256, "one V unit per thread at most");
    const size_t rstride = (size_t)a.Hkv * D;
    const __bf16 *kbase = kp + ((size_t)tl.b * a.S) * rstride + (size_t)tl.g * D;
    const __bf16 *vbase = vp + ((size_t)tl.b * a.S) * rstride + (size_t)tl.g * D;
    const bool vact = (VUN == 256) || tid < VUN;
    // V units: consecutive lanes take consecutive 4-key groups, so one LDS store
    // instruction of 16 lanes fills a whole 128-byte row of the transposed tile
    const int vkg = tid % (kN / 4), vcol = tid / (kN / 4);
    // per-thread K chunk coordinates (chunk c = tid + 256 u)
    const int kc0 = tid, kc1 = tid + 256, kc2 = tid + 512, kc3 = tid + 768;
    uint4 kr0, kr1, kr2, kr3, vr0, vr1, vr2, vr3;

#define MOBA_KLD(c) (*reinterpret_cast<const uint4 *>(ks + ((c) / (D / 8)) * rstride + ((c) % (D / 8)) * 8))
#define MOBA_KST(c, x) (*reinterpret_cast<uint4 *>(&sm.k[buf][(c) / (D / 8)][((c) % (D / 8)) * 8]) = (x))
    auto load_kv = [&](int kb) {
        const __bf16 *ks = kbase + (size_t)kb * rstride;
        kr0 = MOBA_KLD(kc0);
        kr1 = MOBA_KLD(kc1);
        if constexpr (KCH > 2) {
            kr2 = MOBA_KLD(kc2);
            kr3 = MOBA_KLD(kc3);
        }
        if (vact) {
            const __bf16 *vs = vbase + (size_t)(kb + vkg * 4) * rstride + vcol * 8;
            vr0 = *reinterpret_cast<const uint4 *>(vs);
            vr1 = *reinterpret_cast<const uint4 *>(vs + rstride);
            vr2 = *reinterpret_cast<const uint4 *>(vs + 2 * rstride);
            vr3 = *reinterpret_cast<const uint4 *>(vs + 3 * rstride);
        }
    };
    auto store_kv = [&](int buf) {
        MOBA_KST(kc0, kr0);
        MOBA_KST(kc1, kr1);
        if constexpr (KCH > 2) {
            MOBA_KST(kc2, kr2);
            MOBA_KST(kc3, kr3);
        }
        if (vact) {
            // dims vcol*8 + 2p (low halves) and + 2p + 1 (high halves), keys vkg*4 .. +3
            __bf16 *dst = &sm.vt[buf][vcol * 8][vt_col(vkg * 4)];
            constexpr int VS = kN + kPad;
            constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;   // v_perm byte selectors
#define MOBA_VT(p, a0, a1, a2, a3)                                                        \
            {                                                                             \
                uint2 lo, hi;                                                             \
                lo.x = __builtin_amdgcn_perm((a1), (a0), kLo);                            \
                lo.y = __builtin_amdgcn_perm((a3), (a2), kLo);                            \
                hi.x = __builtin_amdgcn_perm((a1), (a0), kHi);                            \
                hi.y = __builtin_amdgcn_perm((a3), (a2), kHi);                            \
                *reinterpret_cast<uint2 *>(dst + (2 * (p)) * VS) = lo;                    \
                *reinterpret_cast<uint2 *>(dst + (2 * (p) + 1) * VS) = hi;                \
            }
            MOBA_VT(0, vr0.x, vr1.x, vr2.x, vr3.x)
            MOBA_VT(1, vr0.y, vr1.y, vr2.y, vr3.y)
            MOBA_VT(2, vr0.z, vr1.z, vr2.z, vr3.z)
            MOBA_VT(3, vr0.w, vr1.w, vr2.w, vr3.w)
#undef MOBA_VT
        }
    };
#undef MOBA_KLD
#undef MOBA_KST

    load_kv(tl.key_begin);
    store_kv(0);
    __syncthreads();

    const f32x16_t zero16 = {};
    for (int s = 0; s < tl.nsub; ++s) {
        const int buf = s & 1;
        const int kb = tl.key_begin + s * kN;
        // prefetch the next sub-tile (the last iteration re-reads the last one)
        load_kv(tl.key_begin + min(s + 1, tl.nsub - 1) * kN);

        if (MODE == kPast || kb <= wtmax) {
            f32x16_t sacc[kN / 32];
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt) {
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(
                        &sm.k[buf][kt * 32 + col][kk * 16 + half * 8]);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        av, qf[kk], kk == 0 ? zero16 : sacc[kt], 0, 0, 0);
                }
            }
            if (MODE != kPast && kb + kN - 1 > wtmin) {
#pragma unroll
                for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                        if (key > tq) sacc[kt][i] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[kt][i], sacc[kt][i + 1]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
            if (__any(mx > m_run + kRescaleSlack)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            }
            float psum = 0.f;
            bf16x8_t pb[kN / 32][2];
#pragma unroll
            for (int kt = 0; kt < kN / 32; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], sl2, -m_run));
                    psum += pv;
                    pb[kt][i >> 3][i & 7] = (__bf16)pv;
                }
            l_run += psum;
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
        if (s + 1 < tl.nsub) store_kv(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    const float lse = m_run + __log2f(l_tot);
    constexpr int LPR = D / 8;          // lanes per 256-byte (D = 128) output row
    constexpr int RPP = 64 / LPR;       // rows per store pass

    if (MODE == kPast) {
        // normalised partial (bf16) -> LDS -> whole-row stores
        __bf16 *stg = reinterpret_cast<__bf16 *>(smem_raw) + wave * 32 * (D + kPad);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                *reinterpret_cast<uint2 *>(stg + col * (D + kPad) + dt * 32 + 8 * g4 + 4 * half) =
                    pack4(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv,
                          oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
            }
        const long long row_slot_id =
            rvalid ? (((long long)tl.b * a.Hq + h) * a.S + t) * a.nslot + slot : -1ll;
        if (rvalid && half == 0) a.part_lse[row_slot_id] = lse;
        __syncthreads();
        __bf16 *po = static_cast<__bf16 *>(a.part_o);
        const int lo32 = (int)(row_slot_id & 0xffffffffll), hi32 = (int)(row_slot_id >> 32);
#pragma unroll
        for (int it = 0; it < 32 / RPP; ++it) {
            const int rr = it * RPP + lane / LPR, ch = lane % LPR;
            const long long id = ((long long)__shfl(hi32, rr, 64) << 32) |
                                 (unsigned)__shfl(lo32, rr, 64);
            if (id >= 0)
                *reinterpret_cast<uint4 *>(po + id * D + ch * 8) =
                    *reinterpret_cast<const uint4 *>(stg + rr * (D + kPad) + ch * 8);
        }
        return;
    }

    // OWN / DENSE: own result (fp32) -> LDS, then merge with the past partials
    float *stf = reinterpret_cast<float *>(smem_raw) + wave * 32 * (D + 4);
    float *stl = reinterpret_cast<float *>(smem_raw) + 4 * 32 * (D + 4) + wave * 32;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4 *>(stf + col * (D + 4) + dt * 32 + 8 * g4 + 4 * half) =
                make_float4(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv,
                            oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
    if (half == 0) stl[col] = lse;
    __syncthreads();
    const __bf16 *po = static_cast<const __bf16 *>(a.part_o);
    __bf16 *outp = static_cast<__bf16 *>(a.out);
#pragma unroll
    for (int it = 0; it < 32 / RPP; ++it) {
        const int rr = it * RPP + lane / LPR, ch = lane % LPR;
        const int tr = tl.t0 + wave * 32 + rr;
        if (tr >= tl.tend) continue;
        float o[8];
        const float4 x0 = *reinterpret_cast<const float4 *>(stf + rr * (D + 4) + ch * 8);
        const float4 x1 = *reinterpret_cast<const float4 *>(stf + rr * (D + 4) + ch * 8 + 4);
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
        if (MODE == kOwn && tl.npast > 0) {
            const long long rid = (((long long)tl.b * a.Hq + tl.h) * a.S + tr) * a.nslot;
            const float lo = stl[rr];
            float mxl = lo;
            for (int sl = 0; sl < tl.npast; ++sl) mxl = fmaxf(mxl, a.part_lse[rid + sl]);
            const float wo = exp2f(lo - mxl);
            float wsum = wo;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= wo;
            for (int sl = 0; sl < tl.npast; ++sl) {
                const float w = exp2f(a.part_lse[rid + sl] - mxl);
                wsum += w;
                float f[8];
                unpack8(*reinterpret_cast<const uint4 *>(po + (rid + sl) * D + ch * 8), f);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(w, f[e], o[e]);
            }
            const float iw = 1.f / wsum;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= iw;
        }
        *reinterpret_cast<uint4 *>(outp + (((size_t)tl.b * a.S + tr) * a.Hq + tl.h) * D + ch * 8) =
            pack8(o);
    }
}

// ------------------------------------------------------------------ fp32 VALU path
//
// fp32 inputs keep fp32 end to end (no matrix-core rounding).  Two threads
// share a query row, each holding half of the head dimensions; the partial
// dot products meet through one lane exchange.  Keys stream through LDS in
// sub-tiles of 32.  The own-block pass merges the past partials of its row.

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
    int t, h, slot = 0;
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
    const float lse = m_run + log2f(l_run);
    const long long row_id = ((long long)tl.b * a.Hq + h) * a.S + t;
    if (MODE == kPast) {
        float *dst = static_cast<float *>(a.part_o) + (row_id * a.nslot + slot) * D + dh * DH;
#pragma unroll
        for (int i = 0; i < DH; ++i) dst[i] = o[i] * inv;
        if (dh == 0) a.part_lse[row_id * a.nslot + slot] = lse;
        return;
    }
#pragma unroll
    for (int i = 0; i < DH; ++i) o[i] *= inv;
    if (MODE == kOwn && tl.npast > 0) {
        const float *ls = a.part_lse + row_id * a.nslot;
        float mxl = lse;
        for (int sl = 0; sl < tl.npast; ++sl) mxl = fmaxf(mxl, ls[sl]);
        const float wo = exp2f(lse - mxl);
        float wsum = wo;
#pragma unroll
        for (int i = 0; i < DH; ++i) o[i] *= wo;
        for (int sl = 0; sl < tl.npast; ++sl) {
            const float w = exp2f(ls[sl] - mxl);
            wsum += w;
            const float *src = static_cast<const float *>(a.part_o) + (row_id * a.nslot + sl) * D + dh * DH;
#pragma unroll
            for (int i = 0; i < DH; ++i) o[i] = fmaf(w, src[i], o[i]);
        }
#pragma unroll
        for (int i = 0; i < DH; ++i) o[i] /= wsum;
    }
    float *dst = static_cast<float *>(a.out) + (((size_t)tl.b * a.S + t) * a.Hq + h) * D + dh * DH;
#pragma unroll
    for (int i = 0; i < DH; ++i) dst[i] = o[i];
}

// ------------------------------------------------------------------ launchers

static AttnArgs make_args(const AttnBuffers &bf, const Problem &p) {
    AttnArgs a;
    a.q = bf.q; a.k = bf.k; a.v = bf.v; a.out = bf.out;
    a.part_o = bf.part_o; a.part_lse = bf.part_lse;
    a.lists = bf.lists; a.list_off = bf.list_off; a.tile_off = bf.tile_off;
    a.batch = p.batch; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.B = p.B; a.n = p.n;
    a.topk = p.topk;
    a.nslot = part_slots(p);
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

}  // namespace moba
