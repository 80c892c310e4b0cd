// Block-sparse attention over the selected KV blocks (write-up "MoBA:
// Mixture of Block Attention", implementation steps three and four: per-KV-
// block attention of the queries assigned to it, outputs put back in query
// order; Taiwan AI overview, section "技術細節與優勢": the own block is always
// attended, causally).  The online-softmax merge of step five is in merge.hip.
//
// Three tile kinds share one kernel body:
//   PAST  : up to M listed query rows of one (batch, KV head, past block j)
//           attend all B keys of block j (fully visible, no mask) and write a
//           normalised partial output plus its base-2 log-sum-exp to the
//           row's slot of the partial buffer;
//   OWN   : M consecutive query rows of one head attend their own block
//           causally (mask only on the slices that cross the diagonal) and
//           write the own-block partial, or the final output when the rows
//           have no past blocks;
//   DENSE : M consecutive query rows attend every key <= t and write the
//           final output (full causal attention, used when every causal block
//           is selected).
// M is 256 for bf16 (matrix-core path below) and 128 for fp32 (vector path).
// On the bf16 path results leave through LDS so that every global store
// writes whole 16-byte pieces of contiguous rows.
#include <math.h>

#include <type_traits>

#include "moba_internal.hpp"

namespace moba {

enum Mode { kPast = 0, kOwn = 1, kDense = 2 };

// Thread and workgroup indices straight from the hardware registers.  This
// file is built without IEEE mode, so the device library's index helpers
// (built with it) are not inlined here: they would be calls, and their
// results would not be known to be uniform.
__device__ inline int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ inline unsigned wg_x() { return __builtin_amdgcn_workgroup_id_x(); }

constexpr float kRescaleSlack = 8.f;  // log2 units a row max may exceed the running max

struct AttnArgs {
    const void *q, *k, *v;
    void *out;
    void *part_o;
    float *part_lse;
    const uint64_t *lists, *list_off;
    const uint32_t *tile_off, *tile_list;
    const float *kmax2;    // [batch][Hkv][n] largest squared key norm per block
    int batch, S, Hq, Hkv, G, B, n, topk, nslot;
    int r0, R;             // query chunk [r0, r0 + R): partial buffers are chunk-local
    int M;                 // query rows per tile
    int dense_heads;       // DENSE: heads per tile (M / dense_heads tokens of each); else 1
    long long L;           // number of lists
    unsigned ntiles;       // tiles of OWN / DENSE launches
    unsigned nwg;          // workgroups of the launch
    float scale_log2;      // log2(e) / sqrt(D)
    unsigned *defer_count;  // tiles whose logit bound fails, for the tracking pass
    unsigned *defer_list;
    float *lse_out;         // optional natural-log LSE of rows written to the output
    int fuse_merge;         // OWN (bf16): merge rows with past blocks here, no merge kernel
};

struct Tile {
    int b, g;
    int key_begin;   // first key of the range
    int nslice;      // slices of 32 keys to visit (bf16 path)
    int tmax;        // last token of the tile's rows (OWN / DENSE)
    // PAST
    uint64_t row_begin;
    int nrows;
    // OWN / DENSE: rows t0 + r for t0 + r < tend
    int t0, h, tend, npast;
};

// Load of index data written by an earlier kernel, through the constant
// address space: a scalar load for a uniform address, even after this
// kernel's own stores (which never touch these arrays).
template <typename T>
__device__ inline T ld_index(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// This workgroup's tile.  PAST / OWN: consecutive tiles share keys, so each
// XCD takes a contiguous share (past-block launches are sized by an upper
// bound on the tile count, so their shares come from the count itself).
// DENSE: tiles are ordered longest first, so a contiguous share would leave
// one XCD with all the long tiles; the workgroup index itself deals them
// round-robin (XCD x gets every 8th tile, longest first), and with the
// (token range, KV group) order the tiles an XCD runs together read the same
// keys whenever the group count divides 8.
__device__ inline unsigned first_tile(const AttnArgs &a, int mode) {
    if (mode == kPast) return xcd_tile_counted(wg_x(), ld_index(a.tile_off + a.L));
    return mode == kDense ? wg_x() : xcd_tile(wg_x(), a.nwg);
}

__device__ inline bool decode_tile(const AttnArgs &a, int mode, unsigned tile, Tile &tl) {
    if (mode == kPast) {
        if (tile >= ld_index(a.tile_off + a.L)) return false;
        const long long lid = ld_index(a.tile_list + tile);
        const int j = (int)(lid % a.n);
        tl.g = (int)((lid / a.n) % a.Hkv);
        tl.b = (int)(lid / ((long long)a.n * a.Hkv));
        tl.row_begin = ld_index(a.list_off + lid) + (uint64_t)(tile - ld_index(a.tile_off + lid)) * a.M;
        const uint64_t rend = ld_index(a.list_off + lid + 1);
        tl.nrows = (int)min((uint64_t)a.M, rend - tl.row_begin);
        tl.key_begin = j * a.B;
        tl.nslice = a.B / 32;
        tl.tmax = 0x7fffffff;
        return true;
    }
    if (tile >= a.ntiles) return false;
    if (mode == kOwn) {
        const int tpb = (a.B + a.M - 1) / a.M;
        const int nr = (a.R + a.B - 1) / a.B;       // blocks of the chunk
        unsigned rest = tile;
        const int tt = rest % tpb; rest /= tpb;
        const int hh = rest % a.G; rest /= a.G;
        const int i = a.r0 / a.B + (int)(rest % nr); rest /= nr;
        tl.g = rest % a.Hkv;
        tl.b = rest / a.Hkv;
        tl.h = tl.g * a.G + hh;
        tl.t0 = i * a.B + tt * a.M;
        tl.tend = min(i * a.B + a.B, a.S);     // a short last block ends at S
        if (tl.t0 >= tl.tend) return false;    // tiles past the end of a short block
        tl.key_begin = i * a.B;
        tl.npast = min(a.topk - 1, i);
    } else {
        // M / Gd tokens of Gd heads of one KV group (heads h .. h + Gd - 1), the
        // latest (heaviest) token ranges first
        const int hpt = a.dense_heads, TT = a.M / hpt, nhc = a.Hq / hpt;
        const int ntt = (a.S + TT - 1) / TT;
        const int bhc = tile % (a.batch * nhc);
        const int tt = ntt - 1 - (int)(tile / (a.batch * nhc));
        tl.b = bhc / nhc;
        tl.h = (bhc % nhc) * hpt;
        tl.g = tl.h / a.G;
        tl.t0 = tt * TT;
        tl.tend = a.S;
        tl.key_begin = 0;
        tl.npast = 0;
    }
    tl.tmax = min(tl.t0 + a.M / a.dense_heads, tl.tend) - 1;
    tl.nslice = (tl.tmax - tl.key_begin) / 32 + 1;
    return true;
}

// ------------------------------------------------------------------ bf16 MFMA path
//
// One workgroup = 256 query rows: 8 waves of 32 rows for d = 128 (two waves
// per SIMD, up to 256 registers each), 4 waves of 64 rows (two 32-query column
// groups, so every K or V^T operand read from LDS feeds two MFMAs) for d = 64.
// Keys are consumed in slices of 32.  Step h pairs the matrix-core work of one
// slice with the vector work of the previous one:
//   S(h+1) = K(h+1) Q^T    (matrix cores)
//   P(h) = 2^(S(h) - m), row sums, O += V(h)^T P(h)^T
//   mask and row max of S(h+1), so that step h+1 knows whether its running
//   maximum has to move before it exponentiates.
//
// K and V travel from global memory straight into LDS (global_load_lds, 16
// bytes per lane, no registers) as row-major [key][d] slices whose 16-byte
// chunks are XOR-swizzled per row.  Both rings have 4 slots: step h reads
// V(h) and the K operand of slice h+2 while K(h+4) and V(h+3) start loading,
// so every load has about two steps to land.  The compiler must see that no read aliases a load in
// flight, or it waits for the load before the read, so every slot is its own
// LDS array and the loop is unrolled by 4 with the slots named at each step.
// K operand rows are single 16-byte reads (swizzle: row mod 16).  The V^T
// operand of the PV product is assembled by two transposing reads
// (ds_read_b64_tr_b16): within each 16-lane group, lane j receives element
// j mod 4 of the 8 bytes that lane 4e + j/4 addresses, for e = 0..3, so 16
// lanes addressing 4 key rows x 4 dim chunks each receive 4 keys of one dim.
// The V swizzle (chunk ^ {0, 4, 10, 14}[row mod 4]) keeps both 16-lane and
// 32-lane servicing of those reads conflict-free.
//
// Logits are taken in log2 units (scaled by log2(e)/sqrt(d)).  Every logit of
// a tile is bounded by |q| * max|k| (Cauchy-Schwarz, max|k| per block from
// the pool pass).  When that bound is <= 64 for every row of the tile, 2^s can
// neither overflow nor underflow, so the softmax runs against a fixed
// reference of 0: no row max, no rescale, no subtraction.  Otherwise the tile
// goes to the tracking pass, which keeps a running max (moved lazily, only
// when a row max exceeds it by more than 2^8).

// Rows per tile and waves per workgroup (rows per wave in 32-row column
// groups).  d = 128: 32 rows per wave, two waves per SIMD, so one wave's
// matrix-core work overlaps the other's vector work (measured: same
// past-block speed, own-block pass 13% faster than 4 waves of 64 rows); past-
// block and dense tiles hold 256 rows (8 waves, one workgroup per CU), own-
// block tiles 128 (4 waves, two workgroups per CU: one's merge epilogue, bound
// by HBM, runs beside the other's key loop).  d = 64: 4 waves of 64 rows (the
// 32-key slice staging needs at least 64 lanes x 16 B per wave).
template <int D, int MODE>
constexpr int attn_rows() { return (D == 128 && MODE == kOwn) ? 128 : 256; }
template <int D, int MODE>
constexpr int attn_waves() { return D == 128 ? attn_rows<D, MODE>() / 32 : 4; }
// waves per SIMD the launch bounds ask for: 2 for the 4-wave d = 128 tiles (two
// workgroups per CU, at most 256 registers each), else 1
template <int D, int MODE>
constexpr int attn_occupancy() { return (D == 128 && attn_waves<D, MODE>() == 4) ? 2 : 1; }
constexpr int kS = 32;                 // keys per slice

// 16-byte chunk swizzles (XOR on the chunk index within a row)
template <int D>
__device__ inline int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ inline int swz_v(int r) {
    if constexpr (D == 128) return (0xEA40 >> (4 * (r & 3))) & 15;   // {0, 4, 10, 14}
    else return 2 * (r & 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) __bf16 lds_bf16_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline void unpack8(const uint4 u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

__device__ inline uint4 pack8(const float *f) {
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
    return __builtin_bit_cast(uint4, v);
}

// Four floats as bf16, in one 64-bit word (a single 8-byte LDS store: split
// into two 32-bit stores, the second one loses the LDS alias information and
// the compiler then waits for every LDS-bound load in flight before it).
__device__ inline uint64_t pack4(float a, float b, float c, float d) {
    bf16x4_t v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    return __builtin_bit_cast(uint64_t, v);
}

// End of a pipeline step: this wave's loads other than the newest n have
// landed and its LDS reads have completed (vmcnt <= n, lgkmcnt = 0), then the
// workgroup meets.  A plain s_barrier: the workgroup fence of __syncthreads
// would also wait for the newest loads.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
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

// The workgroup meets once this wave's LDS accesses have completed
// (lgkmcnt = 0); its vector memory accesses in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7: no wait; lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Online-softmax merge of an own tile's rows with the partial outputs of
// their past blocks (write-up "MoBA: Mixture of Block Attention",
// implementation step five), in the tile's epilogue: the merge kernel's order
// of operations (with the hardware exp2 and log2), on the same bf16 own-block
// row, read from the LDS staging instead of its partial slot.  With l_j the
// base-2 log-sum-exp of part j and o_j its normalised output:
// out = sum_j 2^(l_j - M) o_j / sum_j 2^(l_j - M), M the largest l_j.
// Lane (row rr, 16-byte piece ch) as in the store pass;
// two rows per lane at a time, every slot's loads issued before any is used
// (slots past the row's count read its last slot again and get weight 0).
template <int D, int NG>
__device__ __forceinline__ void merge_rows(const AttnArgs &a, const Tile &tl, lds_bf16_t *(&stg)[NG],
                                           const long long (&dst)[NG], const long long (&prow)[NG],
                                           const float (&lse)[NG]) {
    constexpr int CPR = D / 8, LPR = D / 8, RPP = 64 / LPR;
    const int lane = tid_x() & 63, ch = lane % LPR;
    const int np = tl.npast;           // 1 .. kFuseMaxPast
    const __bf16 *po = static_cast<const __bf16 *>(a.part_o);
    __bf16 *outp = static_cast<__bf16 *>(a.out);
    // natural-log LSE index of partial row pr: same (batch, head), token r0 + (pr mod R)
    const long long lse_shift = ((long long)tl.b * a.Hq + tl.h) * (a.S - a.R) + a.r0;
    const long long prow_last = (long long)a.batch * a.Hq * a.R - 1;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int it = 0; it < 32 / RPP; it += 2) {
            int rr[2];
            long long o[2], pr[2];
            float lown[2];
            uint4 pc[2][kFuseMaxPast];
            float lv[2][kFuseMaxPast];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                rr[u] = (it + u) * RPP + lane / LPR;     // lane rr holds row rr
                o[u] = __shfl(dst[g], rr[u], 64);
                pr[u] = __shfl(prow[g], rr[u], 64);
                lown[u] = __shfl(lse[g], rr[u], 64);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                // a padding row reads some partial row (clamped into the buffer) and stores nothing
                if (o[u] < 0) pr[u] = min(pr[u], prow_last);
                const __bf16 *src = po + pr[u] * a.nslot * D + ch * 8;
                const float *ls = a.part_lse + pr[u] * a.nslot;
#pragma unroll
                for (int s4 = 0; s4 < kFuseMaxPast; s4 += 4) {
                    if (s4 >= np) break;
#pragma unroll
                    for (int s = s4; s < s4 + 4; ++s) {
                        const int sc = min(s, np - 1);
                        pc[u][s] = *reinterpret_cast<const uint4 *>(src + (size_t)sc * D);
                        lv[u][s] = ls[sc];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (o[u] < 0) continue;
                float acc[8];
                const bf16x8_t own = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
                    stg[g] + rr[u] * D + ((ch ^ (rr[u] & (CPR - 1))) << 3));
                unpack8(__builtin_bit_cast(uint4, own), acc);
                float mx = lown[u];
#pragma unroll
                for (int s4 = 0; s4 < kFuseMaxPast; s4 += 4) {
                    if (s4 >= np) break;
#pragma unroll
                    for (int s = s4; s < s4 + 4; ++s) mx = fmaxf(mx, lv[u][s]);
                }
                const float w_own = __builtin_amdgcn_exp2f(lown[u] - mx);
                float wsum = w_own;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] *= w_own;
#pragma unroll
                for (int s4 = 0; s4 < kFuseMaxPast; s4 += 4) {
                    if (s4 >= np) break;
#pragma unroll
                    for (int s = s4; s < s4 + 4; ++s) {
                        const float w = s < np ? __builtin_amdgcn_exp2f(lv[u][s] - mx) : 0.f;
                        wsum += w;
                        float f[8];
                        unpack8(pc[u][s], f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, f[e], acc[e]);
                    }
                }
                const float iw = 1.f / wsum;
                if (a.lse_out && ch == 0) a.lse_out[pr[u] + lse_shift] = (mx + __log2f(wsum)) * kLn2;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] *= iw;
                __builtin_nontemporal_store(__builtin_bit_cast(bf16x8_t, pack8(acc)),
                                            reinterpret_cast<bf16x8_t *>(outp + o[u] + ch * 8));
            }
        }
    }
}

// One tile.  FAST: the bounded softmax; a tile whose bound fails is appended
// to the deferred list and left to the tracking pass.  !FAST: running-max
// tracking.  PAD (PAST only): the block's slice count is not a multiple of 4,
// so the loop runs up to 2 padding slices that must be emptied.  sK0..sK3 are
// the K ring slots, sV0..sV3 the V slots; each is its own LDS array, and the
// caller passes them in by name; sFlag holds one word per wave.
template <int D, int MODE, bool FAST, bool PAD, int NW>
__device__ __forceinline__ void attn_bf16_tile(const AttnArgs &a, unsigned tile, __bf16 *sK0,
                                               __bf16 *sK1, __bf16 *sK2, __bf16 *sK3, __bf16 *sV0,
                                               __bf16 *sV1, __bf16 *sV2, __bf16 *sV3, int *sFlag) {
    constexpr int ROWS = attn_rows<D, MODE>();
    constexpr int RPW = ROWS / NW;      // query rows per wave
    constexpr int NG = RPW / 32;        // 32-row column groups per wave
    static_assert(NG >= 1 && RPW * NW == ROWS, "wave layout");
    Tile tl;
    if (!decode_tile(a, MODE, tile, tl)) return;

    int tid = tid_x();
    // An opaque copy, so that in the kernels that loop over tiles the
    // lane-dependent addresses are recomputed per tile instead of hoisted out
    // of the tile loop, where they would stay live across the key loop.
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave: scalar
    const int col = lane & 31, half = lane >> 5;
    const __bf16 *__restrict__ qp = static_cast<const __bf16 *>(a.q);
    const __bf16 *__restrict__ kp = static_cast<const __bf16 *>(a.k);
    const __bf16 *__restrict__ vp = static_cast<const __bf16 *>(a.v);
    const int nh = tl.nslice;
    // OWN / DENSE: row r of the tile is token t0 + r mod TT of head h + r / TT
    const int TT = a.M / a.dense_heads;
    const int wfirst = tl.t0 + (wave * RPW) % TT;   // the wave's first row (one head per wave)

    // this lane's two query rows (column groups g = 0, 1)
    bool rvalid[NG];
    int t[NG], h[NG], slot[NG], tq[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int r = wave * RPW + g * 32 + col;
        slot[g] = 0;
        if (MODE == kPast) {
            rvalid[g] = r < tl.nrows;
            const uint64_t rec = rvalid[g] ? a.lists[tl.row_begin + r] : 0ull;
            t[g] = (int)row_t(rec);
            h[g] = tl.g * a.G + (int)row_hh(rec);
            slot[g] = (int)row_slot(rec);
        } else {
            t[g] = tl.t0 + r % TT;
            rvalid[g] = t[g] < tl.tend;
            h[g] = tl.h + r / TT;
        }
        tq[g] = rvalid[g] ? t[g] : 0x7fffffff;    // padding rows never mask anything
    }

    // ---- K / V staging: global -> LDS directly, 1 KB (64 lanes x 16 B) per instruction
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;           // rows per instruction
    constexpr int IPS = kS / RPI / NW;      // instructions per wave per slice
    static_assert(IPS >= 1, "slice too small for the staging pattern");
    const size_t rstride = (size_t)a.Hkv * D;
    const size_t kvoff = ((size_t)tl.b * a.S + tl.key_begin) * rstride + (size_t)tl.g * D;
    // uniform across the workgroup: kept in scalar registers for the loads' base
    const size_t kvoff_u = ((size_t)__builtin_amdgcn_readfirstlane((unsigned)(kvoff >> 32)) << 32) |
                           (unsigned)__builtin_amdgcn_readfirstlane((unsigned)kvoff);
    const __bf16 *kbase = kp + kvoff_u;
    const __bf16 *vbase = vp + kvoff_u;
    // element offsets (row * rstride + chunk * 8) this lane loads in each of its instructions
    unsigned ld_k[IPS], ld_v[IPS];
#pragma unroll
    for (int i = 0; i < IPS; ++i) {
        const int r = (wave * IPS + i) * RPI + lane / CPR, pc = lane % CPR;
        ld_k[i] = (unsigned)(r * (int)rstride + ((pc ^ swz_k<D>(r)) << 3));
        ld_v[i] = (unsigned)(r * (int)rstride + ((pc ^ swz_v<D>(r)) << 3));
    }
    // slices past the last are clamped to it (loaded again, never used)
    // byte offsets: a uniform base plus a 32-bit lane offset is the load's
    // scalar-base form, with no 64-bit address arithmetic per load
#pragma unroll
    for (int i = 0; i < IPS; ++i) {
        ld_k[i] *= 2u;
        ld_v[i] *= 2u;
    }
    // (the empty asm keeps the compiler from hoisting the 64-bit lane
    // addresses out of the key loop, which would cost a 64-bit add per load)
    auto load_k = [&](int hs, __bf16 *dst) {
        const char *src = reinterpret_cast<const char *>(kbase + (size_t)(min(hs, nh - 1) * kS) * rstride);
#pragma unroll
        for (int i = 0; i < IPS; ++i) {
            asm volatile("" : "+v"(ld_k[i]));
            __builtin_amdgcn_global_load_lds(src + ld_k[i], (lds_void_t *)(dst + (wave * IPS + i) * 512),
                                             16, 0, 0);
        }
    };
    auto load_v = [&](int hs, __bf16 *dst) {
        const char *src = reinterpret_cast<const char *>(vbase + (size_t)(min(hs, nh - 1) * kS) * rstride);
#pragma unroll
        for (int i = 0; i < IPS; ++i) {
            asm volatile("" : "+v"(ld_v[i]));
            __builtin_amdgcn_global_load_lds(src + ld_v[i], (lds_void_t *)(dst + (wave * IPS + i) * 512),
                                             16, 0, 0);
        }
    };
    // the first slices start moving before Q is even loaded
    load_k(0, sK0);
    load_k(1, sK1);
    load_k(2, sK2);
    load_k(3, sK3);
    load_v(0, sV0);
    load_v(1, sV1);
    load_v(2, sV2);

    bf16x8_t qf[NG][D / 16];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (rvalid[g]) {
            const __bf16 *src = qp + (((size_t)tl.b * a.S + t[g]) * a.Hq + h[g]) * D + half * 8;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                qf[g][kk] = *reinterpret_cast<const bf16x8_t *>(src + kk * 16);
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[g][kk][e] = (__bf16)0.f;
        }
    }

    // Logits in log2 units: the matrix cores take the raw bf16 q (exact), and
    // the scale log2(e) / sqrt(d) is applied to the fp32 products at the
    // exponent, in both passes.  (Rounding q * scale to bf16 instead would
    // move a logit by up to 2^-9 of |q| |k|: with the bound at 64 that is up
    // to 0.125 log2 units, and keys that tie along different large channels
    // then get visibly wrong relative weights.)  qn2 = |q|^2 in log2 units.
    const float sl2 = a.scale_log2;
    float qn2[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)qf[g][kk][e], (float)qf[g][kk][e], acc);
        qn2[g] = (acc + __shfl_xor(acc, 32, 64)) * (sl2 * sl2);
    }
    // largest squared key norm over the tile's key range
    float kn2;
    {
        const float *km = a.kmax2 + ((size_t)tl.b * a.Hkv + tl.g) * a.n;
        if (MODE == kDense) {
            kn2 = 0.f;
            for (int j = 0; j <= tl.tmax / a.B; ++j) kn2 = fmaxf(kn2, ld_index(km + j));
        } else {
            kn2 = ld_index(km + tl.key_begin / a.B);
        }
    }
    constexpr float kBound2 = 64.f * 64.f;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's part of the first slices is in LDS
    if constexpr (FAST) {
        bool in_bound = true;
#pragma unroll
        for (int g = 0; g < NG; ++g) in_bound = in_bound && qn2[g] * kn2 <= kBound2;
        // Each wave's flag through LDS; the barrier also makes every wave's part
        // of the first slices visible.
        const bool wave_bad = __any(!in_bound);     // over all 64 lanes: outside the branch below
        if (lane == 0) sFlag[wave] = wave_bad;
        lds_barrier();
        int f = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) f |= sFlag[w];
        if (__builtin_amdgcn_readfirstlane(f) != 0) {
            if (tid == 0) a.defer_list[atomicAdd(a.defer_count, 1u)] = tile;
            return;
        }
    } else {
        __syncthreads();
    }

    f32x16_t oacc[NG][D / 32];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[g][dt][i] = 0.f;
    float m_run[NG], l_run[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
    }

    typedef f32x16_t HTile[NG];    // S^T of one slice, per column group
    typedef bf16x8_t KRegs[D / 16];        // K operand of one slice (this lane's part)
    typedef bf16x8_t VRegs[2][D / 32];     // V^T operand of one slice (this lane's part)
    const f32x16_t zero16 = {};
    // K operand of the slice in ktile: lane (row, half) holds 16-byte chunks 2 kk + half of its row
    auto read_k = [&](KRegs &kr, const __bf16 *ktile) {
        const __bf16 *base = ktile + col * D;
        const int sw = swz_k<D>(col);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            kr[kk] = *reinterpret_cast<const bf16x8_t *>(base + (((kk * 2 + half) ^ sw) << 3));
    };
    // S^T = K Q^T of one slice: rows = 32 keys, columns = queries
    auto s_mfma = [&](HTile &sa, const KRegs &kr) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int g = 0; g < NG; ++g)
                sa[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk], qf[g][kk], kk == 0 ? zero16 : sa[g],
                                                                0, 0, 0);
    };
    // mask, then (when tracking the running max) the row max of slice hs.
    // OWN / DENSE: causal mask on the slices that reach past the wave's first
    // row; it also empties the padding slices, whose keys all lie beyond the
    // tile's last row.  PAST: padding slices are emptied whole.
    auto mask_max = [&](HTile &sa, int hs, float (&mx)[NG], auto fast_c) {
        const int kb = tl.key_begin + hs * kS;
        if constexpr (MODE != kPast) {
            if (kb + kS - 1 > wfirst) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + 8 * (i >> 2) + 4 * half + (i & 3);
                        if (key > tq[g]) sa[g][i] = -INFINITY;
                    }
            }
        } else if constexpr (PAD) {
            if (hs >= nh) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sa[g][i] = -INFINITY;
            }
        }
        if constexpr (!decltype(fast_c)::value) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                float m = fmaxf(sa[g][0], sa[g][1]);
#pragma unroll
                for (int i = 2; i < 16; i += 2) m = fmaxf(m, fmaxf(sa[g][i], sa[g][i + 1]));
                mx[g] = fmaxf(m, __shfl_xor(m, 32, 64)) * sl2;
            }
        }
    };
    auto rescale = [&](const float (&mc)[NG]) {
        bool up = false;
#pragma unroll
        for (int g = 0; g < NG; ++g) up = up || mc[g] > m_run[g] + kRescaleSlack;
        if (__any(up)) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float m_new = fmaxf(m_run[g], mc[g]);
                const float alpha =
                    (m_run[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[g] - m_new);
                m_run[g] = m_new;
                l_run[g] *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[g][dt][i] *= alpha;
            }
        }
    };
    // P = 2^(S c - m) (bounded pass: m = 0, one multiply; tracking pass: the
    // scale folded into the FMA) of column group g, in bf16 for the PV product;
    // the row sums add the same bf16 values, two per dot2.
    const bf16x2_t ones2 = {(__bf16)1.f, (__bf16)1.f};
    auto exp_group = [&](const HTile &sa, int g, bf16x8_t (&pbg)[2], auto fast_c) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            float p0, p1;
            if constexpr (decltype(fast_c)::value) {
                p0 = __builtin_amdgcn_exp2f(sa[g][i] * sl2);
                p1 = __builtin_amdgcn_exp2f(sa[g][i + 1] * sl2);
            } else {
                p0 = __builtin_amdgcn_exp2f(fmaf(sa[g][i], sl2, -m_run[g]));
                p1 = __builtin_amdgcn_exp2f(fmaf(sa[g][i + 1], sl2, -m_run[g]));
            }
            bf16x2_t pp;
            pp[0] = (__bf16)p0;
            pp[1] = (__bf16)p1;
            pbg[i >> 3][i & 7] = pp[0];
            pbg[i >> 3][(i & 7) + 1] = pp[1];
            l_run[g] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, l_run[g], false);
        }
    };
    // V^T operand of the PV product for dims dt*32 .. +31 and the 16 keys of key
    // group h2: lane (d, c) needs V[16 h2 + 4 c + e][d] and V[16 h2 + 8 + 4 c + e][d]
    const int tr_g = lane >> 4, tr_j = lane & 15;
    const int tr_row = 4 * (tr_g >> 1) + (tr_j >> 2);           // + 16 h2 (+ 8)
    const int tr_dim = 16 * (tr_g & 1) + 4 * (tr_j & 3);        // + dt*32
    auto read_v = [&](VRegs &vr, const __bf16 *vtile) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int r0 = 16 * h2 + tr_row;
            const int sw = swz_v<D>(r0);                     // rows r0 and r0 + 8 share it
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int d = dt * 32 + tr_dim;
                const __bf16 *pl = vtile + r0 * D + (((d >> 3) ^ sw) << 3) + (d & 7);
                const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4_t *)(pl));
                const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4_t *)(pl + 8 * D));
                vr[h2][dt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };
    // O^T += V^T P^T of one slice, column group g
    auto pv_group = [&](const bf16x8_t (&pbg)[2], const VRegs &vr, int g) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                oacc[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[h2][dt], pbg[h2], oacc[g][dt],
                                                                      0, 0, 0);
    };

    {
        const std::integral_constant<bool, FAST> fast_c;
        if (FAST)
#pragma unroll
            for (int g = 0; g < NG; ++g) m_run[g] = 0.f;
        HTile sa, sb;
        float mxa[NG], mxb[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) mxa[g] = mxb[g] = 0.f;
        KRegs kr;
        read_k(kr, sK0);
        s_mfma(sa, kr);
        mask_max(sa, 0, mxa, fast_c);
        read_k(kr, sK1);
        // Step hs, S(hs) in cur, the K operand of slice hs+1 in kr:
        //   A: S(hs+1) on the matrix cores || P(hs) of column group 0, V(hs)
        //      read from vc
        //   -- barrier --
        //   B: O += V(hs)^T P(hs)^T on the matrix cores || P(hs) of group 1,
        //      K(hs+4) -> kl and V(hs+3) -> vl start moving, the K operand of
        //      slice hs+2 is read from kn, S(hs+1) is masked
        // The barrier sits where every wave's loads of K(hs+2) and V(hs+1) (issued
        // two steps back) have landed and every read of the slots that phase B
        // refills has completed.  The last steps compute S values that nothing
        // uses, from the clamped reloads of the last slices.
        auto step = [&](int hs, HTile &cur, float (&mc)[NG], HTile &nxt, float (&mn)[NG],
                        const __bf16 *vc, const __bf16 *kn, __bf16 *kl, __bf16 *vl) {
            // An opaque zero added to the K slot addresses keeps them inside the
            // loop, where the slot base folds into the LDS instruction's offset,
            // instead of per-slot addresses hoisted into registers.
            int z;
            asm volatile("s_mov_b32 %0, 0" : "=s"(z));
            if constexpr (!FAST) rescale(mc);
            s_mfma(nxt, kr);
            bf16x8_t pb[NG][2];
            exp_group(cur, 0, pb[0], fast_c);
            VRegs vr;
            read_v(vr, vc);
            ring_barrier<2 * IPS>();
            if constexpr (MODE == kPast) read_k(kr, kn);
            else read_k(kr, kn + z);
            load_k(hs + 4, kl);
            load_v(hs + 3, vl);
            pv_group(pb[0], vr, 0);
#pragma unroll
            for (int g = 1; g < NG; ++g) {
                exp_group(cur, g, pb[g], fast_c);
                pv_group(pb[g], vr, g);
            }
            mask_max(nxt, hs + 1, mn, fast_c);
            __builtin_amdgcn_sched_barrier(0);
        };
        // a multiple of 4 steps, so that the loop has one exit, at the bottom
        const int nh4 = (nh + 3) & ~3;
        for (int hs = 0; hs < nh4; hs += 4) {
            step(hs, sa, mxa, sb, mxb, sV0, sK2, sK0, sV3);
            step(hs + 1, sb, mxb, sa, mxa, sV1, sK3, sK1, sV0);
            step(hs + 2, sa, mxa, sb, mxb, sV2, sK0, sK2, sV1);
            step(hs + 3, sb, mxb, sa, mxa, sV3, sK1, sK3, sV2);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the clamped reloads have landed before LDS is reused
    __syncthreads();

    float inv[NG], lse[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float l_tot = l_run[g] + __shfl_xor(l_run[g], 32, 64);
        inv[g] = 1.f / l_tot;
        lse[g] = m_run[g] + __log2f(l_tot);
    }
    // Destination of each row: a partial slot with its log-sum-exp (past
    // blocks; the own block of a row that has past blocks to merge with), or
    // the output row.  The normalised rows (bf16) of column group g pass
    // through ring slot g NW + wave (of sK0..3, sV0..3), chunk-swizzled, so that
    // every global store writes whole 16-byte pieces of contiguous rows.
    constexpr int LPR = D / 8;          // lanes per row (8 elements each)
    constexpr int RPP = 64 / LPR;       // rows per store pass
    // LDS-typed pointers: chosen by a runtime index from an array, plain
    // pointers would become generic (flat) accesses, and a flat load waits on
    // the vector-memory counter, i.e. for the previous row's global store.
    lds_bf16_t *const ring[8] = {(lds_bf16_t *)sK0, (lds_bf16_t *)sK1, (lds_bf16_t *)sK2, (lds_bf16_t *)sK3,
                                 (lds_bf16_t *)sV0, (lds_bf16_t *)sV1, (lds_bf16_t *)sV2, (lds_bf16_t *)sV3};
    lds_bf16_t *stg[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) stg[g] = ring[g * NW + wave];
    // OWN rows with past blocks either go to their partial slot, for the merge
    // kernel, or (fused) are merged here with the past blocks' partial outputs.
    const bool fused = MODE == kOwn && tl.npast > 0 && a.fuse_merge;
    const bool to_part = MODE == kPast || (MODE == kOwn && tl.npast > 0 && !fused);
    long long dst[NG];                  // element offset of the row's destination, -1: padding
    long long prow[NG];                 // fused: the row's chunk-local partial row
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        lds_bf16_t *stage = stg[g];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int ch = (dt * 4 + g4) ^ (col & (CPR - 1));
                *reinterpret_cast<__attribute__((address_space(3))) uint64_t *>(stage + col * D + ch * 8 + 4 * half) =
                    pack4(oacc[g][dt][4 * g4] * inv[g], oacc[g][dt][4 * g4 + 1] * inv[g],
                          oacc[g][dt][4 * g4 + 2] * inv[g], oacc[g][dt][4 * g4 + 3] * inv[g]);
            }
        dst[g] = -1;
        if (rvalid[g]) {
            if (to_part) {
                const int sl = MODE == kPast ? slot[g] : a.nslot - 1;
                const long long id = (((long long)tl.b * a.Hq + h[g]) * a.R + (t[g] - a.r0)) * a.nslot + sl;
                dst[g] = id * D;
                if (half == 0) __builtin_nontemporal_store(lse[g], &a.part_lse[id]);
            } else {
                dst[g] = (((long long)tl.b * a.S + t[g]) * a.Hq + h[g]) * D;
                if (a.lse_out && half == 0 && !fused)
                    a.lse_out[((long long)tl.b * a.Hq + h[g]) * a.S + t[g]] = lse[g] * kLn2;
            }
        }
        prow[g] = (((long long)tl.b * a.Hq + h[g]) * a.R + (t[g] - a.r0));
    }
    // Each wave stores (or merges) only the rows it staged: its own LDS writes
    // precede its reads in order, so no barrier is needed here, and its loads
    // and stores start at once.  Outputs and partial outputs are stored
    // non-temporally: they are not read again by this launch, and kept out of
    // L2 they leave it to the K / V slices the XCD's other tiles are streaming
    // (at 1M, 44 GB fewer re-reads of K / V per launch).
    if constexpr (MODE == kOwn) {
        if (fused) {
            merge_rows<D, NG>(a, tl, stg, dst, prow, lse);
            return;
        }
    }
    __bf16 *base = static_cast<__bf16 *>(to_part ? a.part_o : a.out);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const lds_bf16_t *stage = stg[g];
#pragma unroll
        for (int it = 0; it < 32 / RPP; ++it) {
            const int rr = it * RPP + lane / LPR, ch = lane % LPR;
            const long long o = __shfl(dst[g], rr, 64);       // lane rr holds row rr
            if (o >= 0) {
                const bf16x8_t v = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
                    stage + rr * D + ((ch ^ (rr & (CPR - 1))) << 3));
                __builtin_nontemporal_store(v, reinterpret_cast<bf16x8_t *>(base + o + ch * 8));
            }
        }
    }
}

// The ring slots are separate LDS arrays so the compiler can prove that the
// reads of one slot never alias the direct loads into another, and does not
// wait for those loads before reading.
#define MOBA_RING_ARRAYS(D)                                         \
    __shared__ __attribute__((aligned(16))) __bf16 sK0[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sK1[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sK2[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sK3[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sV0[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sV1[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sV2[kS * (D)];   \
    __shared__ __attribute__((aligned(16))) __bf16 sV3[kS * (D)];   \
    __shared__ int sFlag[8];

template <int D, int MODE, bool PAD>
__global__ __launch_bounds__((64 * attn_waves<D, MODE>()), (attn_occupancy<D, MODE>())) void attn_bf16_kernel(
    AttnArgs a) {
    MOBA_RING_ARRAYS(D)
    attn_bf16_tile<D, MODE, true, PAD, attn_waves<D, MODE>()>(a, first_tile(a, MODE), sK0, sK1, sK2, sK3, sV0,
                                                             sV1, sV2, sV3, sFlag);
}

// Tracking pass: a persistent grid walks the deferred tiles (normally none).
template <int D, int MODE, bool PAD>
__global__ __launch_bounds__((64 * attn_waves<D, MODE>()), (attn_occupancy<D, MODE>())) void attn_bf16_track_kernel(
    AttnArgs a) {
    MOBA_RING_ARRAYS(D)
    const unsigned n = *a.defer_count;
    for (unsigned i = wg_x(); i < n; i += a.nwg) {
        attn_bf16_tile<D, MODE, false, PAD, attn_waves<D, MODE>()>(a, a.defer_list[i], sK0, sK1, sK2, sK3, sV0,
                                                                  sV1, sV2, sV3, sFlag);
        __syncthreads();
    }
}

__global__ void zero_count_kernel(unsigned *c) { *c = 0u; }

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
    if (!decode_tile(a, MODE, first_tile(a, MODE), tl)) return;
    constexpr int DH = D / 2;
    const int r = tid_x() >> 1, dh = tid_x() & 1;
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
        for (int e = tid_x(); e < kNF * D / 4; e += 256) {
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
    const long long row_id = ((long long)tl.b * a.Hq + h) * a.R + (t - a.r0);   // chunk-local
    // a partial slot (past blocks; the own block of a row with past blocks) or the output row
    if (MODE == kPast || (MODE == kOwn && tl.npast > 0)) {
        const int sl = MODE == kPast ? slot : a.nslot - 1;
        float *dst = static_cast<float *>(a.part_o) + (row_id * a.nslot + sl) * D + dh * DH;
#pragma unroll
        for (int i = 0; i < DH; ++i) dst[i] = o[i] * inv;
        if (dh == 0) a.part_lse[row_id * a.nslot + sl] = lse;
        return;
    }
    float *dst = static_cast<float *>(a.out) + (((size_t)tl.b * a.S + t) * a.Hq + h) * D + dh * DH;
#pragma unroll
    for (int i = 0; i < DH; ++i) dst[i] = o[i] * inv;
    if (a.lse_out && dh == 0) a.lse_out[((long long)tl.b * a.Hq + h) * a.S + t] = lse * kLn2;
}

// ------------------------------------------------------------------ launchers

static AttnArgs make_args(const AttnBuffers &bf, const Problem &p) {
    AttnArgs a;
    a.q = bf.q; a.k = bf.k; a.v = bf.v; a.out = bf.out;
    a.part_o = bf.part_o; a.part_lse = bf.part_lse;
    a.lists = bf.lists; a.list_off = bf.list_off; a.tile_off = bf.tile_off;
    a.tile_list = bf.tile_list;
    a.kmax2 = bf.kmax2;
    a.defer_count = bf.defer_count;
    a.defer_list = bf.defer_list;
    a.lse_out = bf.lse_out;
    a.fuse_merge = 0;
    a.batch = p.batch; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.B = p.B; a.n = p.n;
    a.r0 = p.r0; a.R = p.R;
    a.topk = p.topk;
    a.nslot = part_slots(p);
    a.L = (long long)p.batch * p.Hkv * p.n;
    a.ntiles = 0;
    a.nwg = 0;
    a.M = tile_rows(p);
    a.dense_heads = 1;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.D));
    return a;
}

static unsigned round8(unsigned long long x) { return (unsigned)((x + 7) / 8 * 8); }

constexpr unsigned kTrackGrid = 256;

// the bounded pass, then the tracking pass over the tiles it deferred
template <int D, int MODE, bool PAD>
static void bf16_pair(AttnArgs a, unsigned grid, hipStream_t st) {
    a.nwg = grid;
    attn_bf16_kernel<D, MODE, PAD><<<grid, 64 * attn_waves<D, MODE>(), 0, st>>>(a);
    a.nwg = kTrackGrid;
    attn_bf16_track_kernel<D, MODE, PAD><<<kTrackGrid, 64 * attn_waves<D, MODE>(), 0, st>>>(a);
}

template <int MODE>
static hipError_t attn_launch(AttnArgs a, const Problem &p, unsigned grid, hipStream_t st) {
    if (grid == 0) return hipSuccess;
    if (p.dtype == kBF16) {
        zero_count_kernel<<<1, 1, 0, st>>>(a.defer_count);
        // PAST tiles visit B / 32 slices; the loop runs a multiple of 4
        bool pad = false;
        if constexpr (MODE == kPast) pad = p.B % 128 != 0;
        if (pad) {
            if constexpr (MODE == kPast) {
                if (p.D == 64) bf16_pair<64, MODE, true>(a, grid, st);
                else bf16_pair<128, MODE, true>(a, grid, st);
            }
        } else {
            if (p.D == 64) bf16_pair<64, MODE, false>(a, grid, st);
            else bf16_pair<128, MODE, false>(a, grid, st);
        }
    } else {
        a.nwg = grid;
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
    a.M = own_tile_rows(p);
    a.ntiles = (unsigned)own_tiles(p);
    a.fuse_merge = merge_in_own_pass(p) ? 1 : 0;
    return attn_launch<kOwn>(a, p, round8(a.ntiles), st);
}

hipError_t launch_attn_dense(const AttnBuffers &bf, const Problem &p, hipStream_t st) {
    AttnArgs a = make_args(bf, p);
    a.dense_heads = dense_heads(p);
    a.ntiles = (unsigned)dense_tiles(p);
    return attn_launch<kDense>(a, p, round8(a.ntiles), st);
}

}  // namespace moba
