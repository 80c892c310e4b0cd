// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Largest number of past blocks the gate keeps per row.
constexpr int kMaxPast = 31;
// Block-count limit for the LDS histograms of the index build.
constexpr int kHistMax = 4096;
// ln 2: base-2 log-sum-exps (the kernels' units) to natural logs.
constexpr float kLn2 = 0.693147180559945309f;

enum DType { kBF16 = 0, kF32 = 1 };

// Packed row record of the per-(KV head, block) lists: token | head-in-group | slot.
__host__ __device__ inline uint64_t pack_row(uint32_t t, uint32_t hh, uint32_t slot) {
    return (uint64_t)t | ((uint64_t)hh << 32) | ((uint64_t)slot << 48);
}
__host__ __device__ inline uint32_t row_t(uint64_t r) { return (uint32_t)(r & 0xffffffffu); }
__host__ __device__ inline uint32_t row_hh(uint64_t r) { return (uint32_t)((r >> 32) & 0xffffu); }
__host__ __device__ inline uint32_t row_slot(uint64_t r) { return (uint32_t)(r >> 48); }

struct Problem {
    int batch, S, Hq, Hkv, D, B, topk, dtype;
    int G;       // Hq / Hkv
    int n;       // ceil(S / B): the last block may be short (S % B tokens)
    int npast;   // topk - 1 capped at n - 1
    bool dense;  // topk >= n: plain causal attention
    // query rows handled by one pass of the sparse stages: tokens [r0, r0 + R),
    // both multiples of B (r0 = 0, R = S unless the prefill runs in chunks).
    // Row-indexed scratch (block indices, lists, partial outputs) is chunk-local.
    int r0, R;
};

// Map a workgroup index to a tile so that consecutive tiles run on the same
// XCD (workgroups are dispatched to the 8 XCDs round-robin).  nb % 8 == 0.
__device__ inline uint32_t xcd_tile(uint32_t bid, uint32_t nb) {
    return (bid & 7u) * (nb >> 3) + (bid >> 3);
}

// The same for a grid that only bounds the tile count from above (past-block
// tiles, counted on the device): XCD x takes the x-th eighth of the ntl real
// tiles, so every XCD gets an equal share however loose the bound.  Workgroups
// past their XCD's share get ntl: no tile.  Needs gridDim.x >= 8 ceil(ntl / 8).
__device__ inline uint32_t xcd_tile_counted(uint32_t bid, uint32_t ntl) {
    const uint32_t c = (ntl + 7u) >> 3, i = bid >> 3;
    if (i >= c) return ntl;
    const uint32_t t = (bid & 7u) * c + i;
    return t < ntl ? t : ntl;
}

// ---- launchers (each returns the launch status) ----
struct PoolBuffers {
    float *kbar;           // [batch][Hkv][n][D] block means
    float *kmax2;          // [batch][Hkv][n] largest squared key norm of each block
    __bf16 *khl;           // [batch][Hkv][n][2][D] bf16 split of the means: hi = rne(x), lo = rne(x - hi)
};
hipError_t launch_pool(const void *k, const PoolBuffers &pb, const Problem &p, hipStream_t st);
hipError_t launch_gate(const void *q, const float *kbar, const __bf16 *khl, int32_t *idx,
                       const Problem &p, hipStream_t st);
hipError_t launch_gate_scores(const void *q, const __bf16 *khl, float *scores, const Problem &p,
                              hipStream_t st);
hipError_t launch_index(const int32_t *idx, uint32_t *cnt, uint32_t *cursor, uint64_t *list_off,
                        uint32_t *tile_off, uint32_t *tile_list, uint64_t tiles_upper,
                        uint64_t *lists, const Problem &p, hipStream_t st);

struct AttnBuffers {
    const void *q, *k, *v;
    void *out;
    void *part_o;           // [row][slots][D], dtype-sized elements
    float *part_lse;        // [row][slots], base-2 log-sum-exp of the scaled logits
    const uint64_t *lists;
    const uint64_t *list_off;
    const uint32_t *tile_off;
    const uint32_t *tile_list;  // [past tiles] list index of each past-block tile
    const float *kmax2;     // [batch][Hkv][n] largest squared key norm per block
    unsigned *defer_count;  // deferred-tile list (tiles that need running-max tracking)
    unsigned *defer_list;
    float *lse_out;         // optional [batch][Hq][S]: natural-log log-sum-exp of each row
};
hipError_t launch_attn_past(const AttnBuffers &b, const Problem &p, uint64_t tiles_upper,
                            hipStream_t st);
hipError_t launch_attn_own(const AttnBuffers &b, const Problem &p, hipStream_t st);
hipError_t launch_attn_dense(const AttnBuffers &b, const Problem &p, hipStream_t st);
hipError_t launch_merge(const AttnBuffers &b, const Problem &p, hipStream_t st);

// Backward pass (bf16): the forward's selection is rebuilt (pool, gate, index),
// then dq through partial slots per (row, block) and dk / dv per key.
struct BwdBuffers {
    const void *q, *k, *v, *out, *dout;
    const float *lse;       // [batch][Hq][S] natural-log log-sum-exp from the forward
    void *dq, *dk, *dv;
    float *l2, *delta;      // [batch][Hq][S] scratch: lse in base 2, dO . O
    void *part_dq;          // [batch][Hq][S][slots][D] bf16 scratch
    const uint64_t *lists;
    const uint64_t *list_off;
    const uint32_t *tile_off;
    const uint32_t *tile_list;
};
hipError_t launch_backward(const BwdBuffers &bb, const Problem &p, uint64_t tiles_upper,
                           hipStream_t st);

// Query rows per attention tile: 256 on the bf16 matrix-core path (8 waves x 32
// rows for d = 128, 4 x 64 for d = 64), 128 on the fp32 path (two threads a row).
inline int tile_rows(const Problem &p) { return p.dtype == kBF16 ? 256 : 128; }

// Own-block tiles of the bf16 d = 128 path hold 128 rows (4 waves): two such
// workgroups share a CU, so one's merge epilogue (bound by HBM) runs beside
// the other's key loop (bound by the matrix cores).
inline int own_tile_rows(const Problem &p) {
    return (p.dtype == kBF16 && p.D == 128) ? 128 : tile_rows(p);
}

// Tiles of each attention launch (the past-block count is an upper bound).
inline unsigned long long own_tiles(const Problem &p) {
    return (unsigned long long)p.batch * p.Hkv * ((p.R + p.B - 1) / p.B) * p.G *
           ((p.B + own_tile_rows(p) - 1) / own_tile_rows(p));
}
// Query heads per full-attention tile: the bf16 path puts 256 / Gd tokens of
// Gd heads of one KV group in a tile, so the key prefix a tile streams serves
// Gd heads at once; Gd is the largest of 8, 4, 2 that divides the group and
// keeps every wave's rows inside one head (1 on the fp32 path).
inline int dense_heads(const Problem &p) {
    if (p.dtype != kBF16) return 1;
    const int rpw = p.D == 128 ? 32 : 64;   // rows per wave
    for (int gd = 8; gd >= 2; gd /= 2)
        if (p.G % gd == 0 && (tile_rows(p) / gd) % rpw == 0) return gd;
    return 1;
}
inline unsigned long long dense_tiles(const Problem &p) {
    const int gd = dense_heads(p), tt = tile_rows(p) / gd;
    return (unsigned long long)p.batch * (p.Hq / gd) * ((p.S + tt - 1) / tt);
}

// Partial-output slots per query row: one per selectable past block, then
// one for the own block (slot topk - 1), which is written only when the row
// has past blocks to merge with.
inline int part_slots(const Problem &p) { return p.topk; }
// The bf16 own-block pass merges its rows with their past blocks' partial
// outputs itself (no merge kernel) when a row has at most kFuseMaxPast.
constexpr int kFuseMaxPast = 12;
inline bool merge_in_own_pass(const Problem &p) { return p.dtype == kBF16 && p.npast <= kFuseMaxPast; }
// Backward dq slots per row: past blocks, then the own block (slot - 1).
inline int bwd_slots(const Problem &p) { return p.topk < p.n ? p.topk : p.n; }


}  // namespace moba
