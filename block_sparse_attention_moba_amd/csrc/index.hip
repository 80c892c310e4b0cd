// Index build: turn each row's selected past blocks into per-(batch, KV head,
// past block) lists of query rows.  This is the dispatch half of the pages'
// recipe (write-up "MoBA: Mixture of Block Attention", implementation steps
// two and three: arrange queries by their assigned KV block so each block's
// attention runs over its own queries), done without moving Q: a list holds
// packed (token, head-in-group, slot) records and the attention kernel
// gathers the query rows it names.
//
//   count   : per-workgroup LDS histogram of the selected past blocks (a
//             workgroup: 256 tokens of the G query heads of a KV group), then
//             one global atomic per (workgroup, block).
//   scan    : one workgroup; exclusive scan of the list lengths (row offsets)
//             and of their tile counts (tile offsets); clears the cursors.
//   tile map: the list index of every attention tile (a binary search over
//             the tile offsets, once per tile), so the attention kernel finds
//             its list with one load instead of a chain of dependent ones.
//   scatter : the same histogram again, one global atomic per (workgroup,
//             block) reserves a range of the list, and a second walk over the
//             selections places each record in it (an LDS atomic per record).
// The order of records inside a list depends on scheduling; no result does,
// because every row's attention is computed independently of its neighbours.
#include "moba_internal.hpp"

namespace moba {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Tokens per workgroup of the count and scatter kernels.
constexpr int kIdxRows = 256;

// The selections of a workgroup's rows are read, per query head, as one
// contiguous span of the block-index array (a head's rows are consecutive,
// topk entries each), 16 bytes per lane.  The buffer is 256-byte aligned, a
// head's rows start at a multiple of R rows (R a multiple of 64), the span at
// a multiple of kIdxRows rows after that, and it holds a multiple of 64 rows,
// so every 16-byte piece is aligned and whole.  Entry e of the span is slot
// e mod topk of row e / topk; the quotient comes from a multiply by
// ceil(2^32 / topk), exact for e * topk < 2^32 (here e < kIdxRows * topk and
// topk <= 32; topk 1 has no past slot and is never launched, but its
// quotient is e itself).
__device__ inline uint32_t div_magic(int topk) {
    return (uint32_t)((0x100000000ull + (unsigned)topk - 1) / (unsigned)topk);
}
__device__ inline int span_row(int e, uint32_t mt, int topk) {
    return topk == 1 ? e : (int)__umulhi((uint32_t)e, mt);
}

// Query rows of the chunk [r0, r0 + R); idx rows are chunk-local.  A
// workgroup takes kIdxRows tokens of every query head of one KV group, the heads
// whose selections feed the same lists, so that one global atomic per
// (workgroup, block) covers G heads.
// grid (ceil(R / kIdxRows), Hkv, batch), 256 threads.
__global__ __launch_bounds__(256) void count_kernel(const int32_t *__restrict__ idx,
                                                    uint32_t *__restrict__ cnt, int r0, int R,
                                                    int Hq, int Hkv, int G, int B, int n,
                                                    int topk) {
    __shared__ uint32_t hist[kHistMax];
    __shared__ int sown[kIdxRows];
    const int g = blockIdx.y, b = blockIdx.z;
    const int tb = r0 + blockIdx.x * kIdxRows, nrow = min(kIdxRows, r0 + R - tb);
    const int jend = (tb + nrow - 1) / B;          // the last row's own block
    const bool use_lds = n <= kHistMax;
    uint32_t *gcnt = cnt + ((size_t)b * Hkv + g) * n;
    for (int r = threadIdx.x; r < nrow; r += 256) sown[r] = (tb + r) / B;
    if (use_lds)
        for (int j = threadIdx.x; j < jend; j += 256) hist[j] = 0u;
    __syncthreads();
    const uint32_t mt = div_magic(topk);
    const int nq = nrow * topk / 4;
    for (int hh = 0; hh < G; ++hh) {
        const int4 *span = reinterpret_cast<const int4 *>(
            idx + (((size_t)b * Hq + g * G + hh) * R + (tb - r0)) * topk);
        for (int q = threadIdx.x; q < nq; q += 256) {
            const int4 v = span[q];
            const int jj[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 4 * q + u, r = span_row(e, mt, topk), c = e - r * topk;
                const int own = sown[r], j = jj[u];
                // past slots only; an index at or past the own block is never produced by the gate
                if (c < min(topk - 1, own) && (unsigned)j < (unsigned)own) {
                    if (use_lds) atomicAdd(&hist[j], 1u);
                    else atomicAdd(&gcnt[j], 1u);
                }
            }
        }
    }
    if (use_lds) {
        __syncthreads();
        for (int j = threadIdx.x; j < jend; j += 256)
            if (hist[j]) atomicAdd(&gcnt[j], hist[j]);
    }
}

// One workgroup of 1024 threads.  list_off[L+1] (rows), tile_off[L+1] (tiles of M rows).
__global__ __launch_bounds__(1024) void scan_kernel(const uint32_t *__restrict__ cnt,
                                                    uint32_t *__restrict__ cursor,
                                                    uint64_t *__restrict__ list_off,
                                                    uint32_t *__restrict__ tile_off, long long L,
                                                    int M) {
    __shared__ uint64_t wrow[16];
    __shared__ uint32_t wtile[16];
    __shared__ uint64_t carry_row;
    __shared__ uint32_t carry_tile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry_row = 0;
        carry_tile = 0;
    }
    __syncthreads();
    for (long long base = 0; base < L; base += 1024) {
        const long long i = base + tid;
        const uint32_t c = (i < L) ? cnt[i] : 0u;
        uint64_t r = c;
        uint32_t tl = (c + M - 1) / M;
        // inclusive scan inside the wave
        for (int off = 1; off < 64; off <<= 1) {
            const uint64_t ro = __shfl_up(r, off, 64);
            const uint32_t to = __shfl_up(tl, off, 64);
            if (lane >= off) {
                r += ro;
                tl += to;
            }
        }
        if (lane == 63) {
            wrow[wave] = r;
            wtile[wave] = tl;
        }
        __syncthreads();
        uint64_t pre_r = carry_row;
        uint32_t pre_t = carry_tile;
        for (int w = 0; w < wave; ++w) {
            pre_r += wrow[w];
            pre_t += wtile[w];
        }
        if (i < L) {
            list_off[i] = pre_r + r - c;
            tile_off[i] = pre_t + tl - (c + M - 1) / M;
            cursor[i] = 0u;
        }
        __syncthreads();
        if (tid == 1023) {
            carry_row = pre_r + r;
            carry_tile = pre_t + tl;
        }
        __syncthreads();
    }
    if (tid == 0) {
        list_off[L] = carry_row;
        tile_off[L] = carry_tile;
    }
}

// grid ceil(tiles_upper / 256), 256 threads: tile_list[t] = the list whose tile range holds t.
__global__ __launch_bounds__(256) void tile_map_kernel(const uint32_t *__restrict__ tile_off,
                                                       uint32_t *__restrict__ tile_list, long long L,
                                                       unsigned long long tiles_upper) {
    const unsigned long long t = (unsigned long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= tiles_upper || t >= tile_off[L]) return;
    long long lo = 0, hi = L;
    while (hi - lo > 1) {
        const long long mid = (lo + hi) >> 1;
        if (tile_off[mid] <= t) lo = mid;
        else hi = mid;
    }
    tile_list[t] = (uint32_t)lo;
}

// grid (ceil(R / kIdxRows), Hkv, batch), 256 threads; the rows of count_kernel.
// With the LDS histogram: (1) count the workgroup's selections per block,
// (2) reserve each block's range of its list with one global atomic and keep
// the range's start (the list's offset included) in LDS, (3) walk the
// selections again, a 64-bit LDS atomic on that start giving each record its
// address in the list array.
// Beyond kHistMax blocks every selection reserves its own place globally.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t *__restrict__ idx,
                                                      uint32_t *__restrict__ cursor,
                                                      const uint64_t *__restrict__ list_off,
                                                      uint64_t *__restrict__ lists, int r0, int R,
                                                      int Hq, int Hkv, int G, int B, int n,
                                                      int topk) {
    __shared__ uint32_t hist[kHistMax];
    __shared__ unsigned long long dst[kHistMax];
    __shared__ int sown[kIdxRows];
    const int g = blockIdx.y, b = blockIdx.z;
    const int tb = r0 + blockIdx.x * kIdxRows, nrow = min(kIdxRows, r0 + R - tb);
    const int jend = (tb + nrow - 1) / B;
    const bool use_lds = n <= kHistMax;
    const size_t lbase = ((size_t)b * Hkv + g) * n;
    for (int r = threadIdx.x; r < nrow; r += 256) sown[r] = (tb + r) / B;
    if (use_lds)
        for (int j = threadIdx.x; j < jend; j += 256) hist[j] = 0u;
    __syncthreads();
    const uint32_t mt = div_magic(topk);
    const int nq = nrow * topk / 4;
    // walk every past selection of the workgroup's rows: f(j, token, head in group, slot)
    auto walk = [&](auto &&f) {
        for (int hh = 0; hh < G; ++hh) {
            const int4 *span = reinterpret_cast<const int4 *>(
                idx + (((size_t)b * Hq + g * G + hh) * R + (tb - r0)) * topk);
            for (int q = threadIdx.x; q < nq; q += 256) {
                const int4 v = span[q];
                const int jj[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = 4 * q + u, r = span_row(e, mt, topk), c = e - r * topk;
                    const int own = sown[r], j = jj[u];
                    if (c < min(topk - 1, own) && (unsigned)j < (unsigned)own) f(j, tb + r, hh, c);
                }
            }
        }
    };
    if (!use_lds) {
        walk([&](int j, int t, int hh, int c) {
            const uint32_t rank = atomicAdd(&cursor[lbase + j], 1u);
            lists[list_off[lbase + j] + rank] = pack_row((uint32_t)t, (uint32_t)hh, (uint32_t)c);
        });
        return;
    }
    walk([&](int j, int, int, int) { atomicAdd(&hist[j], 1u); });
    __syncthreads();
    for (int j = threadIdx.x; j < jend; j += 256)
        if (hist[j]) dst[j] = list_off[lbase + j] + atomicAdd(&cursor[lbase + j], hist[j]);
    __syncthreads();
    walk([&](int j, int t, int hh, int c) {
        const unsigned long long pos = atomicAdd(&dst[j], 1ull);
        lists[pos] = pack_row((uint32_t)t, (uint32_t)hh, (uint32_t)c);
    });
}

hipError_t launch_index(const int32_t *idx, uint32_t *cnt, uint32_t *cursor, uint64_t *list_off,
                        uint32_t *tile_off, uint32_t *tile_list, uint64_t tiles_upper,
                        uint64_t *lists, const Problem &p, hipStream_t st) {
    const long long L = (long long)p.batch * p.Hkv * p.n;
    fill_u32_kernel<<<(unsigned)((L + 255) / 256), 256, 0, st>>>(cnt, L);
    dim3 grid((p.R + kIdxRows - 1) / kIdxRows, p.Hkv, p.batch);
    count_kernel<<<grid, 256, 0, st>>>(idx, cnt, p.r0, p.R, p.Hq, p.Hkv, p.G, p.B, p.n, p.topk);
    scan_kernel<<<1, 1024, 0, st>>>(cnt, cursor, list_off, tile_off, L, tile_rows(p));
    if (tiles_upper > 0)
        tile_map_kernel<<<(unsigned)((tiles_upper + 255) / 256), 256, 0, st>>>(tile_off, tile_list, L,
                                                                              tiles_upper);
    scatter_kernel<<<grid, 256, 0, st>>>(idx, cursor, list_off, lists, p.r0, p.R, p.Hq, p.Hkv,
                                         p.G, p.B, p.n, p.topk);
    return hipGetLastError();
}

}  // namespace moba
