// Index build: turn each row's selected past blocks into per-(batch, KV head,
// past block) lists of query rows.  This is the dispatch half of the pages'
// recipe (write-up "MoBA: Mixture of Block Attention", implementation steps
// two and three: arrange queries by their assigned KV block so each block's
// attention runs over its own queries), done without moving Q: a list holds
// packed (token, head-in-group, slot) records and the attention kernel
// gathers the query rows it names.
//
//   count   : per-workgroup LDS histogram of the selected past blocks, then
//             one global atomic per (workgroup, block).
//   scan    : one workgroup; exclusive scan of the list lengths (row offsets)
//             and of their tile counts (tile offsets); clears the cursors.
//   tile map: the list index of every attention tile (a binary search over
//             the tile offsets, once per tile), so the attention kernel finds
//             its list with one load instead of a chain of dependent ones.
//   scatter : LDS atomics give each selection a rank inside its workgroup,
//             one global atomic per (workgroup, block) reserves a range, and
//             each record is written to its slot of the list.
// The order of records inside a list depends on scheduling; no result does,
// because every row's attention is computed independently of its neighbours.
#include "moba_internal.hpp"

namespace moba {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Query rows of the chunk [r0, r0 + R); idx rows are chunk-local.
// grid (ceil(R / 256), Hq, batch), 256 threads.
__global__ __launch_bounds__(256) void count_kernel(const int32_t *__restrict__ idx,
                                                    uint32_t *__restrict__ cnt, int r0, int R,
                                                    int Hq, int Hkv, int G, int B, int n,
                                                    int topk) {
    __shared__ uint32_t hist[kHistMax];
    const int h = blockIdx.y, b = blockIdx.z, g = h / G;
    const int t = r0 + blockIdx.x * 256 + threadIdx.x;
    const int jend = min(r0 + (int)blockIdx.x * 256 + 255, r0 + R - 1) / B;
    const bool use_lds = n <= kHistMax;
    uint32_t *gcnt = cnt + ((size_t)b * Hkv + g) * n;
    if (use_lds) {
        for (int j = threadIdx.x; j < jend; j += 256) hist[j] = 0u;
        __syncthreads();
    }
    if (t < r0 + R) {
        const int own = t / B;
        const int np = min(topk - 1, own);
        const int32_t *row = idx + (((size_t)b * Hq + h) * R + (t - r0)) * topk;
        for (int c = 0; c < np; ++c) {
            const int j = row[c];
            if ((unsigned)j >= (unsigned)own) continue;   // never produced by the gate
            if (use_lds) atomicAdd(&hist[j], 1u);
            else atomicAdd(&gcnt[j], 1u);
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

// grid (ceil(R / 256), Hq, batch), 256 threads.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t *__restrict__ idx,
                                                      uint32_t *__restrict__ cursor,
                                                      const uint64_t *__restrict__ list_off,
                                                      uint64_t *__restrict__ lists, int r0, int R,
                                                      int Hq, int Hkv, int G, int B, int n,
                                                      int topk) {
    __shared__ uint32_t hist[kHistMax];
    __shared__ uint32_t base[kHistMax];
    const int h = blockIdx.y, b = blockIdx.z, g = h / G, hh = h % G;
    const int t = r0 + blockIdx.x * 256 + threadIdx.x;
    const bool in = t < r0 + R;
    const int jend = min(r0 + (int)blockIdx.x * 256 + 255, r0 + R - 1) / B;
    const bool use_lds = n <= kHistMax;
    const size_t lbase = ((size_t)b * Hkv + g) * n;
    if (use_lds) {
        for (int j = threadIdx.x; j < jend; j += 256) hist[j] = 0u;
        __syncthreads();
    }
    const int own = in ? t / B : 0;
    const int np = in ? min(topk - 1, own) : 0;
    const int32_t *row = idx + (((size_t)b * Hq + h) * R + (in ? t - r0 : 0)) * topk;
    uint32_t rank[kMaxPast];
#pragma unroll
    for (int c = 0; c < kMaxPast; ++c) {
        rank[c] = 0u;
        if (c < np) {
            const int j = row[c];
            if ((unsigned)j >= (unsigned)own) continue;
            rank[c] = use_lds ? atomicAdd(&hist[j], 1u) : atomicAdd(&cursor[lbase + j], 1u);
        }
    }
    if (use_lds) {
        __syncthreads();
        for (int j = threadIdx.x; j < jend; j += 256)
            if (hist[j]) base[j] = atomicAdd(&cursor[lbase + j], hist[j]);
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < kMaxPast; ++c) {
        if (c < np) {
            const int j = row[c];
            if ((unsigned)j >= (unsigned)own) continue;
            const uint64_t pos = list_off[lbase + j] + (use_lds ? base[j] : 0u) + rank[c];
            lists[pos] = pack_row((uint32_t)t, (uint32_t)hh, (uint32_t)c);
        }
    }
}

hipError_t launch_index(const int32_t *idx, uint32_t *cnt, uint32_t *cursor, uint64_t *list_off,
                        uint32_t *tile_off, uint32_t *tile_list, uint64_t tiles_upper,
                        uint64_t *lists, const Problem &p, hipStream_t st) {
    const long long L = (long long)p.batch * p.Hkv * p.n;
    fill_u32_kernel<<<(unsigned)((L + 255) / 256), 256, 0, st>>>(cnt, L);
    dim3 grid((p.R + 255) / 256, p.Hq, p.batch);
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
