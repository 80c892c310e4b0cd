// Block means of the keys (the "aggregated representation of the block keys"
// the gate compares each query with; Taiwan AI overview of MoBA, section
// "技術細節與優勢").
//
// One launch, one workgroup of 1024 threads per (block, KV head, batch): it
// streams the block's B x D keys with 16-byte loads (one D-row per D/8 lanes,
// eight loads in flight per thread), adds them up in a fixed order (per
// thread, then across the rows of a pass through LDS), divides by the tokens
// present (B, or S mod B for a short last block), and writes the mean in fp32
// and as a bf16 hi + lo pair (the operands of the matrix-core gate), with the
// block's largest squared key norm (the attention kernels bound every logit of
// the block by it).  No atomics, so the result is bitwise reproducible.
#include <type_traits>

#include "moba_internal.hpp"

namespace moba {

__device__ inline void load8(const __bf16 *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

__device__ inline void load8(const float *p, float *f) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Sum over each aligned group of N lanes (N = 8 or 16), the result in every
// lane of the group, by DPP moves instead of LDS permutes: swap neighbours,
// swap pairs, mirror within 8 lanes, mirror within 16 lanes.
template <int N>
__device__ inline float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value,
                                                       0xF, 0xF, false));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
    x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    if constexpr (N == 16) x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
    return x;
}

constexpr int kPoolThreads = 1024;
constexpr int kPoolUnroll = 8;

// grid (n * Hkv, batch), 1024 threads.
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const T *__restrict__ k,
                                                            float *__restrict__ kbar,
                                                            float *__restrict__ kmax2,
                                                            __bf16 *__restrict__ khl, int S,
                                                            int Hkv, int B, int n) {
    constexpr int LPT = D / 8;                  // lanes per token row
    constexpr int TPP = kPoolThreads / LPT;     // token rows per pass
    __shared__ float red[TPP][D + 1];
    __shared__ float redn[TPP];
    const int j = blockIdx.x / Hkv;
    const int g = blockIdx.x % Hkv;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int vec = tid % LPT;
    const int tr = tid / LPT;
    const int t0 = j * B;
    const int t1 = min(t0 + B, S);              // a short last block ends at S
    const size_t rstride = (size_t)Hkv * D;
    const T *base = k + ((size_t)b * S * Hkv + g) * D + vec * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float nmax = 0.f;
    for (int t = t0 + tr; t < t1; t += TPP * kPoolUnroll) {
        // all loads issued before any is used: rows past the block end read its
        // last row (in bounds) and are zeroed afterwards, so no load sits in a branch
        float f[kPoolUnroll][8];
#pragma unroll
        for (int u = 0; u < kPoolUnroll; ++u)
            load8(base + (size_t)min(t + u * TPP, t1 - 1) * rstride, f[u]);
#pragma unroll
        for (int u = 0; u < kPoolUnroll; ++u)
            if (t + u * TPP >= t1)
#pragma unroll
                for (int e = 0; e < 8; ++e) f[u][e] = 0.f;
#pragma unroll
        for (int u = 0; u < kPoolUnroll; ++u) {
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[e] += f[u][e];
                sq = fmaf(f[u][e], f[u][e], sq);
            }
            // squared norm of the token: sum over the LPT lanes that hold its row
            nmax = fmaxf(nmax, group_sum<LPT>(sq));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr][vec * 8 + e] = acc[e];
    if (vec == 0) redn[tr] = nmax;
    __syncthreads();
    const size_t blk = ((size_t)b * Hkv + g) * n + j;
    if (tid < D) {
        float sum = 0.f;
        for (int r = 0; r < TPP; ++r) sum += red[r][tid];
        const float m = sum / (float)(t1 - t0);
        kbar[blk * D + tid] = m;
        // bf16 split for the matrix-core gate: m = hi + lo + O(2^-17 |m|)
        const __bf16 hi = (__bf16)m;
        khl[(blk * 2) * D + tid] = hi;
        khl[(blk * 2 + 1) * D + tid] = (__bf16)(m - (float)hi);
    } else if (tid == D) {
        float mx = 0.f;
        for (int r = 0; r < TPP; ++r) mx = fmaxf(mx, redn[r]);
        kmax2[blk] = mx;
    }
}

template <typename T, int D>
static hipError_t pool_impl(const void *k, const PoolBuffers &pb, const Problem &p,
                            hipStream_t st) {
    dim3 grid(p.n * p.Hkv, p.batch);
    pool_kernel<T, D><<<grid, kPoolThreads, 0, st>>>(static_cast<const T *>(k), pb.kbar, pb.kmax2,
                                                     pb.khl, p.S, p.Hkv, p.B, p.n);
    return hipGetLastError();
}

hipError_t launch_pool(const void *k, const PoolBuffers &pb, const Problem &p, hipStream_t st) {
    if (p.dtype == kBF16)
        return p.D == 64 ? pool_impl<__bf16, 64>(k, pb, p, st) : pool_impl<__bf16, 128>(k, pb, p, st);
    return p.D == 64 ? pool_impl<float, 64>(k, pb, p, st) : pool_impl<float, 128>(k, pb, p, st);
}

}  // namespace moba
