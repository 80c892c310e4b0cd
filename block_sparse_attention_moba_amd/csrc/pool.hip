// Block means of the keys (the "aggregated representation of the block keys"
// the gate compares each query with; Taiwan AI overview of MoBA, section
// "技術細節與優勢").
//
// Two launches.  pool_partial: one workgroup per (chunk of CT tokens, block,
// KV head, batch) streams CT x D keys with 16-byte loads (one D-row per
// D/8 lanes, so a wave reads 64 x 16 contiguous bytes per step) and writes
// the chunk's fp32 column sums and the largest squared key norm of the chunk.
// pool_finalize: sums the chunk partials of a block in a fixed order and
// divides by the block's token count (B, or S mod B for a short last block), writes the mean also as a bf16 hi + lo pair (the
// operands of the matrix-core gate), and takes the block's largest squared key
// norm (the attention kernels bound every logit of the block by it).  No atomics,
// so the result is bitwise reproducible.
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

// grid (nchunk, n * Hkv, batch), 256 threads.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_partial_kernel(const T *__restrict__ k,
                                                           float *__restrict__ partial,
                                                           float *__restrict__ partial_nmax, int S,
                                                           int Hkv, int B, int n, int CT) {
    constexpr int LPT = D / 8;       // lanes per token row
    constexpr int TPP = 256 / LPT;   // token rows per pass
    __shared__ float red[TPP][D + 1];
    __shared__ float redn[TPP];
    const int chunk = blockIdx.x;
    const int j = blockIdx.y / Hkv;
    const int g = blockIdx.y % Hkv;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int vec = tid % LPT;
    const int tr = tid / LPT;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float nmax = 0.f;
    const int t0 = j * B + chunk * CT;
    const int t1 = min(t0 + CT, S);              // a short last block ends at S
    for (int t = t0 + tr; t < t1; t += TPP) {
        float f[8];
        load8(k + (((size_t)b * S + t) * Hkv + g) * D + vec * 8, f);
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += f[e];
            sq = fmaf(f[e], f[e], sq);
        }
        // squared norm of token t: sum over the LPT lanes that hold its row
#pragma unroll
        for (int off = 1; off < LPT; off <<= 1) sq += __shfl_xor(sq, off, LPT);
        nmax = fmaxf(nmax, sq);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr][vec * 8 + e] = acc[e];
    if (vec == 0) redn[tr] = nmax;
    __syncthreads();
    const int nchunk = gridDim.x;
    const size_t pc = (((size_t)b * Hkv + g) * n + j) * nchunk + chunk;
    if (tid < D) {
        float s = 0.f;
        for (int r = 0; r < TPP; ++r) s += red[r][tid];
        partial[pc * D + tid] = s;
    }
    if (tid == 0) {
        float m = 0.f;
        for (int r = 0; r < TPP; ++r) m = fmaxf(m, redn[r]);
        partial_nmax[pc] = m;
    }
}

// grid (ceil(batch * Hkv * n * D / 256)), 256 threads: one output element each.
__global__ __launch_bounds__(256) void pool_finalize_kernel(const float *__restrict__ partial,
                                                            const float *__restrict__ partial_nmax,
                                                            float *__restrict__ kbar,
                                                            float *__restrict__ kmax2,
                                                            __bf16 *__restrict__ khl,
                                                            long long total, int D, int nchunk,
                                                            int B, int S, int n) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const long long blk = e / D;
    const int i = (int)(e % D);
    const float *src = partial + (size_t)blk * nchunk * D + i;
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += src[(size_t)c * D];
    const int j = (int)(blk % n);
    const float m = s / (float)min(B, S - j * B);   // tokens present in block j
    kbar[e] = m;
    // bf16 split for the matrix-core gate: m = hi + lo + O(2^-17 |m|)
    const __bf16 hi = (__bf16)m;
    khl[(blk * 2) * D + i] = hi;
    khl[(blk * 2 + 1) * D + i] = (__bf16)(m - (float)hi);
    if (i == 0) {
        float m = 0.f;
        for (int c = 0; c < nchunk; ++c) m = fmaxf(m, partial_nmax[(size_t)blk * nchunk + c]);
        kmax2[blk] = m;
    }
}

template <typename T, int D>
static hipError_t pool_impl(const void *k, const PoolBuffers &pb, const Problem &p,
                            hipStream_t st) {
    const int CT = pool_chunk(p.B);
    const int nchunk = p.B / CT;
    dim3 grid(nchunk, p.n * p.Hkv, p.batch);
    pool_partial_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T *>(k), pb.partial,
                                                    pb.partial_nmax, p.S, p.Hkv, p.B, p.n, CT);
    const long long total = (long long)p.batch * p.Hkv * p.n * D;
    pool_finalize_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
        pb.partial, pb.partial_nmax, pb.kbar, pb.kmax2, pb.khl, total, D, nchunk, p.B, p.S, p.n);
    return hipGetLastError();
}

hipError_t launch_pool(const void *k, const PoolBuffers &pb, const Problem &p, hipStream_t st) {
    if (p.dtype == kBF16)
        return p.D == 64 ? pool_impl<__bf16, 64>(k, pb, p, st) : pool_impl<__bf16, 128>(k, pb, p, st);
    return p.D == 64 ? pool_impl<float, 64>(k, pb, p, st) : pool_impl<float, 128>(k, pb, p, st);
}

}  // namespace moba
