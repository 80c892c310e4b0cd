// C ABI of libmoba.so: argument checks (all before any HIP call), workspace
// carve-up and the launch sequence of the MoBA prefill stages.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moba.h"
#include "moba_internal.hpp"

using namespace moba;

namespace {

constexpr size_t kAlign = 256;
constexpr long long kMaxSeq = 1ll << 24;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
    size_t kbar = 0, kmax2 = 0, khl = 0, defer = 0, idx = 0, cnt = 0, cursor = 0,
           list_off = 0, tile_off = 0, tile_list = 0, lists = 0, part_o = 0, part_lse = 0,
           l2 = 0, delta = 0, part_dq = 0, total = 0;
};

// Past selections over the rows of the chunk: every row in block i keeps
// min(topk - 1, i) past blocks (the last block may hold fewer than B rows).
unsigned long long past_rows(const Problem &p) {
    unsigned long long per_seq = 0;
    const int end = p.r0 + p.R;
    for (int i = p.r0 / p.B; i * p.B < end; ++i)
        per_seq += (unsigned long long)min(p.topk - 1, i) * (unsigned long long)(min(end, (i + 1) * p.B) - i * p.B);
    return per_seq * p.Hq * p.batch;
}

size_t elem_size(const Problem &p) { return p.dtype == kBF16 ? 2 : 4; }

// Upper bound on the past-block attention tiles for prow past selections:
// every list may end in a partial tile.
unsigned long long past_tiles_upper(const Problem &p, unsigned long long prow) {
    const unsigned long long M = (unsigned long long)tile_rows(p);
    const unsigned long long L = (unsigned long long)p.batch * p.Hkv * p.n;
    return (prow + M - 1) / M + L;
}

moba_status_t make_problem(int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                           moba_dtype_t dt, Problem *p) {
    if (batch <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || topk <= 0)
        return MOBA_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv != 0) return MOBA_ERR_INVALID_ARGUMENT;
    if (dt != MOBA_DTYPE_BF16 && dt != MOBA_DTYPE_FP32) return MOBA_ERR_INVALID_ARGUMENT;
    if (D != 64 && D != 128) return MOBA_ERR_UNSUPPORTED;
    if (B % 64 != 0 || S % 64 != 0) return MOBA_ERR_UNSUPPORTED;
    if ((long long)S > kMaxSeq) return MOBA_ERR_UNSUPPORTED;
    p->batch = batch; p->S = S; p->Hq = Hq; p->Hkv = Hkv; p->D = D; p->B = B; p->topk = topk;
    p->dtype = (dt == MOBA_DTYPE_BF16) ? kBF16 : kF32;
    p->G = Hq / Hkv;
    p->n = (S + B - 1) / B;
    p->dense = topk >= p->n;
    p->npast = min(topk - 1, p->n - 1);
    p->r0 = 0;
    p->R = S;
    if (!p->dense && p->npast > kMaxPast) return MOBA_ERR_UNSUPPORTED;
    return MOBA_OK;
}

// Query chunk length in tokens for a requested chunk (<= 0 or >= S: one chunk).
int chunk_len(const Problem &p, int query_chunk) {
    return (query_chunk <= 0 || query_chunk >= p.S) ? p.S : query_chunk;
}

// The longest chunk's rows and the most past selections of any chunk: these
// size every chunk-local buffer.
struct ChunkBound {
    Problem rows;                 // r0 = 0, R = the longest chunk
    unsigned long long prow;      // past selections of the busiest chunk
};

ChunkBound chunk_bound(const Problem &p, int C) {
    ChunkBound cb{p, 0ull};
    cb.rows.r0 = 0;
    cb.rows.R = min(C, p.S);
    Problem w = p;
    for (int r0 = 0; r0 < p.S; r0 += C) {
        w.r0 = r0;
        w.R = min(C, p.S - r0);
        cb.prow = std::max(cb.prow, past_rows(w));
    }
    return cb;
}

Layout gate_layout(const Problem &p) {
    Layout l;
    size_t off = 0;
    const size_t blocks = (size_t)p.batch * p.Hkv * p.n;
    l.kbar = off; off += align_up(blocks * p.D * 4);
    l.kmax2 = off; off += align_up(blocks * 4);
    l.khl = off; off += align_up(blocks * 2 * p.D * 2);
    l.total = off;
    return l;
}

// Workspace of a prefill that runs its sparse stages in query chunks of C
// tokens (C = S: one pass); row-indexed buffers are sized for one chunk.
Layout prefill_layout(const Problem &full, int C) {
    const ChunkBound cb = chunk_bound(full, full.dense ? full.S : C);
    const Problem &p = cb.rows;
    Layout l = gate_layout(p);      // block means and key-norm bounds
    size_t off = l.total;
    // deferred-tile list: a counter then one entry per tile of the largest launch
    const unsigned long long tiles =
        p.dense ? dense_tiles(p) : std::max(past_tiles_upper(p, cb.prow), own_tiles(p));
    l.defer = off; off += align_up(256 + (size_t)tiles * 4);
    if (p.dense) {                  // full causal attention needs nothing more
        l.total = off;
        return l;
    }
    const size_t rows = (size_t)p.batch * p.Hq * p.R;
    const size_t L = (size_t)p.batch * p.Hkv * p.n;
    l.idx = off; off += align_up(rows * p.topk * 4);
    l.cnt = off; off += align_up(L * 4);
    l.cursor = off; off += align_up(L * 4);
    l.list_off = off; off += align_up((L + 1) * 8);
    l.tile_off = off; off += align_up((L + 1) * 4);
    l.tile_list = off; off += align_up((size_t)past_tiles_upper(p, cb.prow) * 4);
    l.lists = off; off += align_up((size_t)cb.prow * 8);
    l.part_o = off; off += align_up(rows * part_slots(p) * p.D * elem_size(p));
    l.part_lse = off; off += align_up(rows * part_slots(p) * 4);
    l.total = off;
    return l;
}

// Workspace of the backward pass: the forward's selection rebuilt (block
// means, block indices, lists), the per-row base-2 log-sum-exp and dO . O, and
// the dq partial slots.
Layout backward_layout(const Problem &p) {
    Layout l = gate_layout(p);
    size_t off = l.total;
    const size_t rows = (size_t)p.batch * p.Hq * p.S;
    const size_t L = (size_t)p.batch * p.Hkv * p.n;
    const unsigned long long prow = past_rows(p);
    l.idx = off; off += align_up(rows * p.topk * 4);
    l.cnt = off; off += align_up(L * 4);
    l.cursor = off; off += align_up(L * 4);
    l.list_off = off; off += align_up((L + 1) * 8);
    l.tile_off = off; off += align_up((L + 1) * 4);
    l.tile_list = off; off += align_up((size_t)past_tiles_upper(p, prow) * 4);
    l.lists = off; off += align_up((size_t)prow * 8);
    l.l2 = off; off += align_up(rows * 4);
    l.delta = off; off += align_up(rows * 4);
    l.part_dq = off; off += align_up(rows * bwd_slots(p) * p.D * 2);
    l.total = off;
    return l;
}

// The backward's problem: bf16 only; a full selection (topk >= n) is run as
// topk = n through the same lists, so it needs n - 1 <= kMaxPast.
moba_status_t backward_problem(int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                               moba_dtype_t dt, Problem *p) {
    moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, p);
    if (rc != MOBA_OK) return rc;
    if (dt != MOBA_DTYPE_BF16) return MOBA_ERR_UNSUPPORTED;
    if (p->dense) {
        if (p->n - 1 > kMaxPast) return MOBA_ERR_UNSUPPORTED;
        rc = make_problem(batch, S, Hq, Hkv, D, B, p->n, dt, p);
    }
    return rc;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

moba_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOBA_OK : MOBA_ERR_HIP; }

PoolBuffers pool_buffers(char *w, const Layout &l, float *kbar_out) {
    PoolBuffers pb;
    pb.kbar = kbar_out ? kbar_out : reinterpret_cast<float *>(w + l.kbar);
    pb.kmax2 = reinterpret_cast<float *>(w + l.kmax2);
    pb.khl = reinterpret_cast<__bf16 *>(w + l.khl);
    return pb;
}

struct Events {
    void *const *ev;
    hipStream_t st;
    hipError_t mark(int i) const {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), st) : hipSuccess;
    }
};

// Checks every sequence of a variable-length batch (host only) and returns the
// largest chunked workspace any of them needs.
moba_status_t varlen_check(const int *cu, int num_seqs, int Hq, int Hkv, int D, int B, int topk,
                           moba_dtype_t dt, int query_chunk, size_t *ws_bytes) {
    if (!cu || num_seqs <= 0 || cu[0] != 0) return MOBA_ERR_INVALID_ARGUMENT;
    if (query_chunk <= 0) return MOBA_ERR_INVALID_ARGUMENT;
    size_t need = 0;
    for (int i = 0; i < num_seqs; ++i) {
        const long long len = (long long)cu[i + 1] - cu[i];
        if (len < 0) return MOBA_ERR_INVALID_ARGUMENT;
        if (len == 0) continue;
        if (len > kMaxSeq || len % 64 != 0) return MOBA_ERR_UNSUPPORTED;
        Problem p;
        const moba_status_t rc = make_problem(1, (int)len, Hq, Hkv, D, B, topk, dt, &p);
        if (rc != MOBA_OK) return rc;
        if (query_chunk % B != 0) return MOBA_ERR_UNSUPPORTED;
        need = std::max(need, prefill_layout(p, chunk_len(p, query_chunk)).total);
    }
    *ws_bytes = need;
    return MOBA_OK;
}

// Pointers of a prefill: present, 16-byte aligned (lse 4-byte), out and lse
// overlapping no input.
moba_status_t check_io(const void *q, const void *k, const void *v, const void *out,
                       const float *lse_out, const Problem &p) {
    if (!q || !k || !v || !out) return MOBA_ERR_INVALID_ARGUMENT;
    const size_t qbytes = (size_t)p.batch * p.S * p.Hq * p.D * elem_size(p);
    const size_t kvbytes = (size_t)p.batch * p.S * p.Hkv * p.D * elem_size(p);
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kvbytes) ||
        overlaps(out, qbytes, v, kvbytes))
        return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(lse_out, 4))
        return MOBA_ERR_UNSUPPORTED;
    if (lse_out && (overlaps(lse_out, (size_t)p.batch * p.Hq * p.S * 4, out, qbytes) ||
                    overlaps(lse_out, (size_t)p.batch * p.Hq * p.S * 4, q, qbytes)))
        return MOBA_ERR_INVALID_ARGUMENT;
    return MOBA_OK;
}

moba_status_t prefill_impl(const void *q, const void *k, const void *v, void *out, int batch,
                           int S, int Hq, int Hkv, int D, int B, int topk, moba_dtype_t dt,
                           int query_chunk, void *ws, size_t ws_bytes, void *stream,
                           void *const *events, float *lse_out = nullptr) {
    Problem p;
    moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    // query_chunk 0: one pass over the whole sequence (moba_prefill)
    if (query_chunk != 0 && query_chunk % B != 0) return MOBA_ERR_UNSUPPORTED;
    const int C = chunk_len(p, query_chunk);
    rc = check_io(q, k, v, out, lse_out, p);
    if (rc != MOBA_OK) return rc;
    const Layout l = prefill_layout(p, C);
    if (ws_bytes < l.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    if (!ws) return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(ws, kAlign)) return MOBA_ERR_UNSUPPORTED;

    hipStream_t st = as_stream(stream);
    const Events E{events, st};
    char *w = static_cast<char *>(ws);
    const PoolBuffers pb = pool_buffers(w, l, nullptr);
    float *kbar = pb.kbar;
    AttnBuffers bf;
    bf.q = q; bf.k = k; bf.v = v; bf.out = out;
    bf.kmax2 = pb.kmax2;
    bf.defer_count = reinterpret_cast<unsigned *>(w + l.defer);
    bf.defer_list = reinterpret_cast<unsigned *>(w + l.defer + 256);
    bf.lse_out = lse_out;
    hipError_t e = hipSuccess;
    if (p.dense) {
        // key-norm bounds (the pool pass), then full causal attention
        if ((e = E.mark(MOBA_STAGE_POOL)) != hipSuccess) return MOBA_ERR_HIP;
        if ((e = launch_pool(k, pb, p, st)) != hipSuccess) return MOBA_ERR_HIP;
        for (int i = MOBA_STAGE_GATE; i <= MOBA_STAGE_ATTN_PAST && e == hipSuccess; ++i) e = E.mark(i);
        if (e == hipSuccess) e = launch_attn_dense(bf, p, st);
        for (int i = MOBA_STAGE_ATTN_OWN; i <= MOBA_NUM_STAGES && e == hipSuccess; ++i) e = E.mark(i);
        return hip_status(e);
    }
    int32_t *idx = reinterpret_cast<int32_t *>(w + l.idx);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(w + l.cnt);
    uint32_t *cursor = reinterpret_cast<uint32_t *>(w + l.cursor);
    uint64_t *list_off = reinterpret_cast<uint64_t *>(w + l.list_off);
    uint32_t *tile_off = reinterpret_cast<uint32_t *>(w + l.tile_off);
    uint32_t *tile_list = reinterpret_cast<uint32_t *>(w + l.tile_list);
    uint64_t *lists = reinterpret_cast<uint64_t *>(w + l.lists);
    bf.part_o = w + l.part_o;
    bf.part_lse = reinterpret_cast<float *>(w + l.part_lse);
    bf.lists = lists; bf.list_off = list_off; bf.tile_off = tile_off; bf.tile_list = tile_list;

    if ((e = E.mark(MOBA_STAGE_POOL)) != hipSuccess) return MOBA_ERR_HIP;
    if ((e = launch_pool(k, pb, p, st)) != hipSuccess) return MOBA_ERR_HIP;
    // the sparse stages, one query chunk at a time (stage events: last chunk)
    for (int r0 = 0; r0 < S; r0 += C) {
        p.r0 = r0;
        p.R = min(C, S - r0);
        const unsigned long long prow = past_rows(p);
        const unsigned long long tiles_upper = past_tiles_upper(p, prow);
        if ((e = E.mark(MOBA_STAGE_GATE)) != hipSuccess) return MOBA_ERR_HIP;
        if ((e = launch_gate(q, kbar, pb.khl, idx, p, st)) != hipSuccess) return MOBA_ERR_HIP;
        if ((e = E.mark(MOBA_STAGE_INDEX)) != hipSuccess) return MOBA_ERR_HIP;
        if (prow > 0 &&
            (e = launch_index(idx, cnt, cursor, list_off, tile_off, tile_list, tiles_upper, lists,
                              p, st)) != hipSuccess)
            return MOBA_ERR_HIP;
        if ((e = E.mark(MOBA_STAGE_ATTN_PAST)) != hipSuccess) return MOBA_ERR_HIP;
        if (prow > 0 && (e = launch_attn_past(bf, p, tiles_upper, st)) != hipSuccess)
            return MOBA_ERR_HIP;
        if ((e = E.mark(MOBA_STAGE_ATTN_OWN)) != hipSuccess) return MOBA_ERR_HIP;
        if ((e = launch_attn_own(bf, p, st)) != hipSuccess) return MOBA_ERR_HIP;
        if (prow > 0 && !merge_in_own_pass(p) && (e = launch_merge(bf, p, st)) != hipSuccess)
            return MOBA_ERR_HIP;
    }
    if ((e = E.mark(MOBA_NUM_STAGES)) != hipSuccess) return MOBA_ERR_HIP;
    return MOBA_OK;
}

// ---- allocation-free prefill: a fixed scratch array per device ----
//
// scratch is this library's own device memory for moba_prefill_noalloc.  Each
// GPU the library runs on holds its copy until the process ends.  In host code
// `scratch` only names the array: its device address, different on every
// device, comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there and kept in scratch_addr.
static_assert(MOBA_NOALLOC_SCRATCH_BYTES % kAlign == 0, "scratch size");
static __device__ __align__(256) char scratch[MOBA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_addr[kMaxDevices];

moba_status_t device_scratch(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOBA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOBA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void *a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return MOBA_ERR_HIP;
        if (!aligned(a, kAlign)) return MOBA_ERR_HIP;
        scratch_addr[dev] = a;
    }
    *ptr = scratch_addr[dev];
    return MOBA_OK;
}

// Query chunk (tokens, a multiple of B; S for one pass) of the largest
// chunked prefill whose workspace fits the scratch array, or 0 if not even
// one block per chunk fits.  The workspace grows with the chunk length.
int noalloc_chunk(const Problem &p) {
    const size_t cap = MOBA_NOALLOC_SCRATCH_BYTES;
    if (p.dense) return prefill_layout(p, p.S).total <= cap ? p.S : 0;
    if (prefill_layout(p, p.S).total <= cap) return p.S;
    int lo = 0, hi = p.n;        // blocks per chunk: lo fits (0 = none), hi does not
    while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (prefill_layout(p, mid * p.B).total <= cap) lo = mid;
        else hi = mid;
    }
    return lo * p.B;
}

}  // namespace

extern "C" {

int moba_abi_version(void) { return MOBA_ABI_VERSION; }

const char *moba_status_string(moba_status_t s) {
    switch (s) {
    case MOBA_OK: return "ok";
    case MOBA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOBA_ERR_UNSUPPORTED: return "unsupported shape, alignment or dtype";
    case MOBA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOBA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

moba_status_t moba_workspace_size(int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                                  moba_dtype_t dt, size_t *prefill_bytes, size_t *gate_bytes) {
    Problem p;
    const moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (prefill_bytes) *prefill_bytes = prefill_layout(p, p.S).total;
    if (gate_bytes) *gate_bytes = gate_layout(p).total;
    return MOBA_OK;
}

moba_status_t moba_workspace_size_chunked(int batch, int S, int Hq, int Hkv, int D, int B,
                                          int topk, moba_dtype_t dt, int query_chunk,
                                          size_t *prefill_bytes) {
    Problem p;
    const moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (query_chunk <= 0) return MOBA_ERR_INVALID_ARGUMENT;
    if (query_chunk % B != 0) return MOBA_ERR_UNSUPPORTED;
    if (!prefill_bytes) return MOBA_ERR_INVALID_ARGUMENT;
    *prefill_bytes = prefill_layout(p, chunk_len(p, query_chunk)).total;
    return MOBA_OK;
}

moba_status_t moba_pool(const void *k, float *kbar, int batch, int S, int Hkv, int D, int B,
                        moba_dtype_t dt, void *ws, size_t ws_bytes, void *stream) {
    Problem p;
    const moba_status_t rc = make_problem(batch, S, Hkv, Hkv, D, B, 1, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (!k || !kbar || !ws) return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(k, 16) || !aligned(kbar, 4) || !aligned(ws, kAlign)) return MOBA_ERR_UNSUPPORTED;
    const Layout l = gate_layout(p);
    if (ws_bytes < l.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    char *w = static_cast<char *>(ws);
    return hip_status(launch_pool(k, pool_buffers(w, l, kbar), p, as_stream(stream)));
}

moba_status_t moba_gate(const void *q, const void *k, int32_t *block_idx, int batch, int S,
                        int Hq, int Hkv, int D, int B, int topk, moba_dtype_t dt, void *ws,
                        size_t ws_bytes, void *stream) {
    Problem p;
    const moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (!q || !k || !block_idx || !ws) return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(block_idx, 4) || !aligned(ws, kAlign))
        return MOBA_ERR_UNSUPPORTED;
    const Layout l = gate_layout(p);
    if (ws_bytes < l.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = as_stream(stream);
    char *w = static_cast<char *>(ws);
    const PoolBuffers pb = pool_buffers(w, l, nullptr);
    hipError_t e = hipSuccess;
    if (!p.dense) e = launch_pool(k, pb, p, st);
    if (e == hipSuccess) e = launch_gate(q, pb.kbar, pb.khl, block_idx, p, st);
    return hip_status(e);
}

moba_status_t moba_gate_scores(const void *q, const void *k, float *scores, int batch, int S,
                               int Hq, int Hkv, int D, int B, moba_dtype_t dt, void *ws,
                               size_t ws_bytes, void *stream) {
    Problem p;
    const moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, 1, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (!q || !k || !scores || !ws) return MOBA_ERR_INVALID_ARGUMENT;
    if (p.dtype != kBF16) return MOBA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 4) || !aligned(ws, kAlign))
        return MOBA_ERR_UNSUPPORTED;
    const Layout l = gate_layout(p);
    if (ws_bytes < l.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = as_stream(stream);
    char *w = static_cast<char *>(ws);
    const PoolBuffers pb = pool_buffers(w, l, nullptr);
    hipError_t e = launch_pool(k, pb, p, st);
    if (e == hipSuccess) e = launch_gate_scores(q, pb.khl, scores, p, st);
    return hip_status(e);
}

moba_status_t moba_prefill(const void *q, const void *k, const void *v, void *out, int batch,
                           int S, int Hq, int Hkv, int D, int B, int topk, moba_dtype_t dt,
                           void *ws, size_t ws_bytes, void *stream) {
    return prefill_impl(q, k, v, out, batch, S, Hq, Hkv, D, B, topk, dt, 0, ws, ws_bytes, stream,
                        nullptr);
}

moba_status_t moba_prefill_chunked(const void *q, const void *k, const void *v, void *out,
                                   int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                                   moba_dtype_t dt, int query_chunk, void *ws, size_t ws_bytes,
                                   void *stream) {
    if (query_chunk <= 0) return MOBA_ERR_INVALID_ARGUMENT;
    return prefill_impl(q, k, v, out, batch, S, Hq, Hkv, D, B, topk, dt, query_chunk, ws,
                        ws_bytes, stream, nullptr);
}

moba_status_t moba_prefill_timed(const void *q, const void *k, const void *v, void *out,
                                 int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                                 moba_dtype_t dt, void *ws, size_t ws_bytes, void *stream,
                                 void *const *stage_events) {
    if (!stage_events) return MOBA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i <= MOBA_NUM_STAGES; ++i)
        if (!stage_events[i]) return MOBA_ERR_INVALID_ARGUMENT;
    return prefill_impl(q, k, v, out, batch, S, Hq, Hkv, D, B, topk, dt, 0, ws, ws_bytes, stream,
                        stage_events);
}

moba_status_t moba_prefill_noalloc(const void *q, const void *k, const void *v, void *out,
                                   int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                                   moba_dtype_t dt, void *stream) {
    Problem p;
    moba_status_t rc = make_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if ((rc = check_io(q, k, v, out, nullptr, p)) != MOBA_OK) return rc;
    const int C = noalloc_chunk(p);
    if (C == 0) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    const moba_status_t src = device_scratch(&ws);
    if (src != MOBA_OK) return src;
    return prefill_impl(q, k, v, out, batch, S, Hq, Hkv, D, B, topk, dt, C >= S ? 0 : C, ws,
                        MOBA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

moba_status_t moba_workspace_size_varlen(const int *cu_seqlens, int num_seqs, int Hq, int Hkv,
                                         int D, int B, int topk, moba_dtype_t dt,
                                         int query_chunk, size_t *prefill_bytes) {
    size_t need = 0;
    const moba_status_t rc =
        varlen_check(cu_seqlens, num_seqs, Hq, Hkv, D, B, topk, dt, query_chunk, &need);
    if (rc != MOBA_OK) return rc;
    if (!prefill_bytes) return MOBA_ERR_INVALID_ARGUMENT;
    *prefill_bytes = need;
    return MOBA_OK;
}

moba_status_t moba_prefill_varlen(const void *q, const void *k, const void *v, void *out,
                                  const int *cu_seqlens, int num_seqs, int Hq, int Hkv, int D,
                                  int B, int topk, moba_dtype_t dt, int query_chunk, void *ws,
                                  size_t ws_bytes, void *stream) {
    size_t need = 0;
    moba_status_t rc =
        varlen_check(cu_seqlens, num_seqs, Hq, Hkv, D, B, topk, dt, query_chunk, &need);
    if (rc != MOBA_OK) return rc;
    if (!q || !k || !v || !out) return MOBA_ERR_INVALID_ARGUMENT;
    const size_t es = dt == MOBA_DTYPE_BF16 ? 2 : 4;
    const size_t total = (size_t)cu_seqlens[num_seqs];
    const size_t qbytes = total * Hq * D * es, kvbytes = total * Hkv * D * es;
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kvbytes) ||
        overlaps(out, qbytes, v, kvbytes))
        return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return MOBA_ERR_UNSUPPORTED;
    if (ws_bytes < need) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    if (!ws && need > 0) return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(ws, kAlign)) return MOBA_ERR_UNSUPPORTED;
    // every sequence passed the checks above, so no call below fails them
    for (int i = 0; i < num_seqs; ++i) {
        const int len = cu_seqlens[i + 1] - cu_seqlens[i];
        if (len == 0) continue;
        const size_t t0 = (size_t)cu_seqlens[i];
        rc = prefill_impl(static_cast<const char *>(q) + t0 * Hq * D * es,
                          static_cast<const char *>(k) + t0 * Hkv * D * es,
                          static_cast<const char *>(v) + t0 * Hkv * D * es,
                          static_cast<char *>(out) + t0 * Hq * D * es, 1, len, Hq, Hkv, D, B,
                          topk, dt, query_chunk, ws, ws_bytes, stream, nullptr);
        if (rc != MOBA_OK) return rc;
    }
    return MOBA_OK;
}

moba_status_t moba_prefill_lse(const void *q, const void *k, const void *v, void *out,
                               float *lse, int batch, int S, int Hq, int Hkv, int D, int B,
                               int topk, moba_dtype_t dt, void *ws, size_t ws_bytes,
                               void *stream) {
    if (!lse) return MOBA_ERR_INVALID_ARGUMENT;
    return prefill_impl(q, k, v, out, batch, S, Hq, Hkv, D, B, topk, dt, 0, ws, ws_bytes, stream,
                        nullptr, lse);
}

moba_status_t moba_workspace_size_backward(int batch, int S, int Hq, int Hkv, int D, int B,
                                           int topk, moba_dtype_t dt, size_t *bytes) {
    Problem p;
    const moba_status_t rc = backward_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (!bytes) return MOBA_ERR_INVALID_ARGUMENT;
    *bytes = backward_layout(p).total;
    return MOBA_OK;
}

moba_status_t moba_backward(const void *q, const void *k, const void *v, const void *out,
                            const void *dout, const float *lse, void *dq, void *dk, void *dv,
                            int batch, int S, int Hq, int Hkv, int D, int B, int topk,
                            moba_dtype_t dt, void *ws, size_t ws_bytes, void *stream) {
    Problem p;
    const moba_status_t rc = backward_problem(batch, S, Hq, Hkv, D, B, topk, dt, &p);
    if (rc != MOBA_OK) return rc;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
        return MOBA_ERR_INVALID_ARGUMENT;
    const size_t qb = (size_t)batch * S * Hq * D * 2, kb = (size_t)batch * S * Hkv * D * 2;
    const size_t lb = (size_t)batch * Hq * S * 4;
    const void *in[6] = {q, k, v, out, dout, lse};
    const size_t inb[6] = {qb, kb, kb, qb, qb, lb};
    void *outp[3] = {dq, dk, dv};
    const size_t outb[3] = {qb, kb, kb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outp[o], outb[o], in[i], inb[i])) return MOBA_ERR_INVALID_ARGUMENT;
        for (int o2 = 0; o2 < o; ++o2)
            if (overlaps(outp[o], outb[o], outp[o2], outb[o2])) return MOBA_ERR_INVALID_ARGUMENT;
    }
    for (int i = 0; i < 5; ++i)
        if (!aligned(in[i], 16)) return MOBA_ERR_UNSUPPORTED;
    if (!aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return MOBA_ERR_UNSUPPORTED;
    const Layout l = backward_layout(p);
    if (ws_bytes < l.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
    if (!ws) return MOBA_ERR_INVALID_ARGUMENT;
    if (!aligned(ws, kAlign)) return MOBA_ERR_UNSUPPORTED;

    hipStream_t st = as_stream(stream);
    char *w = static_cast<char *>(ws);
    const PoolBuffers pb = pool_buffers(w, l, nullptr);
    int32_t *idx = reinterpret_cast<int32_t *>(w + l.idx);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(w + l.cnt);
    uint32_t *cursor = reinterpret_cast<uint32_t *>(w + l.cursor);
    uint64_t *list_off = reinterpret_cast<uint64_t *>(w + l.list_off);
    uint32_t *tile_off = reinterpret_cast<uint32_t *>(w + l.tile_off);
    uint32_t *tile_list = reinterpret_cast<uint32_t *>(w + l.tile_list);
    uint64_t *lists = reinterpret_cast<uint64_t *>(w + l.lists);
    const unsigned long long prow = past_rows(p);
    const unsigned long long tiles_upper = past_tiles_upper(p, prow);
    hipError_t e = launch_pool(k, pb, p, st);
    if (e == hipSuccess) e = launch_gate(q, pb.kbar, pb.khl, idx, p, st);
    if (e == hipSuccess)
        e = launch_index(idx, cnt, cursor, list_off, tile_off, tile_list, tiles_upper, lists, p,
                         st);
    if (e != hipSuccess) return MOBA_ERR_HIP;
    BwdBuffers bb;
    bb.q = q; bb.k = k; bb.v = v; bb.out = out; bb.dout = dout; bb.lse = lse;
    bb.dq = dq; bb.dk = dk; bb.dv = dv;
    bb.l2 = reinterpret_cast<float *>(w + l.l2);
    bb.delta = reinterpret_cast<float *>(w + l.delta);
    bb.part_dq = w + l.part_dq;
    bb.lists = lists; bb.list_off = list_off; bb.tile_off = tile_off; bb.tile_list = tile_list;
    return hip_status(launch_backward(bb, p, prow > 0 ? tiles_upper : 0, st));
}

}  // extern "C"
