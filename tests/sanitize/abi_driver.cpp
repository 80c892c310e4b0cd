// Calls the C-ABI's host-side paths under AddressSanitizer and
// UndefinedBehaviorSanitizer (the library's sources built for the host only by
// tests/test_sanitizers.py): workspace sizing over many shapes, including the
// 1M- and 10M-token ones whose sizes need 64-bit arithmetic, and every
// argument check that must refuse a call before any HIP call.  The device
// addresses passed are never dereferenced.  Prints "ok" and exits 0 when every
// call returns what it should.
#include <cstdint>
#include <cstdio>

#include "moba.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);  \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static void *at(unsigned long long a) { return reinterpret_cast<void *>(a); }
static const unsigned long long FAKE = 1ull << 40;
static const moba_dtype_t BF16 = MOBA_DTYPE_BF16, F32 = MOBA_DTYPE_FP32;

int main() {
    EXPECT(moba_abi_version() == MOBA_ABI_VERSION);
    for (int s = 0; s < 5; ++s) EXPECT(moba_status_string((moba_status_t)s) != nullptr);
    EXPECT(moba_status_string((moba_status_t)99) != nullptr);

    size_t pb = 0, gb = 0;
    // sizing: valid shapes of every kind
    const int shapes[][7] = {{1, 1024, 2, 2, 64, 128, 3},     {2, 640, 4, 2, 64, 64, 4},
                             {1, 1088, 2, 2, 64, 128, 3},     {1, 1088, 2, 2, 64, 128, 9},
                             {1, 4096, 2, 1, 128, 64, 32},    {1, 1 << 17, 32, 8, 128, 4096, 12},
                             {1, 1 << 20, 32, 8, 128, 4096, 12}, {1, 64 * 4160, 4, 1, 128, 64, 12},
                             {1, 10 << 20, 32, 8, 128, 4096, 12}};
    for (const auto &s : shapes) {
        for (moba_dtype_t dt : {BF16, F32}) {
            EXPECT(moba_workspace_size(s[0], s[1], s[2], s[3], s[4], s[5], s[6], dt, &pb, &gb) == MOBA_OK);
            EXPECT(pb >= gb && gb > 0);
            size_t cb = 0;
            EXPECT(moba_workspace_size_chunked(s[0], s[1], s[2], s[3], s[4], s[5], s[6], dt, s[5] * 4, &cb) ==
                   MOBA_OK);
            EXPECT(cb > 0 && cb <= pb);
        }
        size_t bb = 0;
        const moba_status_t rb = moba_workspace_size_backward(s[0], s[1], s[2], s[3], s[4], s[5], s[6], BF16, &bb);
        EXPECT(rb == MOBA_OK || rb == MOBA_ERR_UNSUPPORTED);
    }
    // sizing: refusals
    EXPECT(moba_workspace_size(0, 1024, 2, 2, 64, 128, 3, BF16, &pb, &gb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size(1, 1024, 3, 2, 64, 128, 3, BF16, &pb, &gb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size(1, 1024, 2, 2, 64, 128, 0, BF16, &pb, &gb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size(1, 1024, 2, 2, 64, 128, 3, (moba_dtype_t)7, &pb, &gb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size(1, 1024, 2, 2, 96, 128, 3, BF16, &pb, &gb) == MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_workspace_size(1, 1000, 2, 2, 64, 128, 3, BF16, &pb, &gb) == MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_workspace_size(1, 1 << 25, 2, 2, 64, 4096, 3, BF16, &pb, &gb) == MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_workspace_size(1, 1024, 2, 2, 64, 128, 3, BF16, nullptr, &gb) == MOBA_OK);   // outputs optional
    EXPECT(moba_workspace_size(-1, -1, -1, -1, -1, -1, -1, BF16, &pb, &gb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size(1 << 30, 1 << 24, 1 << 20, 1, 128, 64, 3, BF16, &pb, &gb) != MOBA_OK ||
           pb > 0);   // absurd sizes: refused or sized, never wrapped to a small number
    size_t cb = 0;
    EXPECT(moba_workspace_size_chunked(1, 1024, 2, 2, 64, 128, 3, BF16, 0, &cb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size_chunked(1, 1024, 2, 2, 64, 128, 3, BF16, 100, &cb) == MOBA_ERR_UNSUPPORTED);
    const int cu_ok[] = {0, 640, 1728, 1728, 1792}, cu_bad[] = {0, 128, 64}, cu_odd[] = {0, 100};
    EXPECT(moba_workspace_size_varlen(cu_ok, 4, 4, 2, 128, 128, 3, BF16, 256, &cb) == MOBA_OK);
    EXPECT(moba_workspace_size_varlen(cu_bad, 2, 4, 2, 128, 128, 3, BF16, 256, &cb) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_workspace_size_varlen(cu_odd, 1, 4, 2, 128, 128, 3, BF16, 256, &cb) == MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_workspace_size_varlen(nullptr, 1, 4, 2, 128, 128, 3, BF16, 256, &cb) == MOBA_ERR_INVALID_ARGUMENT);

    // entry points: every call below fails its checks before any HIP call
    void *q = at(FAKE), *k = at(FAKE + (1ull << 32)), *v = at(FAKE + (2ull << 32)), *o = at(FAKE + (3ull << 32));
    void *ws = at(FAKE + (4ull << 32));
    const size_t big = 1ull << 40;
    EXPECT(moba_prefill(nullptr, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_prefill(q, k, v, at(FAKE + 64), 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);   // out overlaps q
    EXPECT(moba_prefill(at(FAKE + 2), k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr) ==
           MOBA_ERR_UNSUPPORTED);        // misaligned
    EXPECT(moba_prefill(q, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, 16, nullptr) == MOBA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moba_prefill(q, k, v, o, 1, 1024, 2, 2, 80, 128, 3, BF16, ws, big, nullptr) == MOBA_ERR_UNSUPPORTED);
    void *ev[MOBA_NUM_STAGES + 1] = {};
    EXPECT(moba_prefill_timed(q, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr, ev) ==
           MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_prefill_chunked(q, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, 0, ws, big, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_prefill_chunked(q, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, 256, ws, 1024, nullptr) ==
           MOBA_ERR_WORKSPACE_TOO_SMALL);
    const int cu72[] = {0, 640, 1728, 1800};
    EXPECT(moba_prefill_varlen(q, k, v, o, cu72, 3, 4, 2, 128, 128, 3, BF16, 256, ws, big, nullptr) ==
           MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_prefill_varlen(q, k, v, o, cu_ok, 4, 4, 2, 128, 128, 3, BF16, 256, ws, 64, nullptr) ==
           MOBA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moba_prefill_lse(q, k, v, o, nullptr, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_prefill_lse(q, k, v, o, static_cast<float *>(at(FAKE + (3ull << 32) + 256)), 1, 1024, 2, 2, 64,
                            128, 3, BF16, ws, big, nullptr) == MOBA_ERR_INVALID_ARGUMENT);   // overlaps out
    float *lse = static_cast<float *>(at(FAKE + (5ull << 32)));
    void *dq = at(FAKE + (6ull << 32)), *dk = at(FAKE + (7ull << 32)), *dv = at(FAKE + (8ull << 32));
    void *dout = at(FAKE + (9ull << 32)), *wsb = at(FAKE + (10ull << 32));
    EXPECT(moba_backward(q, k, v, o, dout, lse, nullptr, dk, dv, 1, 1024, 2, 2, 64, 128, 3, BF16, wsb, big,
                         nullptr) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_backward(q, k, v, o, dout, lse, o, dk, dv, 1, 1024, 2, 2, 64, 128, 3, BF16, wsb, big, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);   // dq overlaps out
    EXPECT(moba_backward(q, k, v, o, dout, lse, dq, dk, dv, 1, 1024, 2, 2, 64, 128, 3, F32, wsb, big, nullptr) ==
           MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_backward(q, k, v, o, dout, lse, dq, dk, dv, 1, 1024, 2, 2, 64, 128, 3, BF16, wsb, 1024, nullptr) ==
           MOBA_ERR_WORKSPACE_TOO_SMALL);
    int32_t *idx = static_cast<int32_t *>(at(FAKE + (11ull << 32)));
    EXPECT(moba_gate(nullptr, k, idx, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, big, nullptr) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_gate(q, k, idx, 1, 1024, 2, 2, 64, 128, 3, BF16, ws, 8, nullptr) == MOBA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moba_gate_scores(nullptr, k, static_cast<float *>(ws), 1, 1024, 2, 2, 64, 128, BF16, ws, big,
                            nullptr) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_gate_scores(q, k, static_cast<float *>(o), 1, 1024, 2, 2, 64, 128, F32, ws, big, nullptr) ==
           MOBA_ERR_UNSUPPORTED);
    EXPECT(moba_gate_scores(q, k, static_cast<float *>(o), 1, 1024, 2, 2, 64, 128, BF16, ws, 8, nullptr) ==
           MOBA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moba_pool(k, nullptr, 1, 1024, 2, 64, 128, BF16, ws, big, nullptr) == MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_pool(k, static_cast<float *>(ws), 1, 1024, 2, 64, 100, BF16, ws, big, nullptr) ==
           MOBA_ERR_UNSUPPORTED);
    // the allocation-free entry point refuses what its scratch array cannot hold, and bad pointers
    EXPECT(moba_prefill_noalloc(q, k, v, o, 1, 1 << 18, 32, 8, 128, 1 << 16, 3, BF16, nullptr) ==
           MOBA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moba_prefill_noalloc(nullptr, k, v, o, 1, 1024, 2, 2, 64, 128, 3, BF16, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);
    EXPECT(moba_prefill_noalloc(q, k, v, at(FAKE + 64), 1, 1024, 2, 2, 64, 128, 3, BF16, nullptr) ==
           MOBA_ERR_INVALID_ARGUMENT);
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
