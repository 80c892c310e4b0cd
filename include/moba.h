/*
 * moba.h -- MoBA (Mixture of Block Attention) causal prefill forward on one
 * AMD Instinct MI355X (gfx950).  C ABI of libmoba.so.
 *
 * The operation.  MoBA splits the context into blocks of `block_size`
 * tokens and routes every query token to a few blocks with a parameter-free
 * top-k gate; attention then runs over the tokens of the chosen blocks only
 * (MoBA tech-report write-up, section "MoBA：將MoE原理應用于注意力機制": the
 * list of MoBA's parts and the five implementation steps).  The gate scores
 * a query against an aggregated representation of each block's keys; the
 * block holding the query is always chosen and no token attends to a future
 * position (Taiwan AI overview, section "技術細節與優勢").  Partial results of
 * the current block and the history blocks are merged by an online softmax
 * (write-up, the fifth implementation step).  With every causal block
 * selected the result is full causal attention (the seamless full / sparse
 * switch the write-up and the overview describe).
 *
 * Blocks.  Block j holds tokens [j * block_size, (j + 1) * block_size); there
 * are n = ceil(seqlen / block_size) blocks, and when block_size does not
 * divide seqlen the last block is short (seqlen mod block_size tokens).  A
 * short last block is only ever a query's own block, never a past block.
 *
 * Readings fixed by this library where the pages are silent:
 *   - block key = mean of the block's keys over the tokens present (fp32);
 *   - gate score = <q, mean key>, unscaled, for past blocks j < t / block_size;
 *   - `topk` counts the own block: a query uses its own block plus the
 *     min(topk - 1, t / block_size) best-scoring past blocks; ties go to the
 *     smaller block index;
 *   - softmax scale 1 / sqrt(head_dim); query head h uses KV head
 *     h / (num_q_heads / num_kv_heads).
 *
 * Layouts (all contiguous, head_dim innermost, element type = `dtype`):
 *   q, out  [batch][seqlen][num_q_heads][head_dim]
 *   k, v    [batch][seqlen][num_kv_heads][head_dim]
 *   block_idx (int32) [batch][num_q_heads][seqlen][topk]: the selected
 *           blocks of each query row, ascending, own block included (it is
 *           the last valid entry), then -1 padding.
 *   kbar (fp32) [batch][num_kv_heads][n][head_dim].
 *
 * Ownership.  Every pointer is caller-owned device memory.  The library
 * allocates nothing, keeps no state between calls and is reentrant: calls on
 * different streams with different workspaces may run concurrently.  Outputs
 * are fully overwritten.  `out` must not overlap q, k or v.  (The one
 * exception is moba_prefill_noalloc, at the end: it works in a scratch array
 * of the library's own, shared by its calls on one GPU.)
 *
 * Errors.  The return code is the only channel.  All argument checks run
 * before any HIP call.  Work is asynchronous on `stream` (a hipStream_t; NULL
 * is the default stream): results are valid once the caller synchronises the
 * stream, and a later device error is reported by the caller's next HIP call.
 *   MOBA_ERR_INVALID_ARGUMENT   null pointer, a size <= 0, num_q_heads not a
 *                               multiple of num_kv_heads, unknown dtype,
 *                               `out` overlapping an input;
 *   MOBA_ERR_UNSUPPORTED        head_dim not 64 or 128; seqlen or block_size
 *                               not a multiple of 64; seqlen > 2^24; topk >
 *                               32 while topk < n; a pointer not 16-byte
 *                               aligned;
 *   MOBA_ERR_WORKSPACE_TOO_SMALL  workspace_bytes below moba_workspace_size;
 *   MOBA_ERR_HIP                a kernel launch was rejected.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_ABI_VERSION 1

/* The enums are int-sized.  In C++ they are declared with int as their
 * underlying type, so that any int a foreign caller passes (an unknown dtype,
 * an unknown status code) is a value of the type and is refused or named by
 * the library rather than being undefined behaviour inside it. */
#ifdef __cplusplus
#define MOBA_ENUM_BASE : int
#else
#define MOBA_ENUM_BASE
#endif

typedef enum moba_status_e MOBA_ENUM_BASE {
    MOBA_OK = 0,
    MOBA_ERR_INVALID_ARGUMENT = 1,
    MOBA_ERR_UNSUPPORTED = 2,
    MOBA_ERR_WORKSPACE_TOO_SMALL = 3,
    MOBA_ERR_HIP = 4
} moba_status_t;

typedef enum moba_dtype_e MOBA_ENUM_BASE { MOBA_DTYPE_BF16 = 0, MOBA_DTYPE_FP32 = 1 } moba_dtype_t;

/* Stages of moba_prefill, in launch order (for moba_prefill_timed). */
enum {
    MOBA_STAGE_POOL = 0,     /* block means of K                                  */
    MOBA_STAGE_GATE = 1,     /* gate scores + causal top-k                        */
    MOBA_STAGE_INDEX = 2,    /* per-(KV head, block) lists of the query rows      */
    MOBA_STAGE_ATTN_PAST = 3,/* attention of listed rows over one past block each */
    MOBA_STAGE_ATTN_OWN = 4, /* causal attention over each query's own block,
                                then the online-softmax merge of the partial
                                outputs                                           */
    MOBA_NUM_STAGES = 5
};

/* ABI version of the loaded library (MOBA_ABI_VERSION at build time). */
int moba_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *moba_status_string(moba_status_t status);

/*
 * Workspace bytes needed by moba_prefill (*prefill_bytes) and by moba_gate /
 * moba_pool (*gate_bytes) for this problem.  Either output pointer may be
 * NULL.  Host-only; validates like the calls it sizes.
 */
moba_status_t moba_workspace_size(int batch, int seqlen, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, int topk, moba_dtype_t dtype,
                                  size_t *prefill_bytes, size_t *gate_bytes);

/*
 * Block means of the keys: kbar[b][g][j][:] = mean of k[b][t][g][:] over the
 * tokens t of block j (block_size of them, fewer in a short last block),
 * accumulated in fp32 (the "aggregated
 * representation of the block keys" of the overview, section "技術細節與優勢").
 * Workspace: at least *gate_bytes of moba_workspace_size.
 */
moba_status_t moba_pool(const void *k, float *kbar, int batch, int seqlen, int num_kv_heads,
                        int head_dim, int block_size, moba_dtype_t dtype, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Gate and causal top-k (write-up, the first implementation step: assign
 * query tokens to KV blocks from the gate and the causal mask).  Writes
 * block_idx as laid out above.  Gate scores: fp32 inputs, fp32 inner products
 * of the query with the fp32 block means; bf16 inputs, the query against the
 * block means split into bf16 hi + lo parts on the matrix cores with fp32
 * accumulation (within about 2^-17 relative of the fp32 product).  Workspace:
 * at least *gate_bytes.
 */
moba_status_t moba_gate(const void *q, const void *k, int32_t *block_idx, int batch, int seqlen,
                        int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int topk, moba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * The gate scores that moba_gate ranks, for checking the gate's arithmetic:
 * scores[b][h][t][j] = q[b][t][h] . kbar[b][h / (Hq/Hkv)][j] for every past
 * block j < t / block_size (the gate of the write-up's first implementation
 * step, on the block means of the overview, section "技術細節與優勢"), NaN for
 * j >= t / block_size.  Computed as the bf16 gate computes them: per 16
 * dimensions the product with the bf16 hi part of the mean, then with the lo
 * part, into one fp32 accumulator.  bf16 only (fp32 inputs: UNSUPPORTED).
 * scores: [batch][num_q_heads][seqlen][n] fp32, n = ceil(seqlen / block_size),
 * 4-byte aligned, caller-owned, fully overwritten.  Workspace: at least
 * *gate_bytes of moba_workspace_size.  Errors as moba_gate.
 */
moba_status_t moba_gate_scores(const void *q, const void *k, float *scores, int batch, int seqlen,
                               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               moba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Whole MoBA causal prefill forward: out = softmax attention of each query
 * over the tokens t' <= t of its selected blocks.  topk >= n gives exact full
 * causal attention (no gating is run).
 * bf16 inputs: scores and softmax in fp32, P and V products in bf16 on the
 * matrix cores with fp32 accumulation, partial outputs kept in bf16, output
 * rounded to bf16 (nearest even).  fp32 inputs: fp32 throughout.
 * Workspace: at least *prefill_bytes.
 */
moba_status_t moba_prefill(const void *q, const void *k, const void *v, void *out, int batch,
                           int seqlen, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int topk, moba_dtype_t dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * moba_prefill that also records caller-created hipEvent_t handles on
 * `stream`: stage_events[s] just before stage s (MOBA_STAGE_*) and
 * stage_events[MOBA_NUM_STAGES] after the last stage; stages that a problem
 * does not need record back-to-back events.  With topk >= n the full causal
 * attention is timed as MOBA_STAGE_ATTN_PAST.  stage_events must hold
 * MOBA_NUM_STAGES + 1 valid events.
 */
moba_status_t moba_prefill_timed(const void *q, const void *k, const void *v, void *out,
                                 int batch, int seqlen, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int topk, moba_dtype_t dtype,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 void *const *stage_events);

/*
 * moba_prefill for sequences whose whole-sequence scratch does not fit: the
 * pool runs once, then the gate, index build, past-block attention, own-block
 * attention and merge run for the query tokens [c, c + query_chunk) of one
 * chunk at a time, reusing one chunk's scratch (the write-up's largest
 * context, 10M tokens, needs about 1 TB of partial outputs in one pass).  The
 * output is the same as moba_prefill's, bit for bit.  query_chunk: tokens per
 * chunk, a positive multiple of block_size (>= seqlen: one chunk).  Full
 * causal attention (topk >= n) needs no chunking and ignores it.  Errors as moba_prefill, plus INVALID_ARGUMENT for
 * query_chunk <= 0 and UNSUPPORTED for query_chunk % block_size != 0.
 */
moba_status_t moba_workspace_size_chunked(int batch, int seqlen, int num_q_heads,
                                          int num_kv_heads, int head_dim, int block_size,
                                          int topk, moba_dtype_t dtype, int query_chunk,
                                          size_t *prefill_bytes);
moba_status_t moba_prefill_chunked(const void *q, const void *k, const void *v, void *out,
                                   int batch, int seqlen, int num_q_heads, int num_kv_heads,
                                   int head_dim, int block_size, int topk, moba_dtype_t dtype,
                                   int query_chunk, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * Variable-length batch: packed sequences of different lengths, each an
 * independent MoBA prefill with its own blocks (the last one possibly short),
 * the setting of the write-up's variable-length FlashAttention step.
 * Sequence i holds tokens [cu_seqlens[i], cu_seqlens[i + 1]) of
 *   q, out  [total][num_q_heads][head_dim]
 *   k, v    [total][num_kv_heads][head_dim]     (total = cu_seqlens[num_seqs])
 * and attends only within itself.  cu_seqlens is a HOST array of num_seqs + 1
 * offsets, read during the call: cu_seqlens[0] = 0, non-decreasing, every
 * length a multiple of 64 (empty sequences are skipped).  The sequences run
 * one after another on `stream`, each over the whole GPU, sharing one
 * workspace; query_chunk is as in moba_prefill_chunked (per sequence).
 * Errors as moba_prefill_chunked, checked for every sequence before any HIP
 * call, plus INVALID_ARGUMENT for a null cu_seqlens, num_seqs <= 0,
 * cu_seqlens[0] != 0 or a decreasing offset, and UNSUPPORTED for a length
 * that is not a multiple of 64.
 */
moba_status_t moba_workspace_size_varlen(const int *cu_seqlens, int num_seqs, int num_q_heads,
                                         int num_kv_heads, int head_dim, int block_size,
                                         int topk, moba_dtype_t dtype, int query_chunk,
                                         size_t *prefill_bytes);
moba_status_t moba_prefill_varlen(const void *q, const void *k, const void *v, void *out,
                                  const int *cu_seqlens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int topk,
                                  moba_dtype_t dtype, int query_chunk, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * moba_prefill that also writes lse [batch][num_q_heads][seqlen] (fp32): for
 * every query row the natural log of its softmax normaliser, log sum over the
 * row's attended keys of exp(q.k / sqrt(head_dim)).  The backward pass reads
 * it.  Errors as moba_prefill, plus INVALID_ARGUMENT for a null lse or one
 * overlapping q or out, UNSUPPORTED for lse not 4-byte aligned.
 */
moba_status_t moba_prefill_lse(const void *q, const void *k, const void *v, void *out,
                               float *lse, int batch, int seqlen, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int topk,
                               moba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Backward pass: gradients dq, dk, dv of the attention for the upstream
 * gradient dout, under the selection the forward made (rebuilt here from q
 * and k: pool, gate, index, so it matches the forward's bit for bit).  The
 * write-up trains with MoBA; the selection itself gets no gradient (the top-k
 * is piecewise constant and the gate has no parameters).  With P the softmax
 * weights over a row's attended keys, dP = dout . v and delta = dout . out:
 *   dv = sum P dout,  dS = P (dP - delta),  dq = sum dS k / sqrt(d),
 *   dk = sum dS q / sqrt(d).
 * Inputs: q, k, v, out (the forward's output), dout as laid out above, lse
 * from moba_prefill_lse; outputs dq like q, dk and dv like k, fully
 * overwritten.  bf16 only: P and dS are rounded to bf16 for the matrix-core
 * products, accumulation is fp32, dq is summed from bf16 per-block partials.
 * Errors as moba_prefill, plus UNSUPPORTED for fp32 inputs and for topk >= n
 * with n > 32 blocks, INVALID_ARGUMENT for any output overlapping an input or
 * another output.  Workspace: moba_workspace_size_backward.
 */
moba_status_t moba_workspace_size_backward(int batch, int seqlen, int num_q_heads,
                                           int num_kv_heads, int head_dim, int block_size,
                                           int topk, moba_dtype_t dtype, size_t *bytes);
moba_status_t moba_backward(const void *q, const void *k, const void *v, const void *out,
                            const void *dout, const float *lse, void *dq, void *dk, void *dv,
                            int batch, int seqlen, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int topk, moba_dtype_t dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Allocation-free moba_prefill, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: its scratch is a fixed array of
 * MOBA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call itself allocates nothing (no hipMalloc,
 * no hipFree).  The output is moba_prefill's, bit for bit: the sparse stages
 * run in query chunks of the most blocks whose scratch fits (one pass when
 * the whole problem fits).  The GPU is the current device, and `stream` must
 * belong to it.  Every call on one GPU shares that GPU's scratch array and
 * leaves its contents behind (each call clears what it reads): calls that may
 * overlap on one GPU -- on different streams, or from different host
 * threads -- race and must be serialised by the caller.
 * Errors as moba_prefill, plus MOBA_ERR_WORKSPACE_TOO_SMALL when even one
 * block per query chunk needs more scratch than the array holds (at head_dim
 * 128, 32 query heads and top-k 12 that is a block size above 4096 tokens);
 * MOBA_ERR_HIP if the array's device address cannot be obtained.
 */
#define MOBA_NOALLOC_SCRATCH_BYTES (512ull << 20)
moba_status_t moba_prefill_noalloc(const void *q, const void *k, const void *v, void *out,
                                   int batch, int seqlen, int num_q_heads, int num_kv_heads,
                                   int head_dim, int block_size, int topk, moba_dtype_t dtype,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H */
