"""Bench: MoBA causal prefill on one MI355X.

One step = one whole moba_prefill (pool, gate + top-k, index build, past-
block attention, own-block attention, merge) over the resident synthetic
input of the 1M-token workload (batch 1, 32 query / 8 KV heads, d 128, bf16,
block 4096, top-k 12).  Prints one JSON line: the 1M workload's figures at
the top level, the 128K workload under "secondary", and under "workloads"
the other synthetic workloads measured in the same run -- the 1K, 8K and 32K
workloads (each with the fp64 CPU oracle timed on the whole problem), the 1M
backward, the 10M-token query-chunked prefill and the packed ~1.09M-token
variable-length batch.  The CPU-oracle legs run in a background thread while
the GPU legs run.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-dense] [--no-cpu] [--no-secondary] [--no-extra]
                  [--query-chunk T]

--workload NAME, --backward: one JSON line for that workload (or its
backward) alone, as below.

--backward times moba_backward (dq, dk, dv; the selection rebuilt inside)
on the workload, after one moba_prefill_lse for its inputs.

--workload moba-varlen-1m-gqa32x8-d128 times a packed batch of 7 sequences
(about 1.09M tokens, every one ending in a short block) through
moba_prefill_varlen, whole steps timed with HIP events, and the same batch
with every block selected as its dense comparison.

--workload moba-10m-gqa32x8-d128 times the 10M-token prefill instead: the
sparse stages run over query chunks of T tokens (default 262144) with one
chunk's scratch (moba_prefill_chunked), each step timed whole with HIP events;
its dense comparison is timed on one query/KV head and scaled by the head
count (heads are independent), and it has no CPU-oracle leg.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoBA prefill tokens/s + attn TFLOP/s (% bf16 MFMA peak) at 128K and 1M tokens")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector (the fp32 path runs on the vector units)
MAIN = "moba-1m-gqa32x8-d128"
SECONDARY = "moba-128k-gqa32x8-d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_past_1m_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_moba_amd", "csrc", "attn.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def work_counts(cfg):
    """Algorithmic work of one prefill (selected-block pairs only; the last
    block holds S - (n - 1) B rows)."""
    B, n, k, d = cfg.block_size, cfg.n_blocks, cfg.topk, cfg.head_dim
    heads = cfg.hq * cfg.batch
    S = cfg.seqlen
    rows = [min(B, S - b * B) for b in range(n)]
    past_pairs = sum(r * B * min(b, k - 1) for b, r in enumerate(rows)) * heads
    own_pairs = sum(r * (r + 1) // 2 for r in rows) * heads
    esz = 2 if cfg.dtype == "bf16" else 4
    return {
        "flops_past": 4.0 * d * past_pairs,
        "flops_own": 4.0 * d * own_pairs,
        "flops_total": 4.0 * d * (past_pairs + own_pairs),
        "flops_dense": 4.0 * d * heads * S * (S + 1) / 2,
        "pool_bytes": cfg.batch * S * cfg.hkv * d * esz + cfg.batch * cfg.hkv * n * d * 4,
        "gate_bytes": (cfg.batch * S * cfg.hq * d * esz + cfg.batch * S * cfg.hq * k * 4
                       + cfg.batch * cfg.hkv * n * d * 4),
    }


def file_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(workload):
    """HBM bytes per launch of the past-block attention kernel from committed
    rocprofv3 counter runs, or None when absent or taken on other kernel code."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("attn_src_sha256") != file_hash(ATTN_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_prefill(moba, torch, cfg, q, k, v, steps, warmup):
    ws_bytes, _ = moba.moba_workspace_size(cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv,
                                           cfg.head_dim, cfg.block_size, cfg.topk,
                                           moba.MOBA_DTYPE_BF16 if cfg.dtype == "bf16"
                                           else moba.MOBA_DTYPE_FP32)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    for i in range(warmup):
        moba.moba_prefill(q, k, v, cfg.block_size, cfg.topk, out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{warmup} done")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(moba.MOBA_NUM_STAGES + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        moba.moba_prefill(q, k, v, cfg.block_size, cfg.topk, out=out, workspace=ws,
                          stage_events=ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = [0.0] * moba.MOBA_NUM_STAGES
    for s in range(steps):
        for i in range(moba.MOBA_NUM_STAGES):
            stage_ms[i] += ev[s][i].elapsed_time(ev[s][i + 1]) / steps
    total_ev = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)) / steps
    del ws
    return wall * 1000.0 / steps, total_ev, dict(zip(moba.STAGE_NAMES, stage_ms)), out


def time_prefill_cold(moba, torch, cfg, q, k, v, reps=5):
    """Median of reps prefills, each after 1 GiB of writes that evict the
    inputs from the 256 MB last-level cache (small workloads fit in it), ms."""
    ws_bytes, _ = moba.moba_workspace_size(cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv,
                                           cfg.head_dim, cfg.block_size, cfg.topk,
                                           moba.MOBA_DTYPE_BF16 if cfg.dtype == "bf16"
                                           else moba.MOBA_DTYPE_FP32)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.device)
    times = []
    for r in range(reps):
        flush.fill_(r & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moba.moba_prefill(q, k, v, cfg.block_size, cfg.topk, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del ws, out, flush
    return sorted(times)[reps // 2]


def time_prefill_chunked(moba, torch, cfg, q, k, v, steps, warmup, chunk):
    """Whole-step HIP-event timing of the query-chunked prefill."""
    ws_bytes = moba.moba_workspace_size_chunked(cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv,
                                                cfg.head_dim, cfg.block_size, cfg.topk, chunk)
    log(f"chunked workspace {ws_bytes / 1e9:.2f} GB for {chunk}-token query chunks")
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    for i in range(warmup):
        moba.moba_prefill(q, k, v, cfg.block_size, cfg.topk, out=out, workspace=ws,
                          query_chunk=chunk)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        moba.moba_prefill(q, k, v, cfg.block_size, cfg.topk, out=out, workspace=ws,
                          query_chunk=chunk)
        ev[s][1].record()
        torch.cuda.synchronize()
        log(f"step {s + 1}/{steps}: {ev[s][0].elapsed_time(ev[s][1]):.1f} ms")
    wall = time.perf_counter() - t0
    total_ev = sum(a.elapsed_time(b) for a, b in ev) / steps
    del ws, out
    return wall * 1000.0 / steps, total_ev, ws_bytes


def time_dense_one_head(moba, torch, cfg, q, k, v):
    """Full causal attention of query head 0 over KV head 0 (one launch), ms."""
    q1, k1, v1 = (x[:, :, :1].contiguous() for x in (q, k, v))
    out = torch.empty_like(q1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    moba.moba_prefill(q1, k1, v1, cfg.block_size, cfg.n_blocks, out=out)
    e1.record()
    torch.cuda.synchronize()
    del q1, k1, v1, out
    return e0.elapsed_time(e1)


def base_line(metric, value, steps, warmup, ms, dtype, config, data=None):
    return {
        "metric": metric,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": data or "synthetic (seeded Gaussian Q/K/V with planted high-affinity blocks)",
        "config": config,
    }


def cfg_config(cfg, **extra):
    c = {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen,
         "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv, "head_dim": cfg.head_dim,
         "block_size": cfg.block_size, "topk": cfg.topk}
    c.update(extra)
    c["parallelism"] = "single-gpu"
    return c


def run_chunked(moba, torch, cfg, dev, steps, warmup, query_chunk, dense):
    """The 10M-token workload through the query-chunked prefill: a JSON-line dict."""
    from synth import make_inputs
    log(f"{cfg.name}: generating inputs on the GPU in {cfg.gen_slice}-token slices")
    inp = make_inputs(cfg, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    torch.cuda.synchronize()
    log(f"{cfg.name}: inputs ready")
    ms, ms_ev, ws_bytes = time_prefill_chunked(moba, torch, cfg, q, k, v, steps, warmup,
                                               query_chunk)
    torch.cuda.empty_cache()
    w = work_counts(cfg)
    line = base_line(METRIC, cfg.batch * cfg.seqlen / (ms / 1000.0), steps, warmup, ms, cfg.dtype,
                     cfg_config(cfg, query_chunk=query_chunk))
    line["roofline"] = {"kernel": "whole chunked prefill (all stages, every chunk)",
                        "bound": "mfma", "achieved": w["flops_total"] / (ms_ev / 1000.0) / 1e12,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": w["flops_total"] / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                        "traffic": None, "avg_launch_ms": round(ms_ev, 3)}
    line["workspace_gb"] = ws_bytes / 1e9
    line["selected_tflop"] = w["flops_total"] / 1e12
    if dense:
        one = time_dense_one_head(moba, torch, cfg, q, k, v)
        est = one * cfg.hq * cfg.batch
        log(f"{cfg.name}: dense causal, one head {one:.1f} ms -> {est:.0f} ms for all heads")
        line["dense_causal_one_head_ms"] = round(one, 3)
        line["dense_causal_ms_scaled"] = round(est, 3)
        line["speedup_vs_dense"] = est / ms
        line["dense_tflops"] = w["flops_dense"] / (est / 1000.0) / 1e12
    del q, k, v, inp
    torch.cuda.empty_cache()
    return line


def run_varlen(moba, torch, name, dev, steps, warmup, dense):
    """A packed variable-length batch through moba_prefill_varlen: a JSON-line dict."""
    from synth import VARLEN_WORKLOADS, make_varlen_inputs
    base, lengths = VARLEN_WORKLOADS[name]
    log(f"{name}: generating {len(lengths)} sequences on the GPU")
    inp = make_varlen_inputs(base, lengths, device=dev)
    q, k, v, cu = inp["q"], inp["k"], inp["v"], inp["cu_seqlens"]
    total = cu[-1]
    chunk = -(-max(lengths) // base.block_size) * base.block_size
    ws_bytes = moba.moba_workspace_size_varlen(cu, base.hq, base.hkv, base.head_dim,
                                               base.block_size, base.topk, chunk)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    call = lambda topk: moba.moba_prefill_varlen(q, k, v, cu, base.block_size, topk, out=out,
                                                 workspace=ws, query_chunk=chunk)
    for i in range(warmup):
        call(base.topk)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        call(base.topk)
        ev[s][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    ms_ev = sum(a.elapsed_time(b) for a, b in ev) / steps
    seqs = [c for c in inp["configs"] if c is not None]
    flops = sum(work_counts(c)["flops_total"] for c in seqs)
    line = base_line(METRIC, total / (ms / 1000.0), steps, warmup, ms, base.dtype,
                     {"workload": name, "total_tokens": total, "seq_lens": lengths,
                      "num_q_heads": base.hq, "num_kv_heads": base.hkv,
                      "head_dim": base.head_dim, "block_size": base.block_size,
                      "topk": base.topk, "parallelism": "single-gpu"})
    line["roofline"] = {"kernel": "whole varlen prefill (all stages, every sequence)",
                        "bound": "mfma", "achieved": flops / (ms_ev / 1000.0) / 1e12,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": flops / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                        "traffic": None, "avg_launch_ms": round(ms_ev, 3)}
    line["selected_tflop"] = flops / 1e12
    if dense:
        dense_topk = max(c.n_blocks for c in seqs)
        call(dense_topk)                              # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        call(dense_topk)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1)
        log(f"{name}: dense causal {dense_ms:.1f} ms")
        line["dense_causal_ms"] = round(dense_ms, 3)
        line["speedup_vs_dense"] = dense_ms / ms
    del q, k, v, ws, out, inp
    torch.cuda.empty_cache()
    return line


def run_backward(moba, torch, cfg, dev, steps, warmup, inputs=None):
    """moba_backward on the workload (whole backward per step): a JSON-line dict."""
    if inputs is None:
        from synth import make_inputs
        log(f"{cfg.name}: generating inputs on the GPU")
        inputs = make_inputs(cfg, device=dev)
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    log(f"{cfg.name}: upstream gradient and forward log-sum-exp for the backward")
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 99)
    dout = (torch.randn(q.shape, generator=gen, device=dev) * 0.05).to(q.dtype)
    out, lse = moba.moba_prefill_lse(q, k, v, cfg.block_size, cfg.topk)
    nb = moba.moba_workspace_size_backward(cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim,
                                           cfg.block_size, cfg.topk)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    for i in range(warmup):
        moba.moba_backward(q, k, v, out, dout, lse, cfg.block_size, cfg.topk, workspace=ws)
        torch.cuda.synchronize()
        log(f"backward warmup {i + 1}/{warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        moba.moba_backward(q, k, v, out, dout, lse, cfg.block_size, cfg.topk, workspace=ws)
        ev[s][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    ms_ev = sum(a.elapsed_time(b) for a, b in ev) / steps
    log(f"{cfg.name}: backward {ms:.1f} ms/step")
    # algorithmic backward work: 5 products per attended pair (QK^T again, dO V^T,
    # P^T dO, dS K, dS^T Q), 2.5x the forward's 2
    flops = 2.5 * work_counts(cfg)["flops_total"]
    line = base_line("MoBA attention backward (dq, dk, dv) tokens/s",
                     cfg.batch * cfg.seqlen / (ms / 1000.0), steps, warmup, ms, cfg.dtype,
                     cfg_config(cfg, **{"pass": "backward"}),
                     "synthetic (seeded Gaussian Q/K/V/dO with planted high-affinity blocks)")
    line["roofline"] = {"kernel": "whole backward (selection rebuild, dq, dk/dv)", "bound": "mfma",
                        "achieved": flops / (ms_ev / 1000.0) / 1e12, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s",
                        "frac": flops / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                        "traffic": None, "avg_launch_ms": round(ms_ev, 3)}
    line["backward_tflop"] = flops / 1e12
    line["workspace_gb"] = nb / 1e9
    del ws, out, lse, dout
    torch.cuda.empty_cache()
    return line


def time_dense(moba, torch, cfg, q, k, v):
    """Full causal attention on the same inputs (topk = number of blocks)."""
    out = torch.empty_like(q)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moba.moba_prefill(q, k, v, cfg.block_size, cfg.n_blocks, out=out)     # warm-up
    torch.cuda.synchronize()
    e0.record()
    moba.moba_prefill(q, k, v, cfg.block_size, cfg.n_blocks, out=out)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def row_work(cfg, rows):
    """(scored past blocks, attended (query, key) pairs) of the rows [R, 3] (b, h, t)."""
    import numpy as np
    t = rows[:, 2].astype(np.int64)
    own = t // cfg.block_size
    past = np.minimum(own, cfg.topk - 1)
    return int(own.sum()), int((t - own * cfg.block_size + 1).sum() + (past * cfg.block_size).sum())


def total_work(cfg):
    """(scored past blocks, attended pairs) of the whole problem."""
    B, S = cfg.block_size, cfg.seqlen
    scored = sum(min(B, S - j * B) * j for j in range(cfg.n_blocks))
    w = work_counts(cfg)
    pairs = (w["flops_total"] / (4.0 * cfg.head_dim))
    return scored * cfg.hq * cfg.batch, int(round(pairs))


def cpu_prepare(cfg, host, mode):
    """Host-side inputs of one CPU-oracle leg: the oracle's views of Q, K and V
    and the row sets.  Built on the calling thread, between GPU timings, so
    that the leg's own thread runs only oracle calls (which release the
    interpreter lock) and never holds up the launches of a timed region."""
    import numpy as np
    import oracle
    from synth import sample_rows, to_oracle_array
    qa, code = to_oracle_array(host["q"])
    ka, _ = to_oracle_array(host["k"])
    va, _ = to_oracle_array(host["v"])
    b, S, hq, hkv = cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv
    # 8192 random rows on top of the strata (about 13K rows at 128K and 1M):
    # a few hundred rows leave the oracle's per-call costs in the extrapolation
    n_random = 8192
    if mode == "full":
        sample = gate_rows = oracle.all_rows(b, hq, S)
    else:
        sample = sample_rows(cfg, tile=32, n_random=n_random)
        if mode == "group":
            # every row of the first KV group's query heads, and the sample rows,
            # in (b, h, t) order without repeats
            key = lambda r: (r[:, 0] * hq + r[:, 1]) * S + r[:, 2]
            keys = np.unique(np.concatenate([key(oracle.all_rows(b, hq // hkv, S)), key(sample)]))
            gate_rows = np.stack([keys // (hq * S), (keys // S) % hq, keys % S], axis=1)
        else:
            gate_rows = oracle.all_rows(b, hq, S)
    # where each sample row sits among the gate rows (both in (b, h, t) order)
    key = lambda r: (r[:, 0] * hq + r[:, 1]) * S + r[:, 2]
    pos = None if mode == "full" else np.searchsorted(key(gate_rows), key(sample))
    return {"qa": qa, "ka": ka, "va": va, "code": code, "sample": sample, "gate_rows": gate_rows,
            "sample_pos": pos, "scored_g": row_work(cfg, gate_rows)[0],
            "pairs_s": row_work(cfg, sample)[1]}


def cpu_baseline(cfg, prep, mode):
    """The fp64 oracle as it stands on the host cores, timed on one workload.

    mode "full": pool, gate and attention of every row.
    mode "gate": pool and gate of every row, attention of the stratified row
      sample (whole 32-row tiles of blocks 0, k-1, k, a middle and the last
      block of every head, plus 8192 random rows), extrapolated by attended
      (query, key) pairs.
    mode "group": pool of every block; the gate of every row of the first KV
      group's query heads plus the sample rows, extrapolated by scored blocks
      (the groups are alike: the same rows, the same block counts); attention
      of the same row sample, extrapolated by attended pairs.  Sized for 10-30 s
      of oracle time on 16 cores at 1M, where the full gate alone takes about
      30 s (3.6 s per KV group) and would bring the leg to about 45 s.
    """
    import oracle
    qa, ka, va, code = prep["qa"], prep["ka"], prep["va"], prep["code"]
    sample, gate_rows = prep["sample"], prep["gate_rows"]
    b, S, hq, hkv, d, B, k = (cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim,
                              cfg.block_size, cfg.topk)
    t0 = time.perf_counter()
    kbar = oracle.pool(ka, code, b, S, hkv, d, B)
    t1 = time.perf_counter()
    idx, _, _ = oracle.gate(qa, code, kbar, b, S, hq, hkv, d, B, k, gate_rows)
    t2 = time.perf_counter()
    idx_s = idx if mode == "full" else idx[prep["sample_pos"]]
    oracle.attend(qa, ka, va, code, b, S, hq, hkv, d, B, k, sample, idx_s)
    t3 = time.perf_counter()
    scored_all, pairs_all = total_work(cfg)
    scored_g, pairs_s = prep["scored_g"], prep["pairs_s"]
    t_gate = (t2 - t1) * scored_all / max(scored_g, 1)
    t_attn = (t3 - t2) if mode == "full" else (t3 - t2) * pairs_all / max(pairs_s, 1)
    est = (t1 - t0) + t_gate + t_attn
    what = {"full": "every row: pool, gate and attention",
            "gate": (f"pool and gate of every row ({t2 - t0:.2f} s); attention of {len(sample)} "
                     f"stratified rows ({t3 - t2:.2f} s) extrapolated by attended pairs"),
            "group": (f"pool of every block ({t1 - t0:.2f} s); gate of {len(gate_rows)} rows (every "
                      f"row of the first KV group's heads and the sample rows; {t2 - t1:.2f} s) "
                      f"extrapolated by scored blocks; attention of {len(sample)} stratified rows "
                      f"({t3 - t2:.2f} s) extrapolated by attended pairs")}[mode]
    return {
        "value": b * S / est,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{what}; {est:.1f} s for the whole prefill" + (
            " (measured)" if mode == "full" else " (extrapolated)"),
        "measured_s": round(t3 - t0, 3),
    }


class CpuLegs:
    """Runs the CPU-oracle legs one after another in a background thread (the
    oracle is a C library: its calls release the interpreter lock)."""

    def __init__(self):
        self.jobs, self.results, self.errors = [], {}, {}
        self.lock = threading.Lock()
        self.thread = None

    def add(self, key, cfg, host, mode):
        try:
            prep = cpu_prepare(cfg, host, mode)       # on this thread, between GPU timings
        except Exception as e:                         # reported in the line, never fatal
            self.errors[key] = repr(e)
            return
        with self.lock:
            self.jobs.append((key, cfg, prep, mode))
        if self.thread is None:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()

    def _run(self):
        while True:
            with self.lock:
                if not self.jobs:
                    self.thread = None
                    return
                key, cfg, prep, mode = self.jobs.pop(0)
            try:
                log(f"cpu oracle: {key} ({mode}) started")
                self.results[key] = cpu_baseline(cfg, prep, mode)
                log(f"cpu oracle: {key} done in {self.results[key]['measured_s']:.1f} s")
            except Exception as e:                     # reported in the line, never fatal
                self.errors[key] = repr(e)

    def join(self):
        while True:
            with self.lock:
                t = self.thread
            if t is None:
                return
            t.join()


def measure(moba, torch, cfg, dev, steps, warmup, dense, want_host, keep_gpu=False):
    from synth import make_inputs
    on_gpu = cfg.seqlen >= 1 << 17
    log(f"{cfg.name}: generating inputs on the {'GPU' if on_gpu else 'host'}")
    inp = make_inputs(cfg, device=dev) if on_gpu else make_inputs(cfg)
    host = {x: inp[x] for x in ("q", "k", "v")} if not on_gpu else None
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    torch.cuda.synchronize()
    if want_host and host is None:
        host = {x: inp[x].cpu() for x in ("q", "k", "v")}
    ms, ms_ev, stages, _ = time_prefill(moba, torch, cfg, q, k, v, steps, warmup)
    log(f"{cfg.name}: {ms:.2f} ms/step; stages {stages}")
    res = {"ms": ms, "ms_events": ms_ev, "stages": stages}
    if not on_gpu:
        res["cold_ms"] = time_prefill_cold(moba, torch, cfg, q, k, v)
        log(f"{cfg.name}: {res['cold_ms']:.3f} ms cold (median of 5)")
    if dense:
        torch.cuda.empty_cache()
        res["dense_ms"] = time_dense(moba, torch, cfg, q, k, v)
        log(f"{cfg.name}: dense causal {res['dense_ms']:.1f} ms")
    gpu = {"q": q, "k": k, "v": v} if keep_gpu else None
    del q, k, v, inp
    torch.cuda.empty_cache()
    return res, (host if want_host else None), gpu


def summarize(cfg, res):
    w = work_counts(cfg)
    st = res["stages"]
    attn_ms = st["attn_past"] + st["attn_own_merge"]
    peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    out = {
        "ms_per_step": round(res["ms"], 3),
        "tokens_per_s": cfg.batch * cfg.seqlen / (res["ms"] / 1000.0),
        "stages_ms": {k: round(v, 3) for k, v in st.items()},
        "selected_tflop": w["flops_total"] / 1e12,
        "attn_tflops": w["flops_total"] / (attn_ms / 1000.0) / 1e12,
        "attn_frac_bf16_peak" if cfg.dtype == "bf16" else "attn_frac_fp32_peak":
            w["flops_total"] / (attn_ms / 1000.0) / 1e12 / peak,
        "end_to_end_tflops": w["flops_total"] / (res["ms"] / 1000.0) / 1e12,
        "past_attn_tflops": w["flops_past"] / (st["attn_past"] / 1000.0) / 1e12
        if st["attn_past"] > 0 else None,
        "own_attn_merge_tflops": w["flops_own"] / (st["attn_own_merge"] / 1000.0) / 1e12,
        "pool_gbs": w["pool_bytes"] / (st["pool"] / 1000.0) / 1e9,
        "pool_frac_hbm_peak": w["pool_bytes"] / (st["pool"] / 1000.0) / 1e9 / HBM_PEAK_GBS,
        "gate_gbs": w["gate_bytes"] / (st["gate"] / 1000.0) / 1e9,
        "gate_frac_hbm_peak": w["gate_bytes"] / (st["gate"] / 1000.0) / 1e9 / HBM_PEAK_GBS,
    }
    if "cold_ms" in res:
        out["ms_per_step_cold"] = round(res["cold_ms"], 3)
        out["tokens_per_s_cold"] = cfg.batch * cfg.seqlen / (res["cold_ms"] / 1000.0)
    if "dense_ms" in res:
        out["dense_causal_ms"] = round(res["dense_ms"], 3)
        out["speedup_vs_dense"] = res["dense_ms"] / res["ms"]
        out["dense_tflops"] = w["flops_dense"] / (res["dense_ms"] / 1000.0) / 1e12
        if st["attn_past"] > 0:
            # dense causal at the past-block kernel's FLOP rate: the speed-up
            # that comes from skipping work, not from a slower dense kernel
            rate = w["flops_past"] / (st["attn_past"] / 1000.0)
            out["speedup_at_equal_efficiency"] = (w["flops_dense"] / rate * 1000.0) / res["ms"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=MAIN)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (small configs, backward, 10M, packed batch)")
    ap.add_argument("--backward", action="store_true",
                    help="time moba_backward (dq, dk, dv) on the workload instead")
    ap.add_argument("--query-chunk", type=int, default=1 << 18,
                    help="query tokens per chunk for workloads generated in slices (10M)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the prefill shards by KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_moba_amd as moba
    from synth import CONFIGS, VARLEN_WORKLOADS, config_by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4,
                          "launches": 3}), flush=True)
        return
    if args.workload in VARLEN_WORKLOADS:
        print(json.dumps(run_varlen(moba, torch, args.workload, dev, args.steps, args.warmup,
                                    not args.no_dense)), flush=True)
        return
    cfg = config_by_name(args.workload)
    if args.backward:
        print(json.dumps(run_backward(moba, torch, cfg, dev, args.steps, args.warmup)), flush=True)
        return
    if cfg.gen_slice > 0:
        print(json.dumps(run_chunked(moba, torch, cfg, dev, args.steps, args.warmup,
                                     args.query_chunk, not args.no_dense)), flush=True)
        return

    full_run = args.workload == MAIN and not args.no_extra
    cpu = CpuLegs()
    extra = {}
    if full_run:
        # the small workloads first, before the CPU legs load the host cores
        for small in CONFIGS[:3]:
            r, h, _ = measure(moba, torch, small, dev, max(args.steps, 5), args.warmup,
                              not args.no_dense, not args.no_cpu)
            extra[small.name] = summarize(small, r)
            if not args.no_cpu:
                cpu.add(small.name, small, h, "full")
    want_secondary = not args.no_secondary and args.workload == MAIN
    if want_secondary:
        cfg2 = config_by_name(SECONDARY)
        res2, host2, _ = measure(moba, torch, cfg2, dev, args.steps, args.warmup,
                                 not args.no_dense, not args.no_cpu)
        if not args.no_cpu:
            cpu.add(cfg2.name, cfg2, host2, "gate")
        host2 = None
    res, host, gpu_in = measure(moba, torch, cfg, dev, args.steps, args.warmup,
                                not args.no_dense, not args.no_cpu, keep_gpu=full_run)
    if not args.no_cpu:
        cpu.add(cfg.name, cfg, host, "group")
    host = None
    main_sum = summarize(cfg, res)
    w = work_counts(cfg)
    past_ms = res["stages"]["attn_past"]
    achieved = w["flops_past"] / (past_ms / 1000.0) / 1e12
    line = base_line(METRIC, main_sum["tokens_per_s"], args.steps, args.warmup,
                     main_sum["ms_per_step"], cfg.dtype, cfg_config(cfg))
    line["roofline"] = {"kernel": "attn_bf16_kernel<128, 0, false> (past-block attention)",
                        "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                        "traffic": traffic_for(cfg.name),
                        "avg_launch_ms": round(past_ms, 3)}
    line.update({k: v for k, v in main_sum.items() if k not in ("ms_per_step",)})
    if want_secondary:
        line["secondary"] = {"workload": cfg2.name, **summarize(cfg2, res2)}
    if full_run:
        bw = run_backward(moba, torch, cfg, dev, 3, 1, inputs=gpu_in)
        gpu_in = None
        torch.cuda.empty_cache()
        extra[cfg.name + "/backward"] = bw
        vname = next(iter(VARLEN_WORKLOADS))
        extra[vname] = run_varlen(moba, torch, vname, dev, 3, 1, not args.no_dense)
        big = config_by_name("moba-10m-gqa32x8-d128")
        extra[big.name] = run_chunked(moba, torch, big, dev, 2, 1, args.query_chunk, False)
    gpu_in = None
    if not args.no_cpu:
        log("waiting for the CPU-oracle legs")
        cpu.join()
        line["cpu_baseline"] = cpu.results.get(cfg.name, {"error": cpu.errors.get(cfg.name)})
        if want_secondary:
            line["secondary"]["cpu_baseline"] = cpu.results.get(
                cfg2.name, {"error": cpu.errors.get(cfg2.name)})
        for name in list(extra):
            if name in cpu.results:
                extra[name]["cpu_baseline"] = cpu.results[name]
            elif name in cpu.errors:
                extra[name]["cpu_baseline"] = {"error": cpu.errors[name]}
    if extra:
        line["workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
