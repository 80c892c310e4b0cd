"""Bench: MoBA causal prefill on one MI355X.

One step = one whole moba_prefill (pool, gate + top-k, index build, past-
block attention, own-block attention, merge) over the resident synthetic
input of the 1M-token workload (batch 1, 32 query / 8 KV heads, d 128, bf16,
block 4096, top-k 12).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-dense] [--no-cpu] [--no-secondary] [--query-chunk T]

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
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoBA prefill tokens/s + attn TFLOP/s (% bf16 MFMA peak) at 128K and 1M tokens")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
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


def run_chunked(moba, torch, cfg, dev, args):
    """The 10M-token workload: one JSON line from the chunked prefill."""
    from synth import make_inputs
    log(f"{cfg.name}: generating inputs on the GPU in {cfg.gen_slice}-token slices")
    inp = make_inputs(cfg, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    torch.cuda.synchronize()
    log(f"{cfg.name}: inputs ready")
    ms, ms_ev, ws_bytes = time_prefill_chunked(moba, torch, cfg, q, k, v, args.steps,
                                               args.warmup, args.query_chunk)
    torch.cuda.empty_cache()
    w = work_counts(cfg)
    line = {
        "metric": METRIC,
        "value": cfg.batch * cfg.seqlen / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V with planted high-affinity blocks)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen,
                   "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "topk": cfg.topk,
                   "query_chunk": args.query_chunk, "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole chunked prefill (all stages, every chunk)",
                     "bound": "mfma", "achieved": w["flops_total"] / (ms_ev / 1000.0) / 1e12,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": w["flops_total"] / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                     "traffic": None, "avg_launch_ms": round(ms_ev, 3)},
        "workspace_gb": ws_bytes / 1e9,
        "selected_tflop": w["flops_total"] / 1e12,
    }
    if not args.no_dense:
        one = time_dense_one_head(moba, torch, cfg, q, k, v)
        est = one * cfg.hq * cfg.batch
        log(f"{cfg.name}: dense causal, one head {one:.1f} ms -> {est:.0f} ms for all heads")
        line["dense_causal_one_head_ms"] = round(one, 3)
        line["dense_causal_ms_scaled"] = round(est, 3)
        line["speedup_vs_dense"] = est / ms
        line["dense_tflops"] = w["flops_dense"] / (est / 1000.0) / 1e12
    print(json.dumps(line), flush=True)


def run_varlen(moba, torch, name, dev, args):
    """A packed variable-length batch: one JSON line from moba_prefill_varlen."""
    import dataclasses
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
    for i in range(args.warmup):
        call(base.topk)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        call(base.topk)
        ev[s][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ms_ev = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    seqs = [c for c in inp["configs"] if c is not None]
    flops = sum(work_counts(c)["flops_total"] for c in seqs)
    line = {
        "metric": METRIC,
        "value": total / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": base.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V with planted high-affinity blocks)",
        "config": {"workload": name, "total_tokens": total, "seq_lens": lengths,
                   "num_q_heads": base.hq, "num_kv_heads": base.hkv,
                   "head_dim": base.head_dim, "block_size": base.block_size,
                   "topk": base.topk, "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole varlen prefill (all stages, every sequence)",
                     "bound": "mfma", "achieved": flops / (ms_ev / 1000.0) / 1e12,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                     "traffic": None, "avg_launch_ms": round(ms_ev, 3)},
        "selected_tflop": flops / 1e12,
    }
    if not args.no_dense:
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
    print(json.dumps(line), flush=True)


def run_backward(moba, torch, cfg, dev, args):
    """moba_backward on the workload: one JSON line (whole backward per step)."""
    from synth import make_inputs
    log(f"{cfg.name}: generating inputs and upstream gradient on the GPU")
    inp = make_inputs(cfg, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 99)
    dout = (torch.randn(q.shape, generator=gen, device=dev) * 0.05).to(q.dtype)
    out, lse = moba.moba_prefill_lse(q, k, v, cfg.block_size, cfg.topk)
    nb = moba.moba_workspace_size_backward(cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim,
                                           cfg.block_size, cfg.topk)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        moba.moba_backward(q, k, v, out, dout, lse, cfg.block_size, cfg.topk, workspace=ws)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        moba.moba_backward(q, k, v, out, dout, lse, cfg.block_size, cfg.topk, workspace=ws)
        ev[s][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ms_ev = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    # algorithmic backward work: 5 products per attended pair (QK^T again, dO V^T,
    # P^T dO, dS K, dS^T Q), 2.5x the forward's 2
    flops = 2.5 * work_counts(cfg)["flops_total"]
    line = {
        "metric": "MoBA attention backward (dq, dk, dv) tokens/s",
        "value": cfg.batch * cfg.seqlen / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V/dO with planted high-affinity blocks)",
        "config": {"workload": cfg.name, "pass": "backward", "batch": cfg.batch,
                   "seq_len": cfg.seqlen, "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size, "topk": cfg.topk,
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole backward (selection rebuild, dq, dk/dv)", "bound": "mfma",
                     "achieved": flops / (ms_ev / 1000.0) / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": flops / (ms_ev / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                     "traffic": None, "avg_launch_ms": round(ms_ev, 3)},
        "backward_tflop": flops / 1e12,
        "workspace_gb": nb / 1e9,
    }
    print(json.dumps(line), flush=True)


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


def cpu_baseline(cfg, host, n_rows=8192, seed=5):
    """The fp64 oracle on the host cores: full pool, gate + attention on a
    random sample of query rows, extrapolated to the whole problem."""
    import numpy as np
    import oracle
    from synth import to_oracle_array
    qa, code = to_oracle_array(host["q"])
    ka, _ = to_oracle_array(host["k"])
    va, _ = to_oracle_array(host["v"])
    b, S, hq, hkv, d, B, k = (cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim,
                              cfg.block_size, cfg.topk)
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, b, n_rows), rng.integers(0, hq, n_rows),
                     rng.integers(0, S, n_rows)], axis=1).astype(np.int64)
    t0 = time.perf_counter()
    kbar = oracle.pool(ka, code, b, S, hkv, d, B)
    t1 = time.perf_counter()
    idx, _, _ = oracle.gate(qa, code, kbar, b, S, hq, hkv, d, B, k, rows)
    oracle.attend(qa, ka, va, code, b, S, hq, hkv, d, B, k, rows, idx)
    t2 = time.perf_counter()
    total_rows = b * hq * S
    est = (t1 - t0) + (t2 - t1) * total_rows / n_rows
    return {
        "value": b * S / est,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"full fp64 pool of K ({t1 - t0:.2f} s) + gate and attention of "
                   f"{n_rows} uniformly random query rows ({t2 - t1:.2f} s), extrapolated "
                   f"to all {total_rows} rows; {est:.0f} s estimated for the whole prefill"),
        "measured_s": round(t2 - t0, 3),
    }


def measure(moba, torch, cfg, dev, steps, warmup, dense, want_host):
    from synth import make_inputs
    log(f"{cfg.name}: generating inputs on the GPU")
    inp = make_inputs(cfg, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    torch.cuda.synchronize()
    ms, ms_ev, stages, _ = time_prefill(moba, torch, cfg, q, k, v, steps, warmup)
    log(f"{cfg.name}: {ms:.2f} ms/step; stages {stages}")
    res = {"ms": ms, "ms_events": ms_ev, "stages": stages}
    if dense:
        torch.cuda.empty_cache()
        res["dense_ms"] = time_dense(moba, torch, cfg, q, k, v)
        log(f"{cfg.name}: dense causal {res['dense_ms']:.1f} ms")
    host = {x: inp[x].cpu() for x in ("q", "k", "v")} if want_host else None
    del q, k, v, inp
    torch.cuda.empty_cache()
    return res, host


def summarize(cfg, res):
    w = work_counts(cfg)
    st = res["stages"]
    attn_ms = st["attn_past"] + st["attn_own_merge"]
    out = {
        "ms_per_step": round(res["ms"], 3),
        "tokens_per_s": cfg.batch * cfg.seqlen / (res["ms"] / 1000.0),
        "stages_ms": {k: round(v, 3) for k, v in st.items()},
        "selected_tflop": w["flops_total"] / 1e12,
        "attn_tflops": w["flops_total"] / (attn_ms / 1000.0) / 1e12,
        "attn_frac_bf16_peak": w["flops_total"] / (attn_ms / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
        "end_to_end_tflops": w["flops_total"] / (res["ms"] / 1000.0) / 1e12,
        "past_attn_tflops": w["flops_past"] / (st["attn_past"] / 1000.0) / 1e12
        if st["attn_past"] > 0 else None,
        "own_attn_merge_tflops": w["flops_own"] / (st["attn_own_merge"] / 1000.0) / 1e12,
        "pool_gbs": w["pool_bytes"] / (st["pool"] / 1000.0) / 1e9,
        "pool_frac_hbm_peak": w["pool_bytes"] / (st["pool"] / 1000.0) / 1e9 / HBM_PEAK_GBS,
        "gate_gbs": w["gate_bytes"] / (st["gate"] / 1000.0) / 1e9,
        "gate_frac_hbm_peak": w["gate_bytes"] / (st["gate"] / 1000.0) / 1e9 / HBM_PEAK_GBS,
    }
    if "dense_ms" in res:
        out["dense_causal_ms"] = round(res["dense_ms"], 3)
        out["speedup_vs_dense"] = res["dense_ms"] / res["ms"]
        out["dense_tflops"] = w["flops_dense"] / (res["dense_ms"] / 1000.0) / 1e12
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
    from synth import config_by_name
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
    from synth import VARLEN_WORKLOADS
    if args.workload in VARLEN_WORKLOADS:
        run_varlen(moba, torch, args.workload, dev, args)
        return
    cfg = config_by_name(args.workload)
    if args.backward:
        run_backward(moba, torch, cfg, dev, args)
        return
    if cfg.gen_slice > 0:
        run_chunked(moba, torch, cfg, dev, args)
        return
    res, host = measure(moba, torch, cfg, dev, args.steps, args.warmup, not args.no_dense,
                        not args.no_cpu)
    main_sum = summarize(cfg, res)
    w = work_counts(cfg)
    past_ms = res["stages"]["attn_past"]
    achieved = w["flops_past"] / (past_ms / 1000.0) / 1e12
    line = {
        "metric": METRIC,
        "value": main_sum["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_sum["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V with planted high-affinity blocks)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen,
                   "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "topk": cfg.topk, "parallelism": "single-gpu"},
        "roofline": {"kernel": "attn_bf16_kernel<128, 0, false> (past-block attention)",
                     "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": traffic_for(cfg.name),
                     "avg_launch_ms": round(past_ms, 3)},
    }
    line.update({k: v for k, v in main_sum.items() if k not in ("ms_per_step",)})
    if not args.no_cpu:
        log("timing the CPU oracle on a row sample")
        line["cpu_baseline"] = cpu_baseline(cfg, host)
    host = None
    if not args.no_secondary and args.workload == MAIN:
        cfg2 = config_by_name(SECONDARY)
        res2, _ = measure(moba, torch, cfg2, dev, args.steps, args.warmup, not args.no_dense,
                          False)
        line["secondary"] = {"workload": cfg2.name, **summarize(cfg2, res2)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
