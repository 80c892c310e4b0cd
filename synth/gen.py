"""Seeded generator for MoBA prefill inputs.

Recipe (one reading of the workload text; every choice is listed in the design
notes):
  * Q, K, V elements are i.i.d. N(0, 1) / sqrt(d), drawn in fp32 from a torch
    generator seeded with the config seed on the target device.
  * Per (batch, KV head) ``planted`` distinct blocks are drawn from
    {0 .. n-2} (so later queries exist).  Each planted block p gets its own
    random unit vector u_p; every key of block p gets ``+= 2 * u_p``; for each
    query head of that KV head's group and every token in a block strictly
    after p, independently with probability ``shift_prob``, ``q += u_p``.
  * Finally the tensors are rounded to the storage dtype (bf16 by
    round-to-nearest-even via torch's cast) or kept fp32.
  * Workloads with ``gen_slice`` > 0 (10M tokens) follow the same recipe one
    token slice [s*T, (s+1)*T) at a time: each slice draws its Q, K, V and
    shift masks from its own torch generator seeded ``seed * 65536 + s``, the
    planted blocks and directions come from the same NumPy draws as above, and
    each slice is rounded into the preallocated storage-dtype tensors.

Layouts are BSHD: q is [batch, S, Hq, d]; k and v are [batch, S, Hkv, d].
"""
import math

import numpy as np
import torch

from .configs import Config


def make_inputs(cfg: Config, device="cpu", seed=None):
    """Return dict(q, k, v, planted) for ``cfg`` on ``device``.

    ``planted`` is an int array [batch, hkv, planted] of the planted block ids.
    Values depend on the device's torch generator: tensors made on the GPU are
    copied back to the host when the oracle needs them.
    """
    seed = cfg.seed if seed is None else seed
    if cfg.gen_slice > 0:
        return _make_sliced(cfg, torch.device(device), seed)
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    bsz, S, hq, hkv, d = cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim
    B = cfg.block_size
    n = cfg.n_blocks
    G = hq // hkv
    inv = 1.0 / math.sqrt(d)

    q = torch.randn((bsz, S, hq, d), generator=g, device=dev, dtype=torch.float32).mul_(inv)
    k = torch.randn((bsz, S, hkv, d), generator=g, device=dev, dtype=torch.float32).mul_(inv)
    v = torch.randn((bsz, S, hkv, d), generator=g, device=dev, dtype=torch.float32).mul_(inv)

    rng = np.random.Generator(np.random.PCG64(seed))
    P = min(cfg.planted, max(n - 1, 0))
    planted = np.zeros((bsz, hkv, P), dtype=np.int64)
    for b in range(bsz):
        for gk in range(hkv):
            blocks = np.sort(rng.choice(n - 1, size=P, replace=False)) if P > 0 else []
            planted[b, gk, :] = blocks
            for p in blocks:
                u = rng.standard_normal(d)
                u /= np.linalg.norm(u)
                ut = torch.tensor(u, dtype=torch.float32, device=dev)
                k[b, p * B:min((p + 1) * B, S), gk, :] += 2.0 * ut
                start = (p + 1) * B
                if start >= S:
                    continue
                for hh in range(G):
                    h = gk * G + hh
                    m = torch.rand((S - start,), generator=g, device=dev) < cfg.shift_prob
                    q[b, start:, h, :].addcmul_(m.to(torch.float32)[:, None], ut[None, :])

    if cfg.dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    elif cfg.dtype != "fp32":
        raise ValueError(cfg.dtype)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(), "planted": planted}


def _plant_plan(cfg: Config, rng, P):
    """Planted block ids [batch, hkv, P] and their unit directions, NumPy draws
    in the order of the unsliced recipe."""
    n, d = cfg.n_blocks, cfg.head_dim
    planted = np.zeros((cfg.batch, cfg.hkv, P), dtype=np.int64)
    dirs = {}
    for b in range(cfg.batch):
        for gk in range(cfg.hkv):
            blocks = np.sort(rng.choice(n - 1, size=P, replace=False)) if P > 0 else []
            planted[b, gk, :] = blocks
            for p in blocks:
                u = rng.standard_normal(d)
                dirs[(b, gk, int(p))] = u / np.linalg.norm(u)
    return planted, dirs


def _make_sliced(cfg: Config, dev, seed):
    bsz, S, hq, hkv, d = cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim
    B, T, G = cfg.block_size, cfg.gen_slice, hq // hkv
    inv = 1.0 / math.sqrt(d)
    if cfg.dtype == "bf16":
        dt = torch.bfloat16
    elif cfg.dtype == "fp32":
        dt = torch.float32
    else:
        raise ValueError(cfg.dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    P = min(cfg.planted, max(cfg.n_blocks - 1, 0))
    planted, dirs = _plant_plan(cfg, rng, P)
    units = {key: torch.tensor(u, dtype=torch.float32, device=dev) for key, u in dirs.items()}
    q = torch.empty((bsz, S, hq, d), dtype=dt, device=dev)
    k = torch.empty((bsz, S, hkv, d), dtype=dt, device=dev)
    v = torch.empty((bsz, S, hkv, d), dtype=dt, device=dev)
    for s, t0 in enumerate(range(0, S, T)):
        t1 = min(S, t0 + T)
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 65536 + s)
        qs = torch.randn((bsz, t1 - t0, hq, d), generator=g, device=dev,
                         dtype=torch.float32).mul_(inv)
        ks = torch.randn((bsz, t1 - t0, hkv, d), generator=g, device=dev,
                         dtype=torch.float32).mul_(inv)
        vs = torch.randn((bsz, t1 - t0, hkv, d), generator=g, device=dev,
                         dtype=torch.float32).mul_(inv)
        for b in range(bsz):
            for gk in range(hkv):
                for p in planted[b, gk, :].tolist():
                    ut = units[(b, gk, p)]
                    k0, k1 = max(p * B, t0), min((p + 1) * B, t1)
                    if k0 < k1:
                        ks[b, k0 - t0:k1 - t0, gk, :] += 2.0 * ut
                    start = max((p + 1) * B, t0)
                    if start >= t1:
                        continue
                    for hh in range(G):
                        h = gk * G + hh
                        m = torch.rand((t1 - start,), generator=g, device=dev) < cfg.shift_prob
                        qs[b, start - t0:, h, :].addcmul_(m.to(torch.float32)[:, None],
                                                          ut[None, :])
        q[:, t0:t1].copy_(qs)
        k[:, t0:t1].copy_(ks)
        v[:, t0:t1].copy_(vs)
        del qs, ks, vs
    return {"q": q, "k": k, "v": v, "planted": planted}


def make_varlen_inputs(cfg: Config, lengths, device="cpu"):
    """Packed sequences for the variable-length prefill.

    Sequence i follows ``cfg``'s recipe with seqlen = lengths[i], batch 1 and
    seed cfg.seed + 7919 * i; the sequences are concatenated along the token
    axis.  Returns dict(q [T, hq, d], k, v [T, hkv, d], cu_seqlens list [n + 1],
    configs: the per-sequence Config, None for an empty sequence).
    """
    import dataclasses
    qs, ks, vs, cfgs, cu = [], [], [], [], [0]
    for i, n in enumerate(lengths):
        cu.append(cu[-1] + n)
        if n == 0:
            cfgs.append(None)
            continue
        c = dataclasses.replace(cfg, batch=1, seqlen=n, seed=cfg.seed + 7919 * i)
        inp = make_inputs(c, device=device)
        qs.append(inp["q"][0])
        ks.append(inp["k"][0])
        vs.append(inp["v"][0])
        cfgs.append(c)
    return {"q": torch.cat(qs).contiguous(), "k": torch.cat(ks).contiguous(),
            "v": torch.cat(vs).contiguous(), "cu_seqlens": cu, "configs": cfgs}


def to_oracle_array(t: torch.Tensor):
    """Host numpy view of a bf16 / fp32 tensor as raw storage: (array, code).

    code 0 = bf16 stored as uint16 bit patterns, 1 = fp32.  The oracle decodes
    each element exactly to double.
    """
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), 0
    if t.dtype == torch.float32:
        return t.numpy(), 1
    raise TypeError(t.dtype)


def sample_rows(cfg: Config, n_random=256, tile=128, seed=None):
    """Stratified sample of query rows (b, h, t) for checks at large sizes.

    For every (batch, head): the first ``tile`` tokens of block 0, of block
    topk-1, of block topk, of a middle block and of the last block (the blocks
    that exist), plus ``n_random`` random rows over the whole problem.  Returns
    an int64 array [R, 3], sorted and unique.
    """
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed + 17))
    B, n, S = cfg.block_size, cfg.n_blocks, cfg.seqlen
    blocks = sorted({0, min(cfg.topk - 1, n - 1), min(cfg.topk, n - 1), n // 2, n - 1})
    rows = []
    for b in range(cfg.batch):
        for h in range(cfg.hq):
            for blk in blocks:
                t0 = blk * B
                t1 = min(t0 + tile, S)
                for t in range(t0, t1):
                    rows.append((b, h, t))
    rb = rng.integers(0, cfg.batch, n_random)
    rh = rng.integers(0, cfg.hq, n_random)
    rt = rng.integers(0, S, n_random)
    rows.extend(zip(rb.tolist(), rh.tolist(), rt.tolist()))
    arr = np.unique(np.array(rows, dtype=np.int64), axis=0)
    return arr
