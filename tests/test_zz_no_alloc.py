"""moba_prefill_noalloc (the entry point for callers that cannot allocate)
against moba_prefill: bit-identical outputs, through the C ABI, on calls in a
row on one GPU -- each one smaller than the one before, so stale contents of
the shared scratch array from a bigger call must never leak into a smaller
one -- including a problem whose whole-sequence workspace exceeds the array
(run in query chunks).  Oversized problems are refused before any HIP call."""
import ctypes

import pytest
import torch

from synth import CONFIGS, Config, make_inputs


def _moba():
    import block_sparse_attention_moba_amd as moba
    return moba


def _cfg(name, **kw):
    base = dict(batch=1, hq=2, hkv=2, seqlen=1024, head_dim=128, dtype="bf16", block_size=128,
                topk=3, planted=2, shift_prob=0.25, seed=91)
    base.update(kw)
    return Config(name=name, **base)


def test_noalloc_refuses_oversized_problems():
    """One 65536-token block of 32 heads with top-k 3 (of 4 blocks) needs
    ~1.6 GB of partial outputs, more than the scratch array: refused with
    WORKSPACE_TOO_SMALL before any HIP call (fake, aligned pointers are never
    touched)."""
    moba = _moba()
    L = moba.lib()
    fake = [ctypes.c_void_p(0x10000 * (i + 1) << 20) for i in range(4)]
    rc = L.moba_prefill_noalloc(*fake, 1, 1 << 18, 32, 8, 128, 1 << 16, 3,
                                moba.MOBA_DTYPE_BF16, None)
    assert rc == 3, rc
    rc = L.moba_prefill_noalloc(None, *fake[1:], 1, 1024, 2, 2, 128, 128, 3,
                                moba.MOBA_DTYPE_BF16, None)
    assert rc == 1, rc


@pytest.mark.gpu
def test_noalloc_matches_prefill_on_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moba = _moba()
    dev = torch.device("cuda:0")
    cases = [
        CONFIGS[2],                    # 32K tokens, 32 heads: chunked to fit the scratch
        CONFIGS[1],                    # 8K, batch 2: one pass
        _cfg("noalloc-fp32-gqa", hq=4, hkv=1, seqlen=768, dtype="fp32", topk=3),
        _cfg("noalloc-small", seqlen=512, block_size=64, topk=4, head_dim=64),
        _cfg("noalloc-dense", seqlen=256, block_size=128, topk=4),
    ]
    for cfg in cases:
        b, S, hq, hkv, d, B, topk = (cfg.batch, cfg.seqlen, cfg.hq, cfg.hkv, cfg.head_dim,
                                     cfg.block_size, cfg.topk)
        print(f"case {cfg.name} dims={(b, S, hq, hkv, d, B, topk)} dtype={cfg.dtype}", flush=True)
        need, _ = moba.moba_workspace_size(b, S, hq, hkv, d, B, topk,
                                           0 if cfg.dtype == "bf16" else 1)
        inp = make_inputs(cfg)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        ref = moba.moba_prefill(q, k, v, B, topk)
        out = torch.full_like(q, float("nan"))
        moba.moba_prefill_noalloc(q, k, v, B, topk, out=out)
        again = moba.moba_prefill_noalloc(q, k, v, B, topk)
        torch.cuda.synchronize()
        print(f"  workspace {need / 2**20:.1f} MiB of {moba._lib.NOALLOC_SCRATCH_BYTES / 2**20:.0f}",
              flush=True)
        assert torch.equal(out, ref), cfg.name
        assert torch.equal(again, ref), cfg.name
    assert moba.moba_workspace_size(*(CONFIGS[2].batch, CONFIGS[2].seqlen, CONFIGS[2].hq,
                                      CONFIGS[2].hkv, CONFIGS[2].head_dim,
                                      CONFIGS[2].block_size, CONFIGS[2].topk))[0] \
        > moba._lib.NOALLOC_SCRATCH_BYTES
