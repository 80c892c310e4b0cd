"""The seeded input generator: determinism, bf16 rounding, planting statistics."""
import numpy as np
import torch

from synth import CONFIGS, make_inputs, sample_rows, to_oracle_array


def test_generator_is_deterministic_per_seed():
    cfg = CONFIGS[0]
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for key in ("q", "k", "v"):
        assert torch.equal(a[key], b[key])
    c = make_inputs(cfg, seed=cfg.seed + 1)
    assert not torch.equal(a["q"], c["q"])


def _rne_bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16 by bit arithmetic (independent of torch's cast)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(3)) * 0.1
    x = torch.cat([x, torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8])])
    ours, code = to_oracle_array(x.to(torch.bfloat16))
    assert code == 0
    np.testing.assert_array_equal(ours, _rne_bf16_bits(x.numpy()))


def test_planting_shifts_keys_and_some_later_queries():
    cfg = CONFIGS[0]                          # 1 planted block per head, shift prob 0.25
    inp = make_inputs(cfg)
    q, k = inp["q"].double(), inp["k"].double()
    B = cfg.block_size
    for g in range(cfg.hkv):
        p = int(inp["planted"][0, g, 0])
        kb = k[0, p * B:(p + 1) * B, g].mean(0)
        assert abs(kb.norm().item() - 2.0) < 0.1             # mean key ~ 2 u
        u = kb / kb.norm()
        later = q[0, (p + 1) * B:, g] @ u                     # shifted queries have q.u ~ 1
        frac = (later > 0.5).double().mean().item()
        assert 0.15 < frac < 0.35
        earlier = q[0, :p * B, g] @ u if p > 0 else torch.zeros(1, dtype=torch.float64)
        assert (earlier > 0.5).double().mean().item() < 0.01


def test_sample_rows_cover_strata():
    cfg = CONFIGS[3]
    rows = sample_rows(cfg)
    assert rows.shape[1] == 3
    assert np.all(rows[:, 2] < cfg.seqlen) and np.all(rows[:, 1] < cfg.hq)
    assert len(np.unique(rows, axis=0)) == len(rows)
    blocks = set((rows[:, 2] // cfg.block_size).tolist())
    assert {0, cfg.topk - 1, cfg.topk, cfg.n_blocks - 1} <= blocks


def test_sliced_generation_keeps_the_recipe():
    """Slices that cut through blocks plant the same blocks with the same statistics."""
    import dataclasses
    whole = CONFIGS[0]
    cfg = dataclasses.replace(whole, gen_slice=320)      # 1024 tokens, block 128: ragged slices
    a, b = make_inputs(cfg), make_inputs(cfg)
    for key in ("q", "k", "v"):
        assert torch.equal(a[key], b[key])
        assert a[key].shape == make_inputs(whole)[key].shape
    np.testing.assert_array_equal(a["planted"], make_inputs(whole)["planted"])
    q, k = a["q"].double(), a["k"].double()
    B = cfg.block_size
    for g in range(cfg.hkv):
        p = int(a["planted"][0, g, 0])
        kb = k[0, p * B:(p + 1) * B, g].mean(0)
        assert abs(kb.norm().item() - 2.0) < 0.1
        u = kb / kb.norm()
        frac = ((q[0, (p + 1) * B:, g] @ u) > 0.5).double().mean().item()
        assert 0.15 < frac < 0.35
        if p > 0:
            assert ((q[0, :p * B, g] @ u) > 0.5).double().mean().item() < 0.01
    # unplanted keys stay N(0, 1/d)
    mask = torch.ones(cfg.seqlen, dtype=torch.bool)
    for g in range(cfg.hkv):
        p = int(a["planted"][0, g, 0])
        mask[p * B:(p + 1) * B] = False
    rest = k[0, mask].reshape(-1)
    assert abs(rest.var().item() * cfg.head_dim - 1.0) < 0.05
