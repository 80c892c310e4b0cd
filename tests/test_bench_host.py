"""Host-side pieces of bench.py: the CPU-oracle legs' row sets and work counts.

The bench scales the oracle's time on a row sample to the whole prefill by
scored blocks (gate) and attended (query, key) pairs (attention); these tests
check those counts and the row sets on small workloads, on the CPU.
"""
import numpy as np
import pytest

import bench
import oracle
from synth import config_by_name, make_inputs


def _key(cfg, rows):
    return (rows[:, 0] * cfg.hq + rows[:, 1]) * cfg.seqlen + rows[:, 2]


@pytest.mark.parametrize("mode", ["full", "gate", "group"])
def test_cpu_prepare_row_sets(mode):
    cfg = config_by_name("moba-8k-b2-h8-d128")
    inp = make_inputs(cfg)
    prep = bench.cpu_prepare(cfg, {x: inp[x] for x in ("q", "k", "v")}, mode)
    gate_rows, sample = prep["gate_rows"], prep["sample"]
    everything = oracle.all_rows(cfg.batch, cfg.hq, cfg.seqlen)
    if mode == "group":
        # every row of the first KV group's heads, plus the sample rows, once each
        want = everything[everything[:, 1] < cfg.hq // cfg.hkv]
        want = np.unique(np.concatenate([want, sample]), axis=0)
        assert np.array_equal(gate_rows, want)
    else:
        assert np.array_equal(gate_rows, everything)
    keys = _key(cfg, gate_rows)
    assert np.all(np.diff(keys) > 0)                       # (b, h, t) order, no repeats
    if mode == "full":
        assert np.array_equal(sample, everything)
        assert prep["sample_pos"] is None
    else:
        assert np.array_equal(gate_rows[prep["sample_pos"]], sample)
    assert prep["scored_g"] == bench.row_work(cfg, gate_rows)[0]
    assert prep["pairs_s"] == bench.row_work(cfg, sample)[1]


@pytest.mark.parametrize("name", ["moba-1k-fp32-d64", "moba-8k-b2-h8-d128"])
def test_work_counts_over_every_row(name):
    """total_work (closed forms) equals row_work summed over every row, and
    the attended pairs equal a per-row count written out from the selection rule."""
    cfg = config_by_name(name)
    rows = oracle.all_rows(cfg.batch, cfg.hq, cfg.seqlen)
    scored, pairs = bench.total_work(cfg)
    assert (scored, pairs) == bench.row_work(cfg, rows)
    B, k = cfg.block_size, cfg.topk
    by_hand_scored = by_hand_pairs = 0
    for t in range(cfg.seqlen):
        own = t // B
        by_hand_scored += own                              # every earlier block is scored
        by_hand_pairs += (t - own * B + 1) + min(own, k - 1) * B
    assert scored == by_hand_scored * cfg.hq * cfg.batch
    assert pairs == by_hand_pairs * cfg.hq * cfg.batch
