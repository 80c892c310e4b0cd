"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test names what it pins.  None of them re-types the oracle's own
formulas: the references are closed forms, textbook routines (numpy softmax,
torch's scaled_dot_product_attention), brute force, invariances and the
sparsity figures the pages print.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from bruteforce import brute_moba
from compare import output_ok, output_report

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(S, hq, hkv, d, batch=1, seed=0, planted=0, block=None):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((batch, S, hq, d)) / math.sqrt(d)).astype(np.float32)
    k = (rng.standard_normal((batch, S, hkv, d)) / math.sqrt(d)).astype(np.float32)
    v = (rng.standard_normal((batch, S, hkv, d)) / math.sqrt(d)).astype(np.float32)
    if planted:
        n = -(-S // block)
        for b in range(batch):
            for g in range(hkv):
                for p in rng.choice(max(n - 1, 1), size=min(planted, max(n - 1, 1)), replace=False):
                    u = rng.standard_normal(d)
                    u /= np.linalg.norm(u)
                    k[b, p * block:(p + 1) * block, g] += (2.0 * u).astype(np.float32)
                    G = hq // hkv
                    for hh in range(G):
                        m = rng.random(S) < 0.3
                        m[:(p + 1) * block] = False
                        q[b, m, g * G + hh] += u.astype(np.float32)
    return q, k, v


def run_oracle(q, k, v, block, topk, rows=None, merged=False):
    batch, S, hq, d = q.shape
    hkv = k.shape[2]
    if rows is None:
        rows = oracle.all_rows(batch, hq, S)
    kbar = oracle.pool(k, 1, batch, S, hkv, d, block)
    idx, margin, _ = oracle.gate(q, 1, kbar, batch, S, hq, hkv, d, block, topk, rows)
    fn = oracle.attend_merged if merged else oracle.attend
    out, lse = fn(q, k, v, 1, batch, S, hq, hkv, d, block, topk, rows, idx)
    return rows, idx, margin, out, lse


def to_bhtd(out, rows, batch, hq, S, d):
    res = np.full((batch, hq, S, d), np.nan)
    res[rows[:, 0], rows[:, 1], rows[:, 2]] = out
    return res


def dense_causal_numpy(q, k, v):
    """Textbook causal softmax attention, one (batch, head) at a time, fp64."""
    batch, S, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    out = np.zeros((batch, hq, S, d))
    for b in range(batch):
        for h in range(hq):
            g = h // G
            z = q[b, :, h].astype(np.float64) @ k[b, :, g].astype(np.float64).T / math.sqrt(d)
            z[np.triu_indices(S, 1)] = -np.inf
            z -= z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = p @ v[b, :, g].astype(np.float64)
    return out


def dense_causal_sdpa(q, k, v):
    """torch's scaled_dot_product_attention (math path, CPU, fp64), causal."""
    hq, hkv = q.shape[2], k.shape[2]
    G = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()


# --------------------------------------------------------------------------- pool

def test_pool_closed_form_block_means():
    """K[t][g][i] = t + 100 g + i/2 has block mean (first + last token)/2 + 100 g + i/2."""
    S, hkv, d, block = 22, 3, 5, 8     # 3 blocks, the last one short (6 tokens)
    t = np.arange(S, dtype=np.float32)[:, None, None]
    g = np.arange(hkv, dtype=np.float32)[None, :, None]
    i = np.arange(d, dtype=np.float32)[None, None, :]
    k = (t + 100 * g + 0.5 * i)[None].astype(np.float32)
    kbar = oracle.pool(k, 1, 1, S, hkv, d, block)
    for j in range(3):
        t0, t1 = j * block, min((j + 1) * block, S) - 1
        expect = (t0 + t1) / 2 + 100 * np.arange(hkv)[:, None] + 0.5 * np.arange(d)[None, :]
        np.testing.assert_array_equal(kbar[0, :, j, :], expect)


def test_pool_decodes_bf16_exactly():
    """bf16 bit patterns 0x3FC0 = 1.5 and 0xC020 = -2.5 decode exactly."""
    S, hkv, d, block = 4, 1, 2, 4
    raw = np.array([0x3FC0, 0xC020] * S, dtype=np.uint16).reshape(1, S, hkv, d)
    kbar = oracle.pool(raw, 0, 1, S, hkv, d, block)
    np.testing.assert_array_equal(kbar[0, 0, 0], [1.5, -2.5])


# --------------------------------------------------------------------------- gate

def test_gate_constructed_scores_and_ties():
    """Keys of block j are w_j * e_j, so K̄_j = w_j e_j and the gate score is q_j w_j.

    Scores chosen by hand: the top two past blocks, a tie broken to the
    smaller block, the margin, and that future blocks are never eligible.
    """
    n, block, d = 6, 2, 6
    S = n * block
    w = np.array([1.0, 2.0, 3.0, 1.0, 5.0, 7.0])
    k = np.zeros((1, S, 1, d), np.float32)
    for j in range(n):
        k[0, j * block:(j + 1) * block, 0, j] = w[j]
    q = np.zeros((1, S, 1, d), np.float32)
    # query at t=10 (block 5): scores for blocks 0..4 = c_j * w_j
    c = np.array([0.5, 0.25, 0.125, 0.5, 0.0625, 9.0])   # scores 0.5, 0.5, 0.375, 0.5, 0.3125; block 5 is own
    q[0, 10, 0, :] = c
    # query at t=8 (block 4): scores blocks 0..3 = 3, 1, 6, 2; blocks 4, 5 not eligible
    q[0, 8, 0, :] = [3.0, 0.5, 2.0, 2.0, 100.0, 100.0]
    rows = np.array([[0, 0, 10], [0, 0, 8]], np.int64)
    kbar = oracle.pool(k, 1, 1, S, 1, d, block)
    idx, margin, scores = oracle.gate(q, 1, kbar, 1, S, 1, 1, d, block, 4, rows, want_scores=True)
    np.testing.assert_allclose(scores[0, :5], [0.5, 0.5, 0.375, 0.5, 0.3125])
    # top-3 past among a three-way tie at 0.5 -> blocks 0, 1, 3; then own block 5
    assert idx[0].tolist() == [0, 1, 3, 5]
    assert margin[0] == pytest.approx(0.5 - 0.375)
    # t=8: top-3 past of (3, 1, 6, 2) -> blocks 0, 2, 3; own block 4; block 5 is future
    assert idx[1].tolist() == [0, 2, 3, 4]
    assert margin[1] == pytest.approx(2.0 - 1.0)
    # topk=3 with a tie at the cut: 0.5 (blocks 0, 1, 3): smaller blocks win
    idx3, margin3, _ = oracle.gate(q, 1, kbar, 1, S, 1, 1, d, block, 3, rows[:1])
    assert idx3[0].tolist() == [0, 1, 5]
    assert margin3[0] == 0.0


def test_gate_trivial_rows_select_every_causal_block():
    q, k, _ = rand_inputs(64, 2, 1, 8, seed=3)
    block, topk = 8, 4
    rows = oracle.all_rows(1, 2, 64)
    kbar = oracle.pool(k, 1, 1, 64, 1, 8, block)
    idx, margin, _ = oracle.gate(q, 1, kbar, 1, 64, 2, 1, 8, block, topk, rows)
    for r, (_, _, t) in enumerate(rows):
        own = t // block
        if own <= topk - 1:
            assert idx[r].tolist() == list(range(own + 1)) + [-1] * (topk - 1 - own)
            assert np.isinf(margin[r])
        else:
            assert (idx[r] >= 0).sum() == topk and idx[r][-1] == own
            assert np.all(np.diff(idx[r]) > 0)


def test_gate_positive_query_scaling_keeps_selection():
    """Scaling q by a positive constant scales every score alike: same selection."""
    q, k, _ = rand_inputs(96, 2, 2, 8, seed=5, planted=2, block=8)
    rows = oracle.all_rows(1, 2, 96)
    kbar = oracle.pool(k, 1, 1, 96, 2, 8, 8)
    idx1, m1, _ = oracle.gate(q, 1, kbar, 1, 96, 2, 2, 8, 8, 3, rows)
    idx2, _, _ = oracle.gate((q * 4.0).astype(np.float32), 1, kbar, 1, 96, 2, 2, 8, 8, 3, rows)
    keep = m1 > 1e-9
    assert np.array_equal(idx1[keep], idx2[keep])


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "sparsity.json")))["cases"],
                         ids=lambda c: f"n{c['n_blocks']}_k{c['topk']}")
def test_topk_counts_own_block_matches_printed_sparsity(case):
    """The printed sparsities fix that top-k counts the query's own block."""
    n, topk = case["n_blocks"], case["topk"]
    block, d = 2, 4
    S = n * block
    q, k, _ = rand_inputs(S, 1, 1, d, seed=11)
    rows = np.array([[0, 0, S - 1]], np.int64)          # a query in the last block sees all n blocks
    kbar = oracle.pool(k, 1, 1, S, 1, d, block)
    idx, _, _ = oracle.gate(q, 1, kbar, 1, S, 1, 1, d, block, topk, rows)
    nsel = int((idx[0] >= 0).sum())
    got = round(100.0 * (1.0 - nsel / n), case["decimals"])
    assert got == pytest.approx(case["printed_sparsity_percent"])
    # the other reading (own block on top of top-k) would not reproduce the figure
    other = round(100.0 * (1.0 - (topk + 1) / n), case["decimals"])
    assert other != pytest.approx(case["printed_sparsity_percent"])


def test_mean_selected_blocks_per_row():
    """|Sel| = min(own + 1, topk), so the mean over a sequence is sum_b min(b+1, k) / n."""
    n, block, topk = 16, 4, 5
    S = n * block
    q, k, _ = rand_inputs(S, 2, 2, 4, seed=13)
    rows = oracle.all_rows(1, 2, S)
    kbar = oracle.pool(k, 1, 1, S, 2, 4, block)
    idx, _, _ = oracle.gate(q, 1, kbar, 1, S, 2, 2, 4, block, topk, rows)
    mean_sel = (idx >= 0).sum(axis=1).mean()
    assert mean_sel == pytest.approx(sum(min(b + 1, topk) for b in range(n)) / n)


# --------------------------------------------------------------------------- selection check

def _onehot_problem():
    """Keys of block j are w_j e_j, so K̄_j = w_j e_j and the gate score of block j is q_j w_j.

    Row t=10 (own block 5) scores blocks 0..4 as 0.5, 0.5, 0.375, 0.5, 0.3125;
    row t=8 (own block 4) scores blocks 0..3 as 3, 1, 6, 2; rows t=2 and t=0
    sit in blocks 1 and 0.
    """
    n, block, d = 6, 2, 6
    S = n * block
    w = np.array([1.0, 2.0, 3.0, 1.0, 5.0, 7.0])
    k = np.zeros((1, S, 1, d), np.float32)
    for j in range(n):
        k[0, j * block:(j + 1) * block, 0, j] = w[j]
    q = np.zeros((1, S, 1, d), np.float32)
    q[0, 10, 0, :] = [0.5, 0.25, 0.125, 0.5, 0.0625, 9.0]
    q[0, 8, 0, :] = [3.0, 0.5, 2.0, 2.0, 100.0, 100.0]
    q[0, 2, 0, :] = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    kbar = oracle.pool(k, 1, 1, S, 1, d, block)
    return q, kbar, S, d, block


def _gap(q, kbar, S, d, block, topk, ts, sels):
    rows = np.array([[0, 0, t] for t in ts], np.int64)
    idx = np.array(sels, np.int32)
    return oracle.selection_gap(q, 1, kbar, 1, S, 1, 1, d, block, topk, rows, idx)


def test_selection_gap_hand_computed_on_one_hot_keys():
    """Valid selections, correct and wrong, and their gaps (lowest selected minus
    highest unselected past score) computed by hand from the known scores."""
    q, kbar, S, d, block = _onehot_problem()
    cases = [
        (10, [0, 1, 3, 5], 0.5 - 0.375),      # the oracle's own pick: gap = margin
        (10, [0, 1, 2, 5], 0.375 - 0.5),      # block 2 (0.375) taken instead of block 3 (0.5)
        (10, [0, 3, 4, 5], 0.3125 - 0.5),     # block 4 (0.3125) in, blocks 1, 2 out
        (8, [0, 2, 3, 4], 2.0 - 1.0),         # the oracle's own pick
        (8, [0, 1, 2, 4], 1.0 - 2.0),         # block 1 (score 1) instead of block 3 (score 2)
        (8, [1, 2, 3, 4], 1.0 - 3.0),         # block 0 (score 3) left out
        (2, [0, 1, -1, -1], np.inf),          # every causal block selected: nothing left out
        (0, [0, -1, -1, -1], np.inf),         # block 0: no past block at all
    ]
    valid, gap = _gap(q, kbar, S, d, block, 4, [c[0] for c in cases], [c[1] for c in cases])
    assert valid.tolist() == [1] * len(cases)
    np.testing.assert_array_equal(gap, [c[2] for c in cases])


def test_selection_gap_rejects_malformed_rows():
    """Each row breaks exactly one rule of a causal top-k listing and must be invalid."""
    q, kbar, S, d, block = _onehot_problem()
    bad = [
        (10, [1, 0, 3, 5]),       # past blocks not ascending
        (10, [0, 3, 3, 5]),       # a past block listed twice
        (10, [0, 1, 3, 4]),       # own block missing (block 4 in its slot)
        (10, [0, 1, 5, 5]),       # the own block listed as a past block
        (8, [0, 2, 5, 4]),        # a future block (5 > own block 4) among the past blocks
        (10, [-1, 0, 1, 5]),      # padding where a past block belongs (too few past blocks)
        (2, [0, 1, -1, 3]),       # a block in the padding
        (2, [0, 1, 0, -1]),       # a repeated block in the padding
        (0, [0, 0, -1, -1]),      # block 0 row with a past entry
        (2, [1, -1, -1, -1]),     # own block in the past slot, nothing after it
    ]
    good = [(10, [0, 1, 3, 5]), (8, [0, 2, 3, 4]), (2, [0, 1, -1, -1]), (0, [0, -1, -1, -1])]
    rows = bad + good
    valid, gap = _gap(q, kbar, S, d, block, 4, [r[0] for r in rows], [r[1] for r in rows])
    assert valid.tolist() == [0] * len(bad) + [1] * len(good)


def test_selection_gap_of_oracle_selection_equals_margin():
    """On planted random inputs (GQA, batch 2, a short last block) the oracle's own
    selection is valid on every row and its gap is the oracle's margin."""
    S, hq, hkv, d, block, topk = 200, 4, 2, 8, 16, 4
    q, k, _ = rand_inputs(S, hq, hkv, d, batch=2, seed=31, planted=3, block=block)
    rows = oracle.all_rows(2, hq, S)
    kbar = oracle.pool(k, 1, 2, S, hkv, d, block)
    idx, margin, _ = oracle.gate(q, 1, kbar, 2, S, hq, hkv, d, block, topk, rows)
    valid, gap = oracle.selection_gap(q, 1, kbar, 2, S, hq, hkv, d, block, topk, rows, idx)
    assert np.all(valid == 1)
    np.testing.assert_allclose(gap, margin, rtol=1e-12, atol=1e-15)
    assert np.isfinite(margin).sum() > 0


def test_selection_gap_of_swapped_selection_matches_numpy_scores():
    """Swap each row's worst selected past block for its best unselected one; the
    gap must equal the one computed from numpy block means and numpy dot products."""
    S, hq, hkv, d, block, topk = 256, 4, 1, 8, 16, 5
    q, k, _ = rand_inputs(S, hq, hkv, d, seed=33, planted=2, block=block)
    n = S // block
    G = hq // hkv
    kbar_np = k[0].astype(np.float64).reshape(n, block, hkv, d).mean(axis=1)   # [n, hkv, d]
    rows = oracle.all_rows(1, hq, S)
    kbar = oracle.pool(k, 1, 1, S, hkv, d, block)
    idx, margin, _ = oracle.gate(q, 1, kbar, 1, S, hq, hkv, d, block, topk, rows)
    mut = idx.copy()
    expect = np.full(len(rows), np.inf)
    for r, (_, h, t) in enumerate(rows):
        own = t // block
        s = kbar_np[:own, h // G] @ q[0, t, h].astype(np.float64)
        sel = [int(x) for x in idx[r] if 0 <= x < own]
        rest = [j for j in range(own) if j not in sel]
        if not sel or not rest:
            continue
        worst = min(sel, key=lambda j: s[j])
        best = max(rest, key=lambda j: s[j])
        new_sel = sorted([j for j in sel if j != worst] + [best])
        new_rest = [j for j in range(own) if j not in new_sel]
        mut[r, :len(new_sel)] = new_sel
        expect[r] = min(s[new_sel]) - max(s[new_rest])
    valid, gap = oracle.selection_gap(q, 1, kbar, 1, S, hq, hkv, d, block, topk, rows, mut)
    assert np.all(valid == 1)
    swapped = np.isfinite(expect)
    assert swapped.sum() > 100
    assert np.all(gap[swapped] < 0)
    np.testing.assert_allclose(gap, expect, rtol=1e-10, atol=1e-13)


def test_selection_gap_rejects_rows_out_of_range():
    q, kbar, S, d, block = _onehot_problem()
    with pytest.raises(RuntimeError):
        _gap(q, kbar, S, d, block, 4, [S], [[0, 1, 2, 3]])


# --------------------------------------------------------------------------- attention

@pytest.mark.parametrize("S,hq,hkv,d,block,batch", [
    (64, 2, 2, 8, 8, 1), (70, 4, 2, 16, 16, 2), (96, 6, 2, 8, 32, 1)])
def test_every_block_selected_equals_dense_causal(S, hq, hkv, d, block, batch):
    """topk >= n: MoBA is full causal attention (the pages' seamless full/sparse switch)."""
    q, k, v = rand_inputs(S, hq, hkv, d, batch=batch, seed=S + d)
    n = -(-S // block)
    for merged in (False, True):
        rows, idx, margin, out, _ = run_oracle(q, k, v, block, n + 1, merged=merged)
        assert np.all(np.isinf(margin))
        got = to_bhtd(out, rows, batch, hq, S, d)
        np.testing.assert_allclose(got, dense_causal_numpy(q, k, v), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got, dense_causal_sdpa(q, k, v), rtol=1e-12, atol=1e-14)


def test_topk_one_is_block_diagonal_causal():
    """topk == 1 keeps only the own block: dense causal attention run per block."""
    S, hq, hkv, d, block = 64, 4, 2, 8, 16
    q, k, v = rand_inputs(S, hq, hkv, d, seed=21)
    rows, idx, margin, out, _ = run_oracle(q, k, v, block, 1)
    got = to_bhtd(out, rows, 1, hq, S, d)
    expect = np.zeros_like(got)
    for j in range(S // block):
        sl = slice(j * block, (j + 1) * block)
        expect[:, :, sl] = dense_causal_sdpa(q[:, sl], k[:, sl], v[:, sl])
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-14)
    assert np.all(np.isinf(margin))


def test_closed_forms_first_token_and_unit_blocks():
    """out[0] = v[0] exactly; with block 1 and topk 1 every token sees only itself."""
    S, hq, hkv, d = 24, 2, 1, 4
    q, k, v = rand_inputs(S, hq, hkv, d, seed=2)
    rows, _, _, out, lse = run_oracle(q, k, v, 8, 2)
    got = to_bhtd(out, rows, 1, hq, S, d)
    for h in range(hq):
        np.testing.assert_array_equal(got[0, h, 0], v[0, 0, 0].astype(np.float64))
    rows, _, _, out, _ = run_oracle(q, k, v, 1, 1)
    got = to_bhtd(out, rows, 1, hq, S, d)
    for h in range(hq):
        np.testing.assert_array_equal(got[0, h], v[0, :, 0].astype(np.float64))


@pytest.mark.parametrize("S,hq,hkv,d,block,topk,seed", [
    (16, 1, 1, 4, 4, 2, 0), (24, 2, 1, 3, 4, 3, 1), (32, 2, 2, 4, 8, 2, 2),
    (40, 4, 2, 2, 4, 4, 3), (30, 1, 1, 3, 4, 3, 4), (48, 2, 1, 4, 2, 5, 5)])
def test_matches_brute_force_on_tiny_inputs(S, hq, hkv, d, block, topk, seed):
    q, k, v = rand_inputs(S, hq, hkv, d, seed=seed)
    rows, idx, margin, out, _ = run_oracle(q, k, v, block, topk)
    bo, bsel = brute_moba(q[0].astype(np.float64).tolist(), k[0].astype(np.float64).tolist(),
                          v[0].astype(np.float64).tolist(), block, topk)
    for r, (_, h, t) in enumerate(rows):
        sel = tuple(int(x) for x in idx[r] if x >= 0)
        assert sel == bsel[t][h], (t, h)
        np.testing.assert_allclose(out[r], bo[t][h], rtol=1e-12, atol=1e-14)


def test_softmax_weights_sum_to_one_and_hull_bounds():
    """V = 1 gives out = 1 (weights sum to 1); outputs lie inside the attended V range."""
    S, hq, hkv, d, block, topk = 80, 4, 2, 8, 8, 3
    q, k, v = rand_inputs(S, hq, hkv, d, seed=8, planted=2, block=block)
    ones = np.ones_like(v)
    rows, idx, _, out1, _ = run_oracle(q, k, ones, block, topk)
    np.testing.assert_allclose(out1, 1.0, rtol=0, atol=1e-12)
    rows, idx, _, out, _ = run_oracle(q, k, v, block, topk)
    G = hq // hkv
    for r, (b, h, t) in enumerate(rows):
        sel = [x for x in idx[r] if x >= 0]
        toks = [tp for tp in range(t + 1) if tp // block in sel]
        vv = v[b, toks, h // G].astype(np.float64)
        assert np.all(out[r] >= vv.min(axis=0) - 1e-12)
        assert np.all(out[r] <= vv.max(axis=0) + 1e-12)


def test_key_shift_invariance():
    """K -> K + c shifts every gate score and logit of a query equally: nothing changes."""
    S, hq, hkv, d, block, topk = 96, 4, 2, 8, 8, 3
    q, k, v = rand_inputs(S, hq, hkv, d, seed=9, planted=2, block=block)
    c = np.random.default_rng(1).standard_normal(d).astype(np.float32) * 0.25
    rows, idx1, m1, out1, _ = run_oracle(q, k, v, block, topk)
    k2 = k + c[None, None, None, :]          # fp32 rounding of the shifted keys sets the tolerance
    _, idx2, _, out2, _ = run_oracle(q, k2, v, block, topk)
    keep = m1 > 1e-6
    assert np.array_equal(idx1[keep], idx2[keep])
    np.testing.assert_allclose(out2[keep], out1[keep], rtol=1e-5, atol=1e-7)


def test_value_affine_map():
    """V -> a V + c gives out -> a out + c."""
    S, hq, hkv, d, block, topk = 64, 2, 1, 8, 8, 3
    q, k, v = rand_inputs(S, hq, hkv, d, seed=10)
    a, c = 2.0, np.linspace(-1, 1, d).astype(np.float32)
    rows, idx, _, out1, _ = run_oracle(q, k, v, block, topk)
    v2 = (a * v + c).astype(np.float32)
    _, _, _, out2, _ = run_oracle(q, k, v2, block, topk)
    np.testing.assert_allclose(out2, a * out1 + c.astype(np.float64), rtol=1e-6, atol=1e-6)


def test_permuting_tokens_inside_another_block_changes_nothing():
    """A query's result depends on a non-own block only through its mean and its token set."""
    S, hq, hkv, d, block, topk = 64, 2, 2, 8, 8, 8
    q, k, v = rand_inputs(S, hq, hkv, d, seed=12)
    perm = np.arange(S)
    perm[16:24] = perm[16:24][::-1]            # reverse block 2
    rows, idx1, _, out1, _ = run_oracle(q, k, v, block, topk)
    _, idx2, _, out2, _ = run_oracle(q, k[:, perm], v[:, perm], block, topk)
    later = rows[:, 2] >= 24
    assert np.array_equal(idx1[later], idx2[later])
    np.testing.assert_allclose(out2[later], out1[later], rtol=1e-12, atol=1e-14)


def test_merged_path_equals_single_softmax():
    """Per-block softmax partials merged by log-sum-exp equal one softmax over the union."""
    S, hq, hkv, d, block, topk = 128, 4, 2, 16, 16, 3
    q, k, v = rand_inputs(S, hq, hkv, d, batch=2, seed=14, planted=2, block=block)
    rows, idx, _, out1, lse1 = run_oracle(q, k, v, block, topk)
    out2, lse2 = oracle.attend_merged(q, k, v, 1, 2, S, hq, hkv, d, block, topk, rows, idx)
    np.testing.assert_allclose(out2, out1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse2, lse1, rtol=1e-12, atol=1e-14)


def test_attend_rejects_future_or_bad_blocks():
    q, k, v = rand_inputs(32, 1, 1, 4, seed=1)
    rows = np.array([[0, 0, 9]], np.int64)   # block 1 with block size 8
    bad = np.array([[0, 2, -1]], np.int32)   # block 2 is in the future
    with pytest.raises(RuntimeError):
        oracle.attend(q, k, v, 1, 1, 32, 1, 1, 4, 8, 3, rows, bad)


# --------------------------------------------------------------------------- harness

def test_comparison_harness_catches_a_swapped_block():
    """The output comparison must fail when one selected past block per row is replaced."""
    S, hq, hkv, d, block, topk = 256, 2, 2, 16, 16, 4
    q, k, v = rand_inputs(S, hq, hkv, d, seed=15, planted=2, block=block)
    rows, idx, _, out, _ = run_oracle(q, k, v, block, topk)
    own = rows[:, 2] // block
    mut = idx.copy()
    sel_rows = []
    for r in range(len(rows)):
        past = [x for x in idx[r] if 0 <= x < own[r]]
        free = [j for j in range(own[r]) if j not in past]
        if past and free:
            mut[r, 0] = free[0]
            mut[r, :topk - 1] = np.sort(mut[r, :topk - 1])
            sel_rows.append(r)
    sel_rows = np.array(sel_rows)
    out_m, _ = oracle.attend(q, k, v, 1, 1, S, hq, hkv, d, block, topk, rows, mut)
    rep = output_report(out_m[sel_rows], out[sel_rows])
    assert not output_ok(rep, "bf16"), rep
    assert output_ok(output_report(out[sel_rows], out[sel_rows]), "fp32")


# ---------------------------------------------------------------- backward

def _selection(q, k, block, topk):
    """idx [b, hq, S, topk] from the oracle's own gate on every row."""
    batch, S, hq, d = q.shape
    rows, idx, _, _, _ = run_oracle(q, k, k, block, topk)
    return idx.reshape(batch, hq, S, topk)


def _loss(q, k, v, dout, block, topk, idx):
    """sum(dout * out) of the attention under the fixed selection idx."""
    batch, S, hq, d = q.shape
    rows = oracle.all_rows(batch, hq, S)
    out, _ = oracle.attend(q, k, v, 1, batch, S, hq, k.shape[2], d, block, topk, rows,
                           idx.reshape(-1, topk))
    out = to_bhtd(out, rows, batch, hq, S, d).transpose(0, 2, 1, 3)
    return float((dout * out).sum())


@pytest.mark.parametrize("S,hq,hkv,d,block,topk", [(16, 2, 1, 4, 4, 2), (24, 2, 2, 4, 8, 2),
                                                   (20, 4, 2, 2, 4, 3)])
def test_backward_matches_central_differences(S, hq, hkv, d, block, topk):
    """Pin: every gradient entry against (L(x + e) - L(x - e)) / 2e of the forward
    oracle with the selection held fixed.  Inputs are multiples of 2^-6 and
    e = 2^-14, so x +- e is exact in fp32 storage; the O(e^2) truncation is far
    below the 1e-6 tolerance."""
    rng = np.random.default_rng(S * 7 + d)
    q = (rng.integers(-48, 49, (1, S, hq, d)) / 64.0).astype(np.float32)
    k = (rng.integers(-48, 49, (1, S, hkv, d)) / 64.0).astype(np.float32)
    v = (rng.integers(-48, 49, (1, S, hkv, d)) / 64.0).astype(np.float32)
    dout = rng.standard_normal((1, S, hq, d))
    idx = _selection(q, k, block, topk)
    dq, dk, dv = oracle.backward(q, k, v, 1, dout, 1, S, hq, hkv, d, block, topk, idx)
    e = 2.0 ** -14
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(grad)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += e
            xm[pos] -= e
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dout, block, topk, idx)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dout, block, topk, idx)
            fd[pos] = (lp - lm) / (2 * e)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")


def test_backward_full_selection_equals_sdpa_autograd():
    """Pin: with every causal block selected the gradients are those of dense
    causal attention: torch autograd through scaled_dot_product_attention in
    fp64 (GQA: each query head uses its KV head; the KV gradients add up)."""
    S, hq, hkv, d, block = 48, 4, 2, 8, 8
    q, k, v = rand_inputs(S, hq, hkv, d, batch=2, seed=11)
    dout = np.random.default_rng(3).standard_normal((2, S, hq, d))
    topk = -(-S // block)
    idx = _selection(q, k, block, topk)
    dq, dk, dv = oracle.backward(q, k, v, 1, dout, 2, S, hq, hkv, d, block, topk, idx)
    G = hq // hkv
    tq = torch.tensor(q, dtype=torch.float64).transpose(1, 2).requires_grad_()
    tk = torch.tensor(k, dtype=torch.float64).transpose(1, 2).requires_grad_()
    tv = torch.tensor(v, dtype=torch.float64).transpose(1, 2).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=True)
    out.backward(torch.tensor(dout, dtype=torch.float64).transpose(1, 2))
    np.testing.assert_allclose(dq, tq.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_backward_sum_rules():
    """Pin: softmax weights of a row sum to 1, so over all keys of a KV head
    sum(dv) = sum of dout over its query heads, and sum(dk) = 0 (each row's
    ds sums to zero)."""
    S, hq, hkv, d, block, topk = 96, 4, 2, 8, 16, 3
    q, k, v = rand_inputs(S, hq, hkv, d, seed=5, planted=1, block=block)
    dout = np.random.default_rng(9).standard_normal((1, S, hq, d))
    idx = _selection(q, k, block, topk)
    dq, dk, dv = oracle.backward(q, k, v, 1, dout, 1, S, hq, hkv, d, block, topk, idx)
    G = hq // hkv
    for g in range(hkv):
        np.testing.assert_allclose(dv[0, :, g].sum(0), dout[0, :, g * G:(g + 1) * G].sum((0, 1)),
                                   rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(dk[0, :, g].sum(0), 0.0, atol=1e-10)
    assert np.abs(dq).max() > 1e-3 and np.abs(dk).max() > 1e-3


def test_backward_row_range_is_exact_past_t_lo():
    """Pin: with rows restricted to t >= t_lo, dq of those rows and dk, dv of
    keys >= t_lo equal the full computation (no earlier row sees a later key),
    while the skipped rows' dq stays zero."""
    S, hq, hkv, d, block, topk = 96, 4, 2, 8, 16, 3
    q, k, v = rand_inputs(S, hq, hkv, d, seed=8, planted=1, block=block)
    dout = np.random.default_rng(4).standard_normal((1, S, hq, d))
    idx = _selection(q, k, block, topk)
    full = oracle.backward(q, k, v, 1, dout, 1, S, hq, hkv, d, block, topk, idx)
    t_lo = 64
    part = oracle.backward(q, k, v, 1, dout, 1, S, hq, hkv, d, block, topk, idx, t_lo=t_lo)
    for f, p in zip(full, part):
        np.testing.assert_allclose(p[:, t_lo:], f[:, t_lo:], rtol=1e-12, atol=1e-14)
    assert np.all(part[0][:, :t_lo] == 0.0)
    assert np.abs(full[1][:, :t_lo] - part[1][:, :t_lo]).max() > 1e-6   # earlier keys differ
