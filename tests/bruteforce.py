"""Brute-force MoBA on tiny inputs, in pure Python (independent of the oracle).

Selection: among all subsets of the past blocks of size min(topk-1, own),
take the one with the largest total gate score (equal to the top-k when no
two scores tie), then add the own block.  Attention: an explicit double loop
over an explicit 0/1 mask of (query, key) pairs.
"""
import itertools
import math


def brute_moba(q, k, v, block, topk):
    """q: [S][hq][d], k and v: [S][hkv][d] nested lists of floats (one sequence).

    Returns (out [S][hq][d], sel [S][hq] as sorted tuples).
    """
    S = len(q)
    hq = len(q[0])
    hkv = len(k[0])
    d = len(q[0][0])
    n = (S + block - 1) // block
    G = hq // hkv

    kbar = [[[0.0] * d for _ in range(n)] for _ in range(hkv)]
    for g in range(hkv):
        for j in range(n):
            toks = [t for t in range(S) if t // block == j]
            for i in range(d):
                kbar[g][j][i] = sum(k[t][g][i] for t in toks) / len(toks)

    out = [[[0.0] * d for _ in range(hq)] for _ in range(S)]
    sel_all = [[None] * hq for _ in range(S)]
    for t in range(S):
        own = t // block
        for h in range(hq):
            g = h // G
            score = [sum(q[t][h][i] * kbar[g][j][i] for i in range(d)) for j in range(own)]
            m = min(topk - 1, own)
            best, best_val = (), None
            for sub in itertools.combinations(range(own), m):
                val = sum(score[j] for j in sub)
                if best_val is None or val > best_val:
                    best, best_val = sub, val
            sel = tuple(sorted(set(best) | {own}))
            sel_all[t][h] = sel
            mask = [1 if (tp <= t and tp // block in sel) else 0 for tp in range(S)]
            logits = [None] * S
            for tp in range(S):
                if mask[tp]:
                    logits[tp] = sum(q[t][h][i] * k[tp][g][i] for i in range(d)) / math.sqrt(d)
            mx = max(z for z in logits if z is not None)
            w = [math.exp(z - mx) if z is not None else 0.0 for z in logits]
            tot = sum(w)
            for i in range(d):
                out[t][h][i] = sum(w[tp] * v[tp][g][i] for tp in range(S)) / tot
    return out, sel_all
