"""fp64 CPU oracle for MoBA causal prefill -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the bench's CPU-baseline
leg may import this package.  The GPU library never imports, links or calls
it, and it shares no code with the GPU library.

The arithmetic lives in ``moba_oracle.c`` (plain loops, fp64, OpenMP over
rows); this module only builds it with gcc and marshals numpy arrays.  Every
function decodes the bf16 / fp32 storage exactly to double.

Parity status per function (pins live in tests/test_oracle_pins.py):
  pool            pinned: closed-form block means (arange keys, tail block).
  gate            pinned: constructed one-hot keys with known scores and ties,
                  brute force over all subsets on tiny inputs, invariances.
  attend          pinned: dense causal SDPA when every block is selected,
                  block-diagonal SDPA when topk == 1, closed forms (first
                  token, block size 1), brute force, V -> aV + c, hull bounds.
  attend_merged   pinned: equals ``attend`` (merge algebra) and the above.
  backward        pinned: central finite differences of ``attend`` under a fixed
                  selection (dyadic inputs), torch autograd of dense causal SDPA
                  in fp64 when every block is selected (GQA), sum rules
                  (sum of dk = 0, sum of dv = sum of dout per KV head).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moba_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_lib = None

_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def build(force=True):
    """Compile moba_oracle.c with gcc (plain -O2, OpenMP, strict IEEE math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, cll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.oracle_pool.argtypes = [vp, ci, ci, ci, ci, ci, ci, _f64p]
    lib.oracle_gate.argtypes = [vp, ci, _f64p, ci, ci, ci, ci, ci, ci, ci, cll, _i64p, _i32p,
                                _f64p, vp]
    for f in (lib.oracle_attend, lib.oracle_attend_merged):
        f.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, cll, _i64p, _i32p, _f64p,
                      _f64p]
    lib.oracle_selection_gap.argtypes = [vp, ci, _f64p, ci, ci, ci, ci, ci, ci, ci, cll, _i64p,
                                         _i32p, _i32p, _f64p]
    lib.oracle_backward.argtypes = [vp, vp, vp, ci, _f64p, ci, ci, ci, ci, ci, ci, ci, _i32p,
                                    ci, _f64p, _f64p, _f64p]
    for f in (lib.oracle_pool, lib.oracle_gate, lib.oracle_attend, lib.oracle_attend_merged,
              lib.oracle_selection_gap, lib.oracle_backward, lib.oracle_num_threads,
              lib.oracle_abi_version):
        f.restype = ci
    _lib = lib
    return lib


def num_threads():
    return _load().oracle_num_threads()


def _raw(a, code):
    a = np.ascontiguousarray(a)
    want = np.uint16 if code == 0 else np.float32
    if a.dtype != want:
        raise TypeError(f"storage code {code} wants {want}, got {a.dtype}")
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def n_blocks(S, block):
    return -(-S // block)


def all_rows(batch, hq, S):
    """Every (b, h, t) row, in (b, h, t) order, as int64 [R, 3]."""
    b, h, t = np.meshgrid(np.arange(batch), np.arange(hq), np.arange(S), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), t.ravel()], axis=1).astype(np.int64)


def pool(k, code, batch, S, hkv, d, block):
    """Block means K̄ as float64 [batch, hkv, n, d]."""
    k, kp = _raw(k, code)
    n = n_blocks(S, block)
    out = np.zeros((batch, hkv, n, d), dtype=np.float64)
    _check(_load().oracle_pool(kp, code, batch, S, hkv, d, block, out), "pool")
    return out


def gate(q, code, kbar, batch, S, hq, hkv, d, block, topk, rows, want_scores=False):
    """Causal top-k per row: (idx int32 [R, topk], margin float64 [R], scores or None)."""
    q, qp = _raw(q, code)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    idx = np.zeros((R, topk), dtype=np.int32)
    margin = np.zeros((R,), dtype=np.float64)
    scores = None
    sp = None
    if want_scores:
        scores = np.zeros((R, n_blocks(S, block)), dtype=np.float64)
        sp = scores.ctypes.data_as(ctypes.c_void_p)
    _check(_load().oracle_gate(qp, code, kbar, batch, S, hq, hkv, d, block, topk, R, rows, idx,
                               margin, sp), "gate")
    return idx, margin, scores


def selection_gap(q, code, kbar, batch, S, hq, hkv, d, block, topk, rows, idx):
    """Validity and fp64 score gap of a supplied selection: (valid int32 [R], gap float64 [R])."""
    q, qp = _raw(q, code)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(R, -1)
    if idx.shape[1] != topk:
        raise ValueError("idx must have topk columns")
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    valid = np.zeros((R,), dtype=np.int32)
    gap = np.zeros((R,), dtype=np.float64)
    _check(_load().oracle_selection_gap(qp, code, kbar, batch, S, hq, hkv, d, block, topk, R,
                                        rows, idx, valid, gap), "selection_gap")
    return valid, gap


def _attend(fn, q, k, v, code, batch, S, hq, hkv, d, block, topk, rows, idx):
    q, qp = _raw(q, code)
    k, kp = _raw(k, code)
    v, vp = _raw(v, code)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(rows.shape[0], -1)
    if idx.shape[1] != topk:
        raise ValueError("idx must have topk columns")
    R = rows.shape[0]
    out = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros((R,), dtype=np.float64)
    _check(fn(qp, kp, vp, code, batch, S, hq, hkv, d, block, topk, R, rows, idx, out, lse),
           "attend")
    return out, lse


def attend(*args):
    """Dense masked softmax attention under a given selection: (out [R, d], lse [R])."""
    return _attend(_load().oracle_attend, *args)


def attend_merged(*args):
    """Per-block softmax partials merged by log-sum-exp: (out [R, d], lse [R])."""
    return _attend(_load().oracle_attend_merged, *args)


def backward(q, k, v, code, dout, batch, S, hq, hkv, d, block, topk, idx, t_lo=0):
    """Gradients (dq [b, S, hq, d], dk, dv [b, S, hkv, d], float64) of the attention under
    the selection idx [b, hq, S, topk] for the upstream gradient dout [b, S, hq, d].

    t_lo > 0: only rows t >= t_lo are processed; dq of those rows and dk, dv of keys
    s >= t_lo are still exact (causality), everything before is left at zero."""
    q, qp = _raw(q, code)
    k, kp = _raw(k, code)
    v, vp = _raw(v, code)
    dout = np.ascontiguousarray(dout, dtype=np.float64).reshape(batch, S, hq, d)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(batch, hq, S, topk)
    dq = np.zeros((batch, S, hq, d), dtype=np.float64)
    dk = np.zeros((batch, S, hkv, d), dtype=np.float64)
    dv = np.zeros((batch, S, hkv, d), dtype=np.float64)
    _check(_load().oracle_backward(qp, kp, vp, code, dout, batch, S, hq, hkv, d, block, topk,
                                   idx, int(t_lo), dq, dk, dv), "backward")
    return dq, dk, dv


def prefill(q, k, v, code, batch, S, hq, hkv, d, block, topk, rows=None):
    """Whole MoBA prefill for ``rows`` (default: all rows).

    Returns dict(rows, out [R, d], lse [R], idx [R, topk], margin [R], kbar).
    """
    if rows is None:
        rows = all_rows(batch, hq, S)
    kbar = pool(k, code, batch, S, hkv, d, block)
    idx, margin, _ = gate(q, code, kbar, batch, S, hq, hkv, d, block, topk, rows)
    out, lse = attend(q, k, v, code, batch, S, hq, hkv, d, block, topk, rows, idx)
    return {"rows": rows, "out": out, "lse": lse, "idx": idx, "margin": margin, "kbar": kbar}
