"""libmoba.so loads, exports what include/moba.h declares, and rejects bad
arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_moba_amd as moba
from block_sparse_attention_moba_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moba.h")
INV, UNS, WS = (_lib.MOBA_ERR_INVALID_ARGUMENT, _lib.MOBA_ERR_UNSUPPORTED,
                _lib.MOBA_ERR_WORKSPACE_TOO_SMALL)
BF16, F32 = _lib.MOBA_DTYPE_BF16, _lib.MOBA_DTYPE_FP32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = moba.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define\s+MOBA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert moba.moba_abi_version() == int(m.group(1))


def test_status_strings():
    for s in range(5):
        assert moba.moba_status_string(s)
    assert moba.moba_status_string(99) == "unknown status"


def ws_size(*args):
    pb, gb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = moba.lib().moba_workspace_size(*args, ctypes.byref(pb), ctypes.byref(gb))
    return rc, pb.value, gb.value


@pytest.mark.parametrize("args,code", [
    ((0, 1024, 2, 2, 64, 128, 3, BF16), INV),        # batch 0
    ((1, 1024, 3, 2, 64, 128, 3, BF16), INV),        # Hq % Hkv
    ((1, 1024, 2, 2, 64, 128, 0, BF16), INV),        # topk 0
    ((1, 1024, 2, 2, 64, 128, 3, 7), INV),           # dtype
    ((1, 1024, 2, 2, 96, 128, 3, BF16), UNS),        # head_dim
    ((1, 1000, 2, 2, 64, 128, 3, BF16), UNS),        # S % 64
    ((1, 1024, 2, 2, 64, 32, 3, BF16), UNS),         # block % 64
    ((1, 1 << 25, 2, 2, 64, 4096, 3, BF16), UNS),    # seqlen limit
    ((1, 64 * 64, 2, 2, 64, 64, 40, BF16), UNS),     # topk > 32 while sparse
])
def test_workspace_size_validation(args, code):
    rc, _, _ = ws_size(*args)
    assert rc == code


def test_short_last_block_is_accepted():
    rc, pb, gb = ws_size(1, 1088, 2, 2, 64, 128, 3, BF16)       # 8 blocks + 64 tokens
    assert rc == 0 and pb > gb > 0
    rc2, pb2, _ = ws_size(1, 1024, 2, 2, 64, 128, 3, BF16)
    assert rc2 == 0 and pb > pb2                                   # a ninth block
    rc, pb, gb = ws_size(1, 1088, 2, 2, 64, 128, 9, BF16)        # topk >= 9 blocks: dense
    assert rc == 0 and gb < pb < gb + (1 << 16)


def test_workspace_sizes():
    rc, pb, gb = ws_size(1, 1024, 2, 2, 64, 128, 3, F32)
    assert rc == 0 and pb > gb > 0
    # topk >= n: full attention needs only the key-norm pass and the deferred-tile list
    rc, pb, gb = ws_size(1, 1024, 2, 2, 64, 128, 8, F32)
    assert rc == 0 and gb < pb < gb + (1 << 16)
    rc, pb2, gb2 = ws_size(1, 64 * 64, 2, 2, 64, 64, 40 + 24, BF16)
    assert rc == 0 and gb2 < pb2 < gb2 + (1 << 16)           # dense again: no topk limit
    # the 1M-token workload fits one 288 GB GPU with its inputs
    rc, pb, _ = ws_size(1, 1 << 20, 32, 8, 128, 4096, 12, BF16)
    assert rc == 0 and 50e9 < pb < 200e9


def ws_chunked(*args):
    pb = ctypes.c_size_t(0)
    rc = moba.lib().moba_workspace_size_chunked(*args, ctypes.byref(pb))
    return rc, pb.value


def test_chunked_workspace():
    dims = (1, 1 << 20, 32, 8, 128, 4096, 12, BF16)
    _, whole, _ = ws_size(*dims)
    assert ws_chunked(*dims, 1 << 20) == (0, whole)          # one chunk: same scratch
    assert ws_chunked(*dims, 1 << 22) == (0, whole)
    rc, quarter = ws_chunked(*dims, 1 << 18)
    assert rc == 0 and whole / 5 < quarter < whole / 3
    rc, one_block = ws_chunked(*dims, 4096)
    assert rc == 0 and one_block < quarter / 32
    # 10M tokens: whole-sequence scratch is near 1 TB, 256K-token chunks fit one GPU
    ten = (1, 10 * (1 << 20), 32, 8, 128, 4096, 12, BF16)
    rc, big, _ = ws_size(*ten)
    assert rc == 0 and big > 900e9
    rc, small = ws_chunked(*ten, 1 << 18)
    assert rc == 0 and small < 30e9
    # a tail chunk shorter than the rest is covered
    rc, tail = ws_chunked(1, 1920, 2, 1, 128, 192, 3, BF16, 3 * 192)
    assert rc == 0 and tail > 0
    assert ws_chunked(*dims, 0)[0] == INV
    assert ws_chunked(*dims, -4096)[0] == INV
    assert ws_chunked(*dims, 4096 + 64)[0] == UNS
    assert ws_chunked(1, 1000, 2, 2, 64, 128, 3, BF16, 128)[0] == UNS
    assert moba.lib().moba_workspace_size_chunked(*dims, 4096, None) == INV


def ws_varlen(cu, *rest):
    arr = (ctypes.c_int * len(cu))(*cu)
    pb = ctypes.c_size_t(0)
    rc = moba.lib().moba_workspace_size_varlen(arr, len(cu) - 1, *rest, ctypes.byref(pb))
    return rc, pb.value


def test_varlen_workspace_and_validation():
    heads = (4, 2, 128, 128, 3, BF16)
    cu = [0, 640, 1728, 1728, 1792]              # 640, 1088 (short last block), 0, 64
    rc, pb = ws_varlen(cu, *heads, 1 << 20)
    assert rc == 0
    per = [ws_chunked(1, n, *heads, 1 << 20)[1] for n in (640, 1088, 64)]
    assert pb == max(per)
    rc, pb2 = ws_varlen(cu, *heads, 256)          # 2-block chunks
    assert rc == 0 and pb2 <= pb
    L = moba.lib()
    assert L.moba_workspace_size_varlen(None, 1, *heads, 256, None) == INV
    assert ws_varlen([0, 64], *heads, 256)[0] == 0
    assert ws_varlen([0], *heads, 256)[0] == INV                 # no sequence
    assert ws_varlen([64, 128], *heads, 256)[0] == INV           # must start at 0
    assert ws_varlen([0, 128, 64], *heads, 256)[0] == INV        # decreasing
    assert ws_varlen([0, 100], *heads, 256)[0] == UNS            # length % 64
    assert ws_varlen([0, 128], *heads, 0)[0] == INV
    assert ws_varlen([0, 128], *heads, 192)[0] == UNS            # chunk % block
    arr = (ctypes.c_int * 2)(0, 128)
    assert L.moba_workspace_size_varlen(arr, 1, *heads, 256, None) == INV


FAKE = 1 << 40          # aligned, never dereferenced: every call below fails validation


def prefill(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), out=FAKE + (3 << 32),
            dims=(1, 1024, 2, 2, 64, 128, 3, BF16), ws=FAKE + (4 << 32), nbytes=1 << 40):
    vp = ctypes.c_void_p
    return moba.lib().moba_prefill(vp(q), vp(k), vp(v), vp(out), *dims, vp(ws), nbytes, None)


def test_prefill_rejects_before_any_hip_call():
    assert prefill(q=0) == INV
    assert prefill(out=0) == INV
    assert prefill(dims=(1, 1024, 2, 2, 80, 128, 3, BF16)) == UNS
    assert prefill(q=FAKE + 2) == UNS                        # misaligned
    assert prefill(out=FAKE + 64) == INV                     # out overlaps q
    assert prefill(nbytes=16) == WS
    assert prefill(ws=0) == INV
    assert prefill(ws=FAKE + (4 << 32) + 16) == UNS          # workspace alignment


def test_chunked_prefill_rejects_before_any_hip_call():
    vp = ctypes.c_void_p

    def call(chunk, nbytes=1 << 40, dims=(1, 1024, 2, 2, 64, 128, 3, BF16)):
        return moba.lib().moba_prefill_chunked(vp(FAKE), vp(FAKE + (1 << 32)),
                                               vp(FAKE + (2 << 32)), vp(FAKE + (3 << 32)), *dims,
                                               chunk, vp(FAKE + (4 << 32)), nbytes, None)
    assert call(0) == INV
    assert call(100) == UNS
    assert call(256, nbytes=1024) == WS
    assert call(256, dims=(1, 1024, 2, 2, 80, 128, 3, BF16)) == UNS


def test_varlen_prefill_rejects_before_any_hip_call():
    vp = ctypes.c_void_p

    def call(cu, chunk=256, nbytes=1 << 40, q=FAKE, out=FAKE + (3 << 32), ws=FAKE + (4 << 32)):
        arr = (ctypes.c_int * len(cu))(*cu)
        return moba.lib().moba_prefill_varlen(vp(q), vp(FAKE + (1 << 32)), vp(FAKE + (2 << 32)),
                                              vp(out), arr, len(cu) - 1, 4, 2, 128, 128, 3,
                                              BF16, chunk, vp(ws), nbytes, None)
    assert call([0, 640, 1728, 1800]) == UNS    # the last sequence holds 72 tokens
    assert call([0, 640], q=0) == INV
    assert call([0, 640], out=FAKE + 64) == INV
    assert call([0, 640], nbytes=64) == WS
    assert call([0, 640], chunk=0) == INV
    assert call([0, 640], ws=FAKE + (4 << 32) + 8) == UNS


def test_backward_workspace_and_validation():
    L = moba.lib()
    nb = ctypes.c_size_t(0)
    assert L.moba_workspace_size_backward(1, 1024, 2, 2, 64, 128, 3, BF16, ctypes.byref(nb)) == 0
    assert nb.value > 2 * 1024 * 3 * 64 * 2                      # dq slots (bf16) and more
    assert L.moba_workspace_size_backward(1, 1024, 2, 2, 64, 128, 3, F32, ctypes.byref(nb)) == UNS
    assert L.moba_workspace_size_backward(1, 1024, 2, 2, 64, 128, 8, BF16, ctypes.byref(nb)) == 0
    assert L.moba_workspace_size_backward(1, 64 * 64, 2, 2, 64, 64, 64, BF16,
                                          ctypes.byref(nb)) == UNS   # full selection, 64 blocks
    assert L.moba_workspace_size_backward(1, 1024, 2, 2, 64, 128, 3, BF16, None) == INV
    vp = ctypes.c_void_p

    def call(dq=FAKE + (6 << 32), q=FAKE, lse=FAKE + (5 << 32), nbytes=1 << 40, dt=BF16):
        return L.moba_backward(vp(q), vp(FAKE + (1 << 32)), vp(FAKE + (2 << 32)),
                               vp(FAKE + (3 << 32)), vp(FAKE + (4 << 32)), vp(lse), vp(dq),
                               vp(FAKE + (7 << 32)), vp(FAKE + (8 << 32)), 1, 1024, 2, 2, 64, 128,
                               3, dt, vp(FAKE + (9 << 32)), nbytes, None)
    assert call(dq=0) == INV
    assert call(lse=0) == INV
    assert call(dq=FAKE + 64) == INV                             # dq overlaps q
    assert call(dq=FAKE + (3 << 32)) == INV                      # dq overlaps out
    assert call(q=FAKE + 8) == UNS
    assert call(lse=FAKE + (5 << 32) + 2) == UNS
    assert call(nbytes=1024) == WS
    assert call(dt=F32) == UNS


def test_prefill_lse_validation():
    vp = ctypes.c_void_p

    def call(lse):
        return moba.lib().moba_prefill_lse(vp(FAKE), vp(FAKE + (1 << 32)), vp(FAKE + (2 << 32)),
                                           vp(FAKE + (3 << 32)), vp(lse), 1, 1024, 2, 2, 64, 128,
                                           3, BF16, vp(FAKE + (4 << 32)), 1 << 40, None)
    assert call(0) == INV
    assert call(FAKE + (5 << 32) + 2) == UNS
    assert call(FAKE + (3 << 32) + 256) == INV                   # overlaps out


def test_timed_prefill_needs_events():
    vp = ctypes.c_void_p
    arr = (vp * (_lib.MOBA_NUM_STAGES + 1))()
    rc = moba.lib().moba_prefill_timed(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE + (3 << 32)),
                                       1, 1024, 2, 2, 64, 128, 3, BF16, vp(FAKE), 1 << 40, None,
                                       arr)
    assert rc == INV


def test_gate_and_pool_validation():
    vp = ctypes.c_void_p
    L = moba.lib()
    assert L.moba_gate(vp(0), vp(FAKE), vp(FAKE), 1, 1024, 2, 2, 64, 128, 3, BF16, vp(FAKE),
                       1 << 40, None) == INV
    assert L.moba_gate(vp(FAKE), vp(FAKE), vp(FAKE + 2), 1, 1024, 2, 2, 64, 128, 3, BF16,
                       vp(FAKE), 1 << 40, None) == UNS
    assert L.moba_gate(vp(FAKE), vp(FAKE), vp(FAKE), 1, 1024, 2, 2, 64, 128, 3, BF16,
                       vp(FAKE), 8, None) == WS
    assert L.moba_pool(vp(FAKE), vp(0), 1, 1024, 2, 64, 128, BF16, vp(FAKE), 1 << 40,
                       None) == INV
    assert L.moba_pool(vp(FAKE), vp(FAKE), 1, 1024, 2, 64, 100, BF16, vp(FAKE), 1 << 40,
                       None) == UNS


def test_gate_scores_validation():
    vp = ctypes.c_void_p
    L = moba.lib()
    assert L.moba_gate_scores(vp(0), vp(FAKE), vp(FAKE + (1 << 32)), 1, 1024, 2, 2, 64, 128, BF16,
                              vp(FAKE + (2 << 32)), 1 << 40, None) == INV
    assert L.moba_gate_scores(vp(FAKE), vp(FAKE), vp(FAKE + (1 << 32)), 1, 1024, 2, 2, 64, 128, F32,
                              vp(FAKE + (2 << 32)), 1 << 40, None) == UNS     # bf16 only
    assert L.moba_gate_scores(vp(FAKE), vp(FAKE), vp(FAKE + (1 << 32) + 2), 1, 1024, 2, 2, 64, 128,
                              BF16, vp(FAKE + (2 << 32)), 1 << 40, None) == UNS
    assert L.moba_gate_scores(vp(FAKE), vp(FAKE), vp(FAKE + (1 << 32)), 1, 1024, 2, 2, 64, 128, BF16,
                              vp(FAKE + (2 << 32)), 8, None) == WS
    assert L.moba_gate_scores(vp(FAKE), vp(FAKE), vp(FAKE + (1 << 32)), 1, 1000, 2, 2, 64, 128, BF16,
                              vp(FAKE + (2 << 32)), 1 << 40, None) == UNS     # S % 64


def test_python_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 128, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moba.moba_prefill(q, q[:, :, :1], q[:, :, :1], 64, 2)
