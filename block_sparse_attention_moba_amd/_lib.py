"""ctypes binding of libmoba.so (argument marshalling only).

Every step of the MoBA prefill runs in the library's HIP kernels; torch is
used here only to own device memory and to name the current HIP stream.
There is no fallback: if libmoba.so is missing or a call fails, an exception
is raised.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoba.so")

MOBA_OK = 0
MOBA_ERR_INVALID_ARGUMENT = 1
MOBA_ERR_UNSUPPORTED = 2
MOBA_ERR_WORKSPACE_TOO_SMALL = 3
MOBA_ERR_HIP = 4
MOBA_DTYPE_BF16 = 0
MOBA_DTYPE_FP32 = 1
MOBA_NUM_STAGES = 5
STAGE_NAMES = ("pool", "gate", "index", "attn_past", "attn_own_merge")
EXPORTS = ("moba_abi_version", "moba_status_string", "moba_workspace_size", "moba_pool",
           "moba_gate", "moba_prefill", "moba_prefill_timed", "moba_workspace_size_chunked",
           "moba_prefill_chunked", "moba_workspace_size_varlen", "moba_prefill_varlen",
           "moba_prefill_lse", "moba_workspace_size_backward", "moba_backward",
           "moba_prefill_noalloc", "moba_gate_scores")
# bytes of moba_prefill_noalloc's scratch array on each GPU (MOBA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 512 << 20


class MobaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {moba_status_string(status)} (status {status})")


_lib = None


def lib():
    """The loaded libmoba.so with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m block_sparse_attention_moba_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    ci, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.moba_abi_version.restype = ci
    L.moba_abi_version.argtypes = []
    L.moba_status_string.restype = ctypes.c_char_p
    L.moba_status_string.argtypes = [ci]
    L.moba_workspace_size.restype = ci
    L.moba_workspace_size.argtypes = [ci] * 8 + [ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.moba_pool.restype = ci
    L.moba_pool.argtypes = [vp, vp] + [ci] * 6 + [vp, sz, vp]
    L.moba_gate.restype = ci
    L.moba_gate.argtypes = [vp, vp, vp] + [ci] * 8 + [vp, sz, vp]
    L.moba_prefill.restype = ci
    L.moba_prefill.argtypes = [vp, vp, vp, vp] + [ci] * 8 + [vp, sz, vp]
    L.moba_prefill_timed.restype = ci
    L.moba_prefill_timed.argtypes = [vp, vp, vp, vp] + [ci] * 8 + [vp, sz, vp,
                                                                  ctypes.POINTER(vp)]
    L.moba_workspace_size_chunked.restype = ci
    L.moba_workspace_size_chunked.argtypes = [ci] * 9 + [ctypes.POINTER(sz)]
    L.moba_prefill_chunked.restype = ci
    L.moba_prefill_chunked.argtypes = [vp, vp, vp, vp] + [ci] * 9 + [vp, sz, vp]
    ip = ctypes.POINTER(ci)
    L.moba_workspace_size_varlen.restype = ci
    L.moba_workspace_size_varlen.argtypes = [ip] + [ci] * 8 + [ctypes.POINTER(sz)]
    L.moba_prefill_varlen.restype = ci
    L.moba_prefill_varlen.argtypes = [vp, vp, vp, vp, ip] + [ci] * 8 + [vp, sz, vp]
    L.moba_prefill_lse.restype = ci
    L.moba_prefill_lse.argtypes = [vp] * 5 + [ci] * 8 + [vp, sz, vp]
    L.moba_workspace_size_backward.restype = ci
    L.moba_workspace_size_backward.argtypes = [ci] * 8 + [ctypes.POINTER(sz)]
    L.moba_backward.restype = ci
    L.moba_backward.argtypes = [vp] * 9 + [ci] * 8 + [vp, sz, vp]
    L.moba_prefill_noalloc.restype = ci
    L.moba_prefill_noalloc.argtypes = [vp, vp, vp, vp] + [ci] * 8 + [vp]
    L.moba_gate_scores.restype = ci
    L.moba_gate_scores.argtypes = [vp, vp, vp] + [ci] * 7 + [vp, sz, vp]
    _lib = L
    return L


def moba_abi_version():
    return lib().moba_abi_version()


def moba_status_string(status):
    return lib().moba_status_string(int(status)).decode()


def _check(status, what):
    if status != MOBA_OK:
        raise MobaError(status, what)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MOBA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MOBA_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def moba_workspace_size(batch, seqlen, num_q_heads, num_kv_heads, head_dim, block_size, topk,
                        dtype=MOBA_DTYPE_BF16):
    """(prefill_bytes, gate_bytes) for a problem."""
    pb, gb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().moba_workspace_size(batch, seqlen, num_q_heads, num_kv_heads, head_dim,
                                     block_size, topk, dtype, ctypes.byref(pb), ctypes.byref(gb)),
           "moba_workspace_size")
    return pb.value, gb.value


def moba_workspace_size_chunked(batch, seqlen, num_q_heads, num_kv_heads, head_dim, block_size,
                                topk, query_chunk, dtype=MOBA_DTYPE_BF16):
    """Workspace bytes of a prefill that runs in query chunks of query_chunk tokens."""
    pb = ctypes.c_size_t(0)
    _check(lib().moba_workspace_size_chunked(batch, seqlen, num_q_heads, num_kv_heads, head_dim,
                                             block_size, topk, dtype, query_chunk,
                                             ctypes.byref(pb)),
           "moba_workspace_size_chunked")
    return pb.value


def _cu_array(cu_seqlens):
    vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist")
                             else cu_seqlens)]
    return (ctypes.c_int * len(vals))(*vals), len(vals) - 1


def moba_workspace_size_varlen(cu_seqlens, num_q_heads, num_kv_heads, head_dim, block_size,
                               topk, query_chunk, dtype=MOBA_DTYPE_BF16):
    """Workspace bytes of moba_prefill_varlen; cu_seqlens: host offsets [num_seqs + 1]."""
    arr, ns = _cu_array(cu_seqlens)
    pb = ctypes.c_size_t(0)
    _check(lib().moba_workspace_size_varlen(arr, ns, num_q_heads, num_kv_heads, head_dim,
                                            block_size, topk, dtype, query_chunk,
                                            ctypes.byref(pb)), "moba_workspace_size_varlen")
    return pb.value


def moba_prefill_varlen(q, k, v, cu_seqlens, block_size, topk, out=None, workspace=None,
                        query_chunk=None):
    """MoBA prefill of packed sequences: q [total, hq, d], k/v [total, hkv, d] -> out like q.

    cu_seqlens: host sequence offsets (list or CPU tensor) [num_seqs + 1], starting at 0.
    query_chunk: tokens per query chunk within a sequence (None: whole sequences).
    """
    _need_cuda(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[0] != q.shape[0]:
        raise ValueError("q must be [total, hq, d] and k, v [total, hkv, d]")
    total, hq, d = q.shape
    hkv = k.shape[1]
    arr, ns = _cu_array(cu_seqlens)
    if arr[ns] != total:
        raise ValueError(f"cu_seqlens ends at {arr[ns]}, tensors hold {total} tokens")
    dt = _dtype_code(q)
    chunk = max(arr[i + 1] - arr[i] for i in range(ns)) if query_chunk is None else query_chunk
    if query_chunk is None:
        chunk = max(block_size, -(-chunk // block_size) * block_size)
    pb = moba_workspace_size_varlen(cu_seqlens, hq, hkv, d, block_size, topk, chunk, dt)
    ws = _workspace(pb, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda(out)
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q in shape and dtype")
    _check(lib().moba_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), arr, ns, hq, hkv, d,
                                     block_size, topk, dt, chunk, _ptr(ws),
                                     _nbytes(ws), _stream()),
           "moba_prefill_varlen")
    return out


def moba_prefill_lse(q, k, v, block_size, topk, out=None, lse=None, workspace=None):
    """moba_prefill that also returns the rows' natural-log log-sum-exp [b, hq, S] (fp32)."""
    _need_cuda(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, S, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [batch, seqlen, num_kv_heads, head_dim]")
    dt = _dtype_code(q)
    pb, _ = moba_workspace_size(b, S, hq, hkv, d, block_size, topk, dt)
    ws = _workspace(pb, q.device, workspace)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((b, hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    _need_cuda(out, lse)
    if out.dtype != q.dtype or out.shape != q.shape or lse.shape != (b, hq, S):
        raise ValueError("out must match q; lse must be float32 [batch, hq, seqlen]")
    _check(lib().moba_prefill_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, S, hq, hkv,
                                  d, block_size, topk, dt, _ptr(ws),
                                  _nbytes(ws), _stream()), "moba_prefill_lse")
    return out, lse


def moba_workspace_size_backward(batch, seqlen, num_q_heads, num_kv_heads, head_dim, block_size,
                                 topk, dtype=MOBA_DTYPE_BF16):
    nb = ctypes.c_size_t(0)
    _check(lib().moba_workspace_size_backward(batch, seqlen, num_q_heads, num_kv_heads, head_dim,
                                              block_size, topk, dtype, ctypes.byref(nb)),
           "moba_workspace_size_backward")
    return nb.value


def moba_backward(q, k, v, out, dout, lse, block_size, topk, workspace=None):
    """Gradients (dq, dk, dv) of the MoBA attention for the upstream gradient dout (bf16)."""
    _need_cuda(q, k, v, out, dout, lse)
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out and dout must share a dtype")
    if out.shape != q.shape or dout.shape != q.shape or k.shape != (b, S, hkv, d) \
            or v.shape != k.shape or lse.shape != (b, hq, S) or lse.dtype != torch.float32:
        raise ValueError("shapes: q, out, dout [b, S, hq, d]; k, v [b, S, hkv, d]; lse [b, hq, S]")
    dt = _dtype_code(q)
    nb = moba_workspace_size_backward(b, S, hq, hkv, d, block_size, topk, dt)
    ws = _workspace(nb, q.device, workspace)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib().moba_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), b, S, hq, hkv, d, block_size, topk,
                               dt, _ptr(ws), _nbytes(ws), _stream()),
           "moba_backward")
    return dq, dk, dv


def _nbytes(t):
    """Size of a tensor's storage in bytes (what the C ABI's *_bytes arguments take)."""
    return t.numel() * t.element_size()


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        _need_cuda(workspace)
        if _nbytes(workspace) < nbytes:
            raise ValueError(f"workspace holds {_nbytes(workspace)} bytes, {nbytes} needed")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def moba_pool(k, block_size, workspace=None):
    """fp32 block means of k [batch, seqlen, hkv, d] -> [batch, hkv, seqlen/block_size, d]."""
    _need_cuda(k)
    b, S, hkv, d = k.shape
    dt = _dtype_code(k)
    _, gb = moba_workspace_size(b, S, hkv, hkv, d, block_size, 1, dt)
    ws = _workspace(gb, k.device, workspace)
    n = -(-S // block_size)            # a short last block has its own mean
    kbar = torch.empty((b, hkv, n, d), dtype=torch.float32, device=k.device)
    _check(lib().moba_pool(_ptr(k), _ptr(kbar), b, S, hkv, d, block_size, dt, _ptr(ws),
                           _nbytes(ws), _stream()), "moba_pool")
    return kbar


def moba_gate(q, k, block_size, topk, workspace=None):
    """Selected blocks per query row: int32 [batch, hq, seqlen, topk], ascending, -1 padded."""
    _need_cuda(q, k)
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    dt = _dtype_code(q)
    if k.dtype != q.dtype:
        raise TypeError("q and k must share a dtype")
    _, gb = moba_workspace_size(b, S, hq, hkv, d, block_size, topk, dt)
    ws = _workspace(gb, q.device, workspace)
    idx = torch.empty((b, hq, S, topk), dtype=torch.int32, device=q.device)
    _check(lib().moba_gate(_ptr(q), _ptr(k), _ptr(idx), b, S, hq, hkv, d, block_size, topk, dt,
                           _ptr(ws), _nbytes(ws), _stream()), "moba_gate")
    return idx


def moba_gate_scores(q, k, block_size, workspace=None):
    """The bf16 gate's scores: fp32 [batch, hq, seqlen, n], NaN for blocks not in a row's past."""
    _need_cuda(q, k)
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    dt = _dtype_code(q)
    if k.dtype != q.dtype:
        raise TypeError("q and k must share a dtype")
    _, gb = moba_workspace_size(b, S, hq, hkv, d, block_size, 1, dt)
    ws = _workspace(gb, q.device, workspace)
    n = -(-S // block_size)
    scores = torch.empty((b, hq, S, n), dtype=torch.float32, device=q.device)
    _check(lib().moba_gate_scores(_ptr(q), _ptr(k), _ptr(scores), b, S, hq, hkv, d, block_size, dt,
                                  _ptr(ws), _nbytes(ws), _stream()), "moba_gate_scores")
    return scores


def moba_prefill(q, k, v, block_size, topk, out=None, workspace=None, stage_events=None,
                 query_chunk=None):
    """MoBA causal prefill forward.  q [b, S, hq, d], k/v [b, S, hkv, d] -> out like q.

    stage_events: optional list of MOBA_NUM_STAGES + 1 torch.cuda.Event(enable_timing=True)
    recorded around the stages on the current stream (with query_chunk: not supported).
    query_chunk: run the sparse stages over query chunks of this many tokens
    (a multiple of block_size) with one chunk's scratch (moba_prefill_chunked).
    """
    _need_cuda(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, S, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [batch, seqlen, num_kv_heads, head_dim]")
    dt = _dtype_code(q)
    if query_chunk is None:
        pb, _ = moba_workspace_size(b, S, hq, hkv, d, block_size, topk, dt)
    else:
        pb = moba_workspace_size_chunked(b, S, hq, hkv, d, block_size, topk, query_chunk, dt)
    ws = _workspace(pb, q.device, workspace)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda(out)
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q in shape and dtype")
    if query_chunk is not None:
        if stage_events is not None:
            raise ValueError("stage_events are not recorded by the chunked prefill")
        _check(lib().moba_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), b, S, hq, hkv,
                                          d, block_size, topk, dt, query_chunk, _ptr(ws),
                                          _nbytes(ws), _stream()),
               "moba_prefill_chunked")
        return out
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), b, S, hq, hkv, d, block_size, topk, dt,
            _ptr(ws), _nbytes(ws), _stream())
    if stage_events is None:
        _check(lib().moba_prefill(*args), "moba_prefill")
    else:
        if len(stage_events) != MOBA_NUM_STAGES + 1:
            raise ValueError(f"need {MOBA_NUM_STAGES + 1} events")
        arr = (ctypes.c_void_p * (MOBA_NUM_STAGES + 1))()
        for i, e in enumerate(stage_events):
            e.record()          # make sure the HIP event exists before handing it over
            arr[i] = ctypes.c_void_p(e.cuda_event)
        _check(lib().moba_prefill_timed(*args, arr), "moba_prefill_timed")
    return out


def moba_prefill_noalloc(q, k, v, block_size, topk, out=None):
    """moba_prefill in the library's own per-GPU scratch array: the call takes no
    workspace and allocates nothing on the device (``out`` is allocated here
    only when not given).  Calls that may overlap on one GPU must be serialised."""
    _need_cuda(q, k, v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, S, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [batch, seqlen, num_kv_heads, head_dim]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda(out)
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q in shape and dtype")
    _check(lib().moba_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), b, S, hq, hkv, d,
                                      block_size, topk, dt, _stream()), "moba_prefill_noalloc")
    return out
