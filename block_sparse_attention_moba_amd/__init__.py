"""MoBA (Mixture of Block Attention) causal prefill forward for AMD Instinct MI355X.

The work runs in libmoba.so (hand-written HIP for gfx950, C ABI in
include/moba.h); this package is its thin Python binding.
"""
from ._lib import (MOBA_DTYPE_BF16, MOBA_DTYPE_FP32, MOBA_NUM_STAGES, STAGE_NAMES, MobaError,
                   lib, moba_abi_version, moba_backward, moba_gate, moba_gate_scores, moba_pool,
                   moba_prefill,
                   moba_prefill_lse, moba_prefill_noalloc, moba_status_string,
                   moba_workspace_size_backward,
                   moba_prefill_varlen, moba_workspace_size, moba_workspace_size_chunked,
                   moba_workspace_size_varlen)

__all__ = ["MOBA_DTYPE_BF16", "MOBA_DTYPE_FP32", "MOBA_NUM_STAGES", "STAGE_NAMES", "MobaError",
           "lib", "moba_abi_version", "moba_backward", "moba_gate", "moba_gate_scores", "moba_pool",
           "moba_prefill",
           "moba_prefill_lse", "moba_prefill_noalloc", "moba_workspace_size_backward",
           "moba_prefill_varlen", "moba_status_string", "moba_workspace_size",
           "moba_workspace_size_chunked", "moba_workspace_size_varlen"]
