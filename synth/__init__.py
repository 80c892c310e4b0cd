"""Seeded synthetic inputs for MoBA prefill (shared by the tests and the bench).

This module holds the workload shapes and the input recipe only.  It does none
of the method's arithmetic (no pooling, gating, selection or attention): both
the GPU library and the CPU oracle receive the tensors it makes and nothing
else from it.
"""
from .configs import CONFIGS, VARLEN_WORKLOADS, Config, config_by_name
from .gen import make_inputs, make_varlen_inputs, sample_rows, to_oracle_array

__all__ = ["CONFIGS", "VARLEN_WORKLOADS", "Config", "config_by_name", "make_inputs", "make_varlen_inputs",
           "sample_rows", "to_oracle_array"]
