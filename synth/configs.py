"""The synthetic MoBA prefill workloads (1K to 10M tokens).

(S, block, top-k) at 128K and 1M tokens follow the long-context model of the
MoBA tech-report write-up (block size 4096, top-k 12, attention sparsity
95.31% at 1M and 62.5% in the 128K-scale RULER evaluation; write-up section
"大語言模型評估").  Head shapes and the planting recipe are this project's
synthetic stand-ins: no dataset or trained weights are used.

The 10M-token workload is the length at which the write-up's section
"效率和可擴展性" reports its speed-up over standard FlashAttention; it keeps
the 1M workload's heads, block size, top-k and planting, and is generated
in 1M-token slices (``gen_slice``) so that no fp32 copy of Q is needed.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    hq: int
    hkv: int
    seqlen: int
    head_dim: int
    dtype: str           # "fp32" or "bf16"
    block_size: int
    topk: int            # counts the query's own block
    planted: int         # planted high-affinity blocks per (batch, KV head)
    shift_prob: float    # probability that a later query is shifted towards a planted block
    seed: int
    gen_slice: int = 0   # > 0: draw the tensors in slices of this many tokens

    @property
    def n_blocks(self) -> int:
        return -(-self.seqlen // self.block_size)

    @property
    def group(self) -> int:
        return self.hq // self.hkv


CONFIGS = [
    Config("moba-1k-fp32-d64", 1, 2, 2, 1024, 64, "fp32", 128, 3, 1, 0.25, 1001),
    Config("moba-8k-b2-h8-d128", 2, 8, 8, 8192, 128, "bf16", 512, 3, 2, 0.20, 1002),
    Config("moba-32k-h32-d128", 1, 32, 32, 32768, 128, "bf16", 512, 3, 4, 0.20, 1003),
    Config("moba-128k-gqa32x8-d128", 1, 32, 8, 131072, 128, "bf16", 4096, 12, 6, 0.20, 1004),
    Config("moba-1m-gqa32x8-d128", 1, 32, 8, 1048576, 128, "bf16", 4096, 12, 16, 0.20, 1005),
    Config("moba-10m-gqa32x8-d128", 1, 32, 8, 10485760, 128, "bf16", 4096, 12, 16, 0.20, 1006,
           gen_slice=1 << 20),
]


# Packed variable-length batches: (per-sequence recipe, sequence lengths).  The
# lengths mix long and short prompts, each ending in a short block, for about
# 1M tokens in all; every sequence uses the 1M workload's heads, block size,
# top-k and planting (capped by its own block count).
VARLEN_WORKLOADS = {
    "moba-varlen-1m-gqa32x8-d128": (
        Config("moba-varlen-1m-gqa32x8-d128", 1, 32, 8, 0, 128, "bf16", 4096, 12, 16, 0.20,
               1007),
        [393216 + 1984, 262144 + 640, 196608 + 3072, 131072 + 64, 65536 + 2048, 32768 + 192,
         4096 + 960]),
}


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
