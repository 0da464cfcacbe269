"""The five synthetic workloads (shapes of the pages' DeepSeek-V3.2 indexer:
64 indexer heads x head_dim 128, one shared fp8 K per position, paged
block_size 64, index_topk 2048 at full size).

  prefill-1k        one request, T = S = 1024 causal, k = 256
  decode-64x16k-32k 64 decode requests, lengths uniform in [16384, 32768]
  prefill-24k+8k    one request, 24576 cached + 8192 new tokens (chunked prefill)
  decode-8x128k     8 decode requests at 131072, 200 planted hot positions each
  stack-16L-32x64k  16 layers, pattern FSSS x4, 32 decode requests at 65536

Seeds are 101..105 in that order.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    kind: str                   # "prefill" | "decode"
    num_reqs: int
    new_tokens: int             # per request
    len_lo: int                 # sequence length range (inclusive); lo == hi for fixed
    len_hi: int
    k: int
    pool_factor: float          # physical pool = factor x blocks needed
    num_layers: int = 1
    pattern: str = "F"
    planted: int = 0            # hot positions per request, K row x3 before rounding
    n_heads: int = 64
    head_dim: int = 128
    block_size: int = 64


CONFIGS = {
    "prefill-1k": WorkloadSpec("prefill-1k", 101, "prefill", 1, 1024, 1024, 1024, 256, 1.0),
    "decode-64x16k-32k": WorkloadSpec("decode-64x16k-32k", 102, "decode", 64, 1, 16384, 32768, 2048, 1.125),
    "prefill-24k+8k": WorkloadSpec("prefill-24k+8k", 103, "prefill", 1, 8192, 32768, 32768, 2048, 1.0),
    "decode-8x128k": WorkloadSpec("decode-8x128k", 104, "decode", 8, 1, 131072, 131072, 2048, 1.125,
                                  planted=200),
    "stack-16L-32x64k": WorkloadSpec("stack-16L-32x64k", 105, "decode", 32, 1, 65536, 65536, 2048, 1.125,
                                     num_layers=16, pattern="FSSS" * 4),
}


def get(name):
    return CONFIGS[name]
