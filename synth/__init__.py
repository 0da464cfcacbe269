"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package draws random numbers and lays out batch / paging metadata.  It
holds none of the indexer's arithmetic (no quantisation, no scores, no
selection): both the oracle and the HIP library consume the same raw inputs
(bf16 q and K bit patterns, raw fp32 head weights) and do their own work.
"""

from .configs import CONFIGS, WorkloadSpec, get  # noqa: F401
from .gen import Workload, make_workload, f32_to_bf16_bits, random_batch  # noqa: F401
