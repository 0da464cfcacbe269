"""CPU oracle for the DeepSeek-V3.2 DSA lightning-indexer path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library (no kernels, headers,
tables or helpers) and the library never imports it.

Precision: fp64 for scores, exact integer arithmetic for the fp8 codec, a
stable full sort for top-k.  The weight fold is done in fp32 because the
pages compute it on an fp32 torch tensor.

Modules
  e4m3      OCP 8-bit float E4M3 encode / decode
  e2m1      OCP 4-bit float E2M1 encode / decode, E8M0 scales
  fp4cache  the FP4 indexer K cache: per-32 quantiser, block layout,
            scatter / gather and its score
  quant     ue8m0 per-128 quantisation, paged-cache scatter, q quantisation
            and weight fold
  paged     the byte layout of one paged K-cache block and gathers through
            a block table
  logits    the lightning-indexer score I[t, s]
  topk      per-row top-k with lower-index tie-break
  schedule  IndexCache F/S layer schedule
  stack     a multi-layer run that reuses the top-k buffer on S layers
  physical  logical -> physical top-k index conversion

Every function names the passage of the pages it follows.  Where the pages
are silent the reading adopted is stated in the docstring.  Functions whose
result no independent pin covers say "parity unpinned".
"""

from . import e4m3, e2m1, quant, paged, logits, fp4cache, topk, schedule, stack, physical  # noqa: F401
from .batch import Batch  # noqa: F401
