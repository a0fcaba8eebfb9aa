"""CPU oracle for the DFlash block-diffusion drafter round. TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what one draft round computes. Only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the product path (the HIP library and its binding) never does, and
this package imports nothing from that path.

Modules:
  dflash  - numerics helpers (bf16 rounding, RMSNorm, RoPE, SiLU), the drafter
            forward (uncached definition), LM-head top-k, first-mismatch accept,
            INT4 unpacking.
  target  - a tiny causal target model and the speculative loop used for the
            losslessness check.

Parity status per function is stated in each docstring ("pinned by ..." or
"parity unpinned").
"""
from . import dflash, target  # noqa: F401
