"""CPU oracle for the gathered affine-quantized MoE expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library or its Python binding.

Every function is the plain definition of what the method computes, written
out step by step in numpy (float64 for floating point unless a step fixes the
precision).  Citations name the source page and its section:

* [MLX#4509]  MLX issue 4509, "gather_qmm at M=1 streams 4-bit expert weights
  at ~half the bandwidth of M=4 (MoE decode)" -- the benchmark script.
* [MLX#4567]  MLX PR 4567, "[Metal] Gather mm improvement" -- description.
* [nuvec]     nuvec-core 0.4.0, tests/quantized.rs -- the named test functions.
* [MLX#4787]  MLX PR 4787, "Affine quantized_matmul at 3-16 rows on GPUs
  without NAX" -- the benchmark script.
* [MTPLX#558] MTPLX PR 558, "One-kernel MoE combine ..." -- Summary/Motivation.
"""
from .core import *  # noqa: F401,F403
