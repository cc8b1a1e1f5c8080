"""CPU oracle for the MXFP8 o_proj chain: test infrastructure only.

Plain, slow, float64 / exact-rational implementations written from the vLLM
pages on MXFP8 activations (PR #60118 and PR #57977).  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does, and this package imports nothing from the library.
"""
from . import chain_ref, mxfp8_ref, rmsnorm_ref  # noqa: F401
