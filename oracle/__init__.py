"""CPU oracle for the CODA GEMM+epilogue path (test infrastructure).

Plain, slow numpy evaluations of what the fused GPU path computes, written
from the CODA paper (arXiv 2605.19269, §3.1 primitives and §3.2.1
GEMM-Residual-RMSNorm-GEMM reparameterisation) and from the textbook
definitions of RMSNorm, SwiGLU, RoPE, QK-norm and softmax cross-entropy.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP path and never imports it.

Every function is pinned by tests/test_oracle_*.py against something other
than itself (brute force, closed forms, finite differences, torch CPU library
routines, exhaustive format round trips).
"""
from . import numerics, ops, block, mx  # noqa: F401
