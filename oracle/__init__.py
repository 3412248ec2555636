"""CPU oracle for the MX block-scaled linear layer (TEST INFRASTRUCTURE ONLY).

Only the test-suite, the package smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never links or calls it, and it shares no code with it.

The arithmetic lives in ``mx_oracle.c`` (plain C, fp64); this module is a thin numpy/ctypes
driver around it.  Format and rule sources are listed in the C file's header: the vLLM API pages
``compressed_tensors_w8a8_mxfp8`` (MXFP8 format: E4M3 values, uint8 E8M0 scales per 32 along K),
``aiter_flydsl`` (row-major [M, K/32] activation scales, bf16 output, bias after the GEMM, the
(16, 16) weight shuffle in ``row_major_weight``) and ``mxfp6`` (E2M3 / E3M2 weights), plus the
OCP MX v1.0 conversion rule that the pages rely on without stating.

Parity pins: every function here is checked in ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines or the pages' own printed inverse; the Inf/NaN-block convention,
which no workload exercises, against torch's E8M0 and E4M3FN formats (the block dequantizes to
NaN).
"""
from .oracle import *  # noqa: F401,F403
from .oracle import __all__  # noqa: F401
