"""CPU oracle for layer-wise 4-bit weight quantization (RTN and GPTQ).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import anything here.  The GPU library
never calls into it, and this package imports nothing from the GPU library.

Everything is plain numpy in float64, written from the method's description on
the source pages; see ``pwq_oracle`` for the functions and what pins each one.
"""
from .pwq_oracle import *  # noqa: F401,F403
