"""CPU oracle for WTConv (float64 NumPy).

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path never does.
"""
from .wtconv_oracle import (  # noqa: F401
    backward,
    corr,
    dwconv,
    forward,
    haar2_analysis,
    haar2_synthesis,
)
