"""WTConv for AMD Instinct MI355X (gfx950).

The operator runs in hand-written HIP kernels behind the C-ABI library
``libwtconv.so`` (declared in ``include/wtconv.h``).  ``binding`` marshals
arguments to that library; ``autograd`` wraps it as a PyTorch autograd
function.  Importing this package does not load the library; the binding
loads it on first use and raises if it is missing.
"""

__all__ = ["binding", "inputs"]
