"""PyTorch autograd wrapper of the fused WTConv kernels.

Only x is saved for the backward pass: the subbands are recomputed on chip,
so no intermediate of the wavelet cascade is kept in device memory.
"""

import math

import torch

from . import binding

__all__ = ["WTConvFunction", "WTConv2d", "wtconv"]


def _activation(t, like=None):
    """t in a layout the library takes: unchanged if it is NCHW- or
    channels-last-contiguous (or, with `like`, copied into like's layout)."""
    if like is not None:
        cl = like.dim() == 4 and not like.is_contiguous() and like.is_contiguous(memory_format=torch.channels_last)
        return t.contiguous(memory_format=torch.channels_last) if cl else t.contiguous()
    if t.is_contiguous() or (t.dim() == 4 and t.is_contiguous(memory_format=torch.channels_last)):
        return t
    return t.contiguous()


class WTConvFunction(torch.autograd.Function):
    """impl = "fused" (the on-chip kernels) or "unfused" (the level-by-level
    baseline, whose kernels keep every band and level result in a device
    workspace while they run).  Channels-last inputs stay channels-last (the
    output and dx follow x's layout).  wl and sl may hold more than L levels;
    their gradients have the parameters' shapes, zero beyond level L."""

    @staticmethod
    def forward(ctx, x, w0, s0, b0, wl, sl, L, impl="fused"):
        if impl not in ("fused", "unfused"):
            raise ValueError(f"impl must be 'fused' or 'unfused', not {impl!r}")
        x = _activation(x)
        ctx.L, ctx.impl = L, impl
        ctx.save_for_backward(x, w0, s0, wl, sl)
        fwd = binding.wtconv_forward if impl == "fused" else binding.wtconv_forward_unfused
        return fwd(x, w0, s0, b0, wl, sl, L)

    @staticmethod
    def backward(ctx, g):
        x, w0, s0, wl, sl = ctx.saved_tensors
        L = ctx.L
        bwd = binding.wtconv_backward if ctx.impl == "fused" else binding.wtconv_backward_unfused
        r = bwd(x, _activation(g, like=x), w0, s0, wl, sl, L)
        dwl, dsl = r["dwl"], r["dsl"]
        if wl is not None and (dwl is None or dwl.shape[0] != wl.shape[0]):
            full = torch.zeros_like(wl)
            if L > 0:
                full[:L] = dwl
            dwl = full
        if sl is not None and (dsl is None or dsl.shape[0] != sl.shape[0]):
            full = torch.zeros_like(sl)
            if L > 0:
                full[:L] = dsl
            dsl = full
        return r["dx"], r["dw0"], r["ds0"], r["db0"], dwl, dsl, None, None


def wtconv(x, w0, s0, b0, wl, sl, L, impl="fused"):
    return WTConvFunction.apply(x, w0, s0, b0, wl, sl, L, impl)


class WTConv2d(torch.nn.Module):
    """Depthwise WTConv layer: same-size output, C channels, L levels, k x k kernels."""

    def __init__(self, channels, kernel_size=5, levels=1, device=None):
        super().__init__()
        if kernel_size % 2 != 1:
            raise ValueError("kernel_size must be odd")
        C, k, L = channels, kernel_size, levels
        f = dict(device=device, dtype=torch.float32)
        self.L = L
        self.w0 = torch.nn.Parameter(torch.randn(C, k, k, **f) / k)
        self.s0 = torch.nn.Parameter(torch.ones(C, **f))
        self.b0 = torch.nn.Parameter(torch.zeros(C, **f))
        self.wl = torch.nn.Parameter(torch.randn(max(L, 1), 4 * C, k, k, **f) / k)
        self.sl = torch.nn.Parameter(torch.full((max(L, 1), 4 * C), 0.1, **f))

    def forward(self, x):
        return wtconv(x, self.w0, self.s0, self.b0, self.wl, self.sl, self.L)
