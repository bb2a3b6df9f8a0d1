"""ctypes binding of libwtconv (include/wtconv.h): argument marshalling only.

Every entry point here has the name of the C function it calls.  Tensors are
PyTorch device tensors (PyTorch supplies device memory and the current
stream); all computation happens in the library's HIP kernels.  A missing
library raises immediately: there is no fallback path.
"""

import ctypes
import os

import torch

__all__ = [
    "WTCError", "load_library", "wtc_desc", "make_desc",
    "wtconv_forward", "wtconv_backward", "wtconv_forward_unfused", "wtconv_backward_unfused",
    "wtconv_backward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "wtconv_forward_workspace", "wtconv_backward_workspace",
    "wtconv_forward_unfused_workspace", "wtconv_backward_unfused_workspace",
    "wtconv_io_model_bytes", "wtconv_flops", "wtconv_status_string",
    "WTC_FP32", "WTC_BF16", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwtconv.so")

WTC_OK, WTC_EINVAL, WTC_ESHAPE, WTC_EDTYPE, WTC_EWORKSPACE, WTC_EHIP, WTC_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 8 << 20   # WTCONV_NOALLOC_SCRATCH_BYTES in include/wtconv.h
WTC_FP32, WTC_BF16 = 0, 1


class WTCError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {wtconv_status_string(status)} (status {status})")


class wtc_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int), ("W", ctypes.c_int),
                ("L", ctypes.c_int), ("k", ctypes.c_int), ("dtype", ctypes.c_int), ("layout", ctypes.c_int)]


_lib = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(wtc_desc)


def load_library(path=None):
    """Load libwtconv.so (built by memory_bound_cnn_amd.build); raises if missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libwtconv.so not found at {p}; run `python -m memory_bound_cnn_amd.build`")
    lib = ctypes.CDLL(p)
    lib.wtconv_status_string.restype = ctypes.c_char_p
    lib.wtconv_status_string.argtypes = [ctypes.c_int]
    for name in ("wtconv_forward_workspace", "wtconv_backward_workspace",
                 "wtconv_forward_unfused_workspace", "wtconv_backward_unfused_workspace"):
        f = getattr(lib, name)
        f.restype = _SZ
        f.argtypes = [_D]
    for name in ("wtconv_forward", "wtconv_forward_unfused"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    for name in ("wtconv_backward", "wtconv_backward_unfused"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.wtconv_backward_noalloc.restype = ctypes.c_int
    lib.wtconv_backward_noalloc.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.wtconv_base_correlation_workspace.restype = _SZ
    lib.wtconv_base_correlation_workspace.argtypes = [_D, ctypes.c_int]
    lib.wtconv_base_correlation.restype = ctypes.c_int
    lib.wtconv_base_correlation.argtypes = [_D, _P, _P, _P, ctypes.c_int, _P, _SZ, _P]
    lib.wtconv_io_model_bytes.restype = ctypes.c_double
    lib.wtconv_io_model_bytes.argtypes = [_D, ctypes.c_int, ctypes.c_int]
    lib.wtconv_flops.restype = ctypes.c_double
    lib.wtconv_flops.argtypes = [_D, ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def wtconv_status_string(status):
    return load_library().wtconv_status_string(int(status)).decode()


def make_desc(B, C, H, W, L, k, dtype="fp32", layout=0):
    """layout 0: NCHW; 1: channels-last (through NCHW copies in the workspace);
    2: channels-last read and written in place (no copies)."""
    dt = {"fp32": WTC_FP32, "bf16": WTC_BF16, torch.float32: WTC_FP32, torch.bfloat16: WTC_BF16}[dtype]
    return wtc_desc(int(B), int(C), int(H), int(W), int(L), int(k), dt, int(layout))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _layout_of(t):
    """0 for an NCHW-contiguous activation tensor, 1 for a channels-last one."""
    if t.is_contiguous():
        return 0
    if t.dim() == 4 and t.is_contiguous(memory_format=torch.channels_last):
        return 1
    raise ValueError("activation tensors must be contiguous in NCHW or in channels-last order")


def _check_tensor(t, name, dtypes, device, shape=None, layout=None):
    """layout None: a parameter (plain contiguous); else the activation layout
    every tensor of the call must share."""
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a CUDA tensor on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if layout is None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if layout is not None and _layout_of(t) != layout:
        raise ValueError(f"{name} must have the memory layout of x")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _desc_of(x, L, k, in_place=False):
    B, C, H, W = x.shape
    lay = _layout_of(x)
    return make_desc(B, C, H, W, L, k, x.dtype, 2 if (lay == 1 and in_place) else lay)


def _check_params(x, w0, s0, b0, wl, sl, L):
    B, C, H, W = x.shape
    k = w0.shape[-1]
    dev = x.device
    f32 = (torch.float32,)
    _check_tensor(x, "x", (torch.float32, torch.bfloat16), dev, layout=_layout_of(x))
    _check_tensor(w0, "w0", f32, dev, (C, k, k))
    _check_tensor(s0, "s0", f32, dev, (C,))
    _check_tensor(b0, "b0", f32, dev, (C,))
    if L > 0:
        if wl is None or sl is None:
            raise ValueError("wl and sl are required when L > 0")
        _check_tensor(wl, "wl", f32, dev)
        _check_tensor(sl, "sl", f32, dev)
        if wl.shape[0] < L or tuple(wl.shape[1:]) != (4 * C, k, k) or sl.shape[0] < L or sl.shape[1] != 4 * C:
            raise ValueError("wl must be [>=L, 4C, k, k] and sl [>=L, 4C]")
    return k


def _workspace(nbytes, device, workspace):
    """The caller's workspace if it is large enough, else a new one.  A given
    workspace must be a contiguous tensor on the call's device."""
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous CUDA tensor on {device}")
    if nbytes == 0:
        return None, 0
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, nbytes


def _fwd_common(fn_name, ws_name, x, w0, s0, b0, wl, sl, L, out, workspace, in_place=False):
    k = _check_params(x, w0, s0, b0, wl, sl, L)
    lib = load_library()
    d = _desc_of(x, L, k, in_place)
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out", (x.dtype,), x.device, x.shape, layout=_layout_of(x))
    ws, wsb = _workspace(getattr(lib, ws_name)(ctypes.byref(d)), x.device, workspace)
    st = getattr(lib, fn_name)(ctypes.byref(d), _ptr(x), _ptr(w0), _ptr(s0), _ptr(b0),
                               _ptr(wl if L > 0 else None), _ptr(sl if L > 0 else None),
                               _ptr(out), _ptr(ws), wsb, _stream(x.device))
    if st != WTC_OK:
        raise WTCError(st, fn_name)
    return out


def _grad_buffers(x, L, k, grads):
    """Output buffers of the weight gradients: new ones, or the caller's,
    checked for device, dtype, shape and contiguity (the library writes through
    these pointers)."""
    C = x.shape[1]
    f32 = dict(dtype=torch.float32, device=x.device)
    shapes = dict(dw0=(C, k, k), ds0=(C,), db0=(C,), dwl=(L, 4 * C, k, k), dsl=(L, 4 * C))
    if grads is None:
        return {name: (torch.empty(shp, **f32) if (L > 0 or name in ("dw0", "ds0", "db0")) else None)
                for name, shp in shapes.items()}
    out = {}
    for name, shp in shapes.items():
        t = grads.get(name)
        if L == 0 and name in ("dwl", "dsl"):
            out[name] = None
            continue
        if t is None:
            raise ValueError(f"grads[{name!r}] is required")
        _check_tensor(t, name, (torch.float32,), x.device, shp)
        out[name] = t
    return out


def _bwd_common(fn_name, ws_name, x, g, w0, s0, wl, sl, L, dx, grads, workspace, in_place=False):
    k = _check_params(x, w0, s0, None, wl, sl, L)
    _check_tensor(g, "g", (x.dtype,), x.device, x.shape, layout=_layout_of(x))
    lib = load_library()
    d = _desc_of(x, L, k, in_place)
    if dx is None:
        dx = torch.empty_like(x)
    _check_tensor(dx, "dx", (x.dtype,), x.device, x.shape, layout=_layout_of(x))
    grads = _grad_buffers(x, L, k, grads)
    args = [ctypes.byref(d), _ptr(x), _ptr(g), _ptr(w0), _ptr(s0),
            _ptr(wl if L > 0 else None), _ptr(sl if L > 0 else None), _ptr(dx),
            _ptr(grads["dw0"]), _ptr(grads["ds0"]), _ptr(grads["db0"]), _ptr(grads["dwl"]), _ptr(grads["dsl"])]
    if ws_name is None:
        # no workspace: the library's fixed scratch array of the current device
        with torch.cuda.device(x.device):
            st = getattr(lib, fn_name)(*args, _stream(x.device))
    else:
        ws, wsb = _workspace(getattr(lib, ws_name)(ctypes.byref(d)), x.device, workspace)
        st = getattr(lib, fn_name)(*args, _ptr(ws), wsb, _stream(x.device))
    if st != WTC_OK:
        raise WTCError(st, fn_name)
    out = dict(grads)
    out["dx"] = dx
    return out


def wtconv_forward(x, w0, s0, b0, wl, sl, L, out=None, workspace=None, in_place=False):
    """out = WTConv(x) on the current stream (fused kernels).  in_place: a
    channels-last x is read (and out written) where it is, without NCHW copies
    (layout 2; slower, no extra workspace)."""
    return _fwd_common("wtconv_forward", "wtconv_forward_workspace", x, w0, s0, b0, wl, sl, L, out, workspace,
                       in_place)


def wtconv_forward_unfused(x, w0, s0, b0, wl, sl, L, out=None, workspace=None):
    """Level-by-level baseline of :func:`wtconv_forward`."""
    return _fwd_common("wtconv_forward_unfused", "wtconv_forward_unfused_workspace", x, w0, s0, b0, wl, sl, L,
                       out, workspace)


def wtconv_backward(x, g, w0, s0, wl, sl, L, dx=None, grads=None, workspace=None, in_place=False):
    """Returns dict(dx, dw0, ds0, db0, dwl, dsl) for upstream gradient g (fused
    kernels).  in_place: as for :func:`wtconv_forward`."""
    return _bwd_common("wtconv_backward", "wtconv_backward_workspace", x, g, w0, s0, wl, sl, L, dx, grads,
                       workspace, in_place)


def wtconv_backward_noalloc(x, g, w0, s0, wl, sl, L, dx=None, grads=None, in_place=False):
    """:func:`wtconv_backward` without a workspace: the library allocates
    nothing (its scratch is a fixed per-GPU array of NOALLOC_SCRATCH_BYTES).
    Pass dx and grads to have no allocation on this side either.  Channels-last
    tensors need in_place=True (NCHW copies would not fit the scratch)."""
    return _bwd_common("wtconv_backward_noalloc", None, x, g, w0, s0, wl, sl, L, dx, grads, None, in_place)


def wtconv_backward_unfused(x, g, w0, s0, wl, sl, L, dx=None, grads=None, workspace=None):
    """Level-by-level baseline of :func:`wtconv_backward`."""
    return _bwd_common("wtconv_backward_unfused", "wtconv_backward_unfused_workspace", x, g, w0, s0, wl, sl, L,
                       dx, grads, workspace)


CORR_VALU, CORR_MFMA = 0, 1


def wtconv_base_correlation(x, g, k, impl=CORR_VALU, out=None, workspace=None):
    """c0[c, ky, kx] = sum over batch and pixels of g * x shifted by
    (ky - k//2, kx - k//2) (x zero outside): the base level's weight-gradient
    correlation alone.  impl CORR_VALU: vector-unit tiles; CORR_MFMA: matrix
    cores (bf16 NCHW planes, k <= 7, H and W <= 64)."""
    dev = x.device
    _check_tensor(x, "x", (torch.float32, torch.bfloat16), dev, layout=0)
    _check_tensor(g, "g", (x.dtype,), dev, x.shape, layout=0)
    B, C, H, W = x.shape
    lib = load_library()
    d = make_desc(B, C, H, W, 0, k, x.dtype, 0)
    if out is None:
        out = torch.empty((C, k, k), dtype=torch.float32, device=dev)
    _check_tensor(out, "out", (torch.float32,), dev, (C, k, k))
    ws, wsb = _workspace(lib.wtconv_base_correlation_workspace(ctypes.byref(d), int(impl)), dev, workspace)
    st = lib.wtconv_base_correlation(ctypes.byref(d), _ptr(x), _ptr(g), _ptr(out), int(impl), _ptr(ws), wsb,
                                     _stream(dev))
    if st != WTC_OK:
        raise WTCError(st, "wtconv_base_correlation")
    return out


def wtconv_base_correlation_workspace(B, C, H, W, k, dtype="fp32", impl=CORR_VALU):
    d = make_desc(B, C, H, W, 0, k, dtype, 0)
    return int(load_library().wtconv_base_correlation_workspace(ctypes.byref(d), int(impl)))


def _ws_query(name, B, C, H, W, L, k, dtype, layout=0):
    d = make_desc(B, C, H, W, L, k, dtype, layout)
    return int(getattr(load_library(), name)(ctypes.byref(d)))


def wtconv_forward_workspace(B, C, H, W, L, k, dtype="fp32", layout=0):
    return _ws_query("wtconv_forward_workspace", B, C, H, W, L, k, dtype, layout)


def wtconv_backward_workspace(B, C, H, W, L, k, dtype="fp32", layout=0):
    return _ws_query("wtconv_backward_workspace", B, C, H, W, L, k, dtype, layout)


def wtconv_forward_unfused_workspace(B, C, H, W, L, k, dtype="fp32", layout=0):
    return _ws_query("wtconv_forward_unfused_workspace", B, C, H, W, L, k, dtype, layout)


def wtconv_backward_unfused_workspace(B, C, H, W, L, k, dtype="fp32", layout=0):
    return _ws_query("wtconv_backward_unfused_workspace", B, C, H, W, L, k, dtype, layout)


def wtconv_io_model_bytes(B, C, H, W, L, k, dtype="fp32", impl=0, direction=0, layout=0):
    d = make_desc(B, C, H, W, L, k, dtype, layout)
    return float(load_library().wtconv_io_model_bytes(ctypes.byref(d), int(impl), int(direction)))


def wtconv_flops(B, C, H, W, L, k, dtype="fp32", direction=0):
    d = make_desc(B, C, H, W, L, k, dtype)
    return float(load_library().wtconv_flops(ctypes.byref(d), int(direction)))
