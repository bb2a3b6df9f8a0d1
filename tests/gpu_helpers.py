"""Shared helpers for the GPU tests: move seeded inputs to the device, run the
library through the C ABI, compare against the float64 oracle."""

import numpy as np
import torch

import oracle
from memory_bound_cnn_amd import binding
from memory_bound_cnn_amd.inputs import make_inputs

TOL = {"fp32": 1e-4, "bf16": 2e-2}   # max|err| <= TOL * RMS(reference), per tensor
GRAD_KEYS = ("dx", "dw0", "ds0", "db0", "dwl", "dsl")


def dev():
    return torch.device("cuda", 0)


def to_dev(d, dtype="fp32", L=None):
    """NumPy input dict -> device tensors (x, g in the storage dtype)."""
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for key, v in d.items():
        if v is None:
            out[key] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if key in ("x", "g"):
            t = t.to(sd)
        out[key] = t.to(dev())
    if L is not None and L == 0:
        out["wl"] = out["sl"] = None
    return out


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    return err / rms if rms > 0 else err


def host(t):
    return None if t is None else t.float().cpu().numpy()


def run_fused(t, L, impl="fused"):
    fwd = binding.wtconv_forward if impl == "fused" else binding.wtconv_forward_unfused
    bwd = binding.wtconv_backward if impl == "fused" else binding.wtconv_backward_unfused
    out = fwd(t["x"], t["w0"], t["s0"], t["b0"], t["wl"], t["sl"], L)
    gr = bwd(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L)
    torch.cuda.synchronize()
    return out, gr


def oracle_ref(d, L, batch=None):
    x, g = d["x"], d["g"]
    if batch is not None:
        x, g = x[batch], g[batch]
    wl = None if d["wl"] is None or L == 0 else d["wl"][:L]
    sl = None if d["sl"] is None or L == 0 else d["sl"][:L]
    out = oracle.forward(x, d["w0"], d["s0"], d["b0"], wl, sl, L, batch_chunk=8)
    gr = oracle.backward(x, g, d["w0"], d["s0"], d["b0"], wl, sl, L, batch_chunk=8)
    return out, gr


def check_all(out, gr, ref_out, ref_gr, dtype, label, batch=None, keys=GRAD_KEYS):
    tol = TOL[dtype]
    errs = {}
    o = host(out)
    if batch is not None:
        o = o[batch]
    errs["out"] = rel_err(o, ref_out)
    for key in keys:
        if ref_gr.get(key) is None:
            continue
        got = host(gr[key])
        if key == "dx" and batch is not None:
            got = got[batch]
        errs[key] = rel_err(got, ref_gr[key])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: max|err|/RMS above {tol}: {bad} (all: {errs})"
    return errs


def inputs(B, C, H, W, L, k, seed, dtype="fp32", L_max=None):
    return make_inputs(B, C, H, W, L, k, seed, dtype, L_max)
