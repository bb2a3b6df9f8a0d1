"""Parity of the fused HIP path (through the C ABI) with the float64 oracle.

Element-by-element comparisons at sizes the oracle finishes in seconds (several
8x8 blocks per plane, ragged tails, every plane-size class the launch planner
distinguishes), and full-size launches at every benchmark shape (out and dx on sampled batch
entries, every weight gradient over the whole batch).
Tolerance per tensor: max|gpu - oracle| <= 1e-4 * RMS(oracle) for float32
storage and 2e-2 * RMS(oracle) for bfloat16 storage.
"""

import functools
import hashlib
import os

import numpy as np
import pytest
import torch

import oracle
from memory_bound_cnn_amd import binding
from memory_bound_cnn_amd.inputs import WORKLOADS, workload_inputs
from tests.gpu_helpers import (check_all, dev, host, inputs, oracle_ref, rel_err, run_fused, to_dev)

pytestmark = pytest.mark.gpu


def _case(B, C, H, W, L, k, seed, dtype="fp32", impl="fused"):
    d = inputs(B, C, H, W, L, k, seed, dtype)
    t = to_dev(d, dtype, L)
    out, gr = run_fused(t, L, impl)
    ref_out, ref_gr = oracle_ref(d, L)
    return check_all(out, gr, ref_out, ref_gr, dtype, f"{impl} B{B} C{C} {H}x{W} L{L} k{k} {dtype}")


# Reduced-batch versions of every benchmark shape (same plane size, level count,
# kernel and dtype, hence the same kernel variant and LDS layout).
REDUCED = [
    (1, 8, 32, 32, 2, 5, 0, "fp32"),       # tiny workload, full size
    (2, 6, 64, 64, 3, 5, 10, "fp32"),      # stage-1 plane
    (3, 8, 32, 32, 3, 5, 20, "bf16"),      # bf16 storage
    (1, 3, 128, 128, 1, 5, 30, "fp32"),    # level sweep planes
    (1, 3, 128, 128, 3, 5, 31, "fp32"),
    (1, 2, 128, 128, 5, 5, 32, "fp32"),
    (2, 2, 112, 112, 2, 5, 33, "fp32"),    # the LL band of the 224x224 planes (peeled path)
    (5, 8, 14, 14, 2, 5, 40, "fp32"),      # odd 14x14
    (9, 8, 7, 7, 1, 5, 41, "fp32"),        # odd 7x7
    (1, 3, 128, 128, 0, 5, 34, "fp32"),    # the depthwise convs WTConv is compared with, on sweep planes
    (1, 3, 128, 128, 0, 7, 35, "fp32"),
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", REDUCED)
def test_reduced_workloads(B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype)


EDGE = [
    (2, 3, 16, 16, 0, 5, 50),      # L = 0: plain depthwise conv
    (2, 3, 13, 10, 3, 3, 51),      # odd, unequal sides, k = 3
    (1, 2, 7, 5, 3, 5, 52),        # deeper than the plane (tail levels)
    (1, 2, 3, 3, 5, 3, 53),        # tail levels on a 1x1 grid
    (2, 2, 1, 1, 2, 5, 54),        # 1x1 planes: every level is a tail level
    (1, 2, 9, 17, 2, 7, 55),       # k = 7, ragged blocks
    (2, 4, 24, 24, 2, 1, 56),      # k = 1
    (1, 2, 40, 24, 4, 5, 57),      # several quad blocks, 4 levels
    (3, 5, 8, 8, 3, 5, 58),        # one block per plane, three levels
    (1, 1, 100, 36, 2, 5, 59),     # 100 quad blocks -> 512-thread plan
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed", EDGE)
def test_edge_cases(B, C, H, W, L, k, seed):
    _case(B, C, H, W, L, k, seed)


# Planes of at most 8 x 8 with k = 5 and 1 <= L <= 2 take the register-resident
# kernel (one quad of lanes per plane): full and partial quads, both levels,
# unequal and tiny sides.
TINY = [
    (3, 5, 8, 8, 2, 5, 70, "fp32"),
    (2, 3, 5, 7, 1, 5, 71, "fp32"),
    (4, 6, 8, 3, 2, 5, 72, "fp32"),
    (17, 2, 7, 7, 2, 5, 73, "fp32"),
    (3, 4, 7, 7, 2, 5, 74, "bf16"),
    (5, 3, 2, 2, 1, 5, 75, "fp32"),
    # 7 x 7 with one level: one plane per lane, 64 batch entries per wave
    (70, 3, 7, 7, 1, 5, 76, "fp32"),       # a full and a partial wave per channel
    (5, 4, 7, 7, 1, 5, 77, "bf16"),
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", TINY)
def test_tiny_planes(B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype)


# Planes without a fixed-geometry instance whose rows are whole 4-pixel vectors
# (at most 128 quad blocks) take the runtime-geometry kernel with direct loads:
# both storage types, the shallow (Lm <= 3) and deep accumulator classes, k = 3,
# 5 and 7, rows wider than one 64-lane copy, ragged heights.
RUNTIME_DL = [
    (3, 4, 32, 32, 3, 5, 80, "fp32"),      # (fixed-geometry instance, like 64x64 L3 bf16 below)
    (3, 4, 32, 32, 4, 5, 88, "fp32"),      # Lm = 4
    (2, 4, 48, 48, 3, 5, 81, "fp32"),
    (2, 3, 40, 72, 4, 5, 82, "fp32"),      # Wq = 80: two row chunks; Lm = 4
    (2, 4, 64, 64, 3, 5, 83, "bf16"),
    (2, 4, 64, 64, 2, 5, 89, "bf16"),
    (2, 3, 36, 44, 5, 3, 84, "bf16"),      # k = 3, five levels
    (2, 2, 56, 56, 2, 7, 85, "fp32"),      # k = 7
    (3, 2, 30, 100, 2, 5, 86, "fp32"),     # ragged height, Wq = 104
    (2, 3, 64, 64, 6, 5, 87, "bf16"),      # Lm = 6
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", RUNTIME_DL)
def test_runtime_geometry_direct_loads(B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype)


# Planes smaller than the fixed-geometry instance they run on (zero-extended
# to its size): the prefetch covers fewer units, rows past the plane are
# dropped by the output resource's range check, and the backward stages its
# planes without the next-plane loads.
PARTIAL_FIXED = [
    (2, 3, 124, 124, 1, 5, 90, "fp32"),    # 128x128 instance, one level (early commit)
    (1, 3, 124, 124, 3, 5, 91, "fp32"),    # 128x128 instance, three levels
    (1, 2, 124, 120, 5, 5, 92, "fp32"),    # 128x128 instance, five levels, unequal sides
    (2, 2, 108, 108, 2, 5, 93, "fp32"),    # 112x112 instance
    (3, 4, 28, 28, 3, 5, 94, "bf16"),      # bf16 32x32 instance
    (2, 3, 124, 124, 0, 5, 95, "fp32"),    # depthwise conv on the 128x128 instance
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", PARTIAL_FIXED)
def test_partial_fixed_geometry(B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype)


def test_bf16_odd_plane():
    _case(3, 4, 14, 14, 2, 5, 60, "bf16")


def test_batch_not_multiple_of_planes_per_workgroup():
    # 7x7 planes run many planes per workgroup; B leaves a ragged last chunk
    _case(37, 3, 7, 7, 1, 5, 61)


def test_deterministic():
    d = inputs(4, 6, 32, 32, 3, 5, 62)
    t = to_dev(d)
    a_out, a = run_fused(t, 3)
    b_out, b = run_fused(t, 3)
    assert torch.equal(a_out, b_out)
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key


def test_adjoint_dot_on_gpu():
    """<g, out(x) - out(0)> = <dx, x> using GPU results only."""
    B, C, H, W, L, k = 2, 4, 32, 32, 3, 5
    d = inputs(B, C, H, W, L, k, 63)
    t = to_dev(d)
    out, gr = run_fused(t, L)
    t0 = dict(t)
    t0["x"] = torch.zeros_like(t["x"])
    out0 = binding.wtconv_forward(t0["x"], t["w0"], t["s0"], t["b0"], t["wl"], t["sl"], L)
    lhs = (host(t["g"]).astype(np.float64) * (host(out) - host(out0))).sum()
    rhs = (host(gr["dx"]).astype(np.float64) * host(t["x"])).sum()
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + abs(rhs) + 1.0)


def test_finite_differences_tiny():
    """Every parameter gradient (and some input coordinates) on the tiny
    workload by exact central differences of <g, out> with h = 1, using only
    the GPU forward: the loss is affine in each single coordinate."""
    wl_ = WORKLOADS["tiny_b1c8_32x32_L2"]
    d = workload_inputs(wl_)
    L = wl_.L
    t = to_dev(d)
    gr = binding.wtconv_backward(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L)
    g64 = d["g"].astype(np.float64)

    def loss(tt):
        o = binding.wtconv_forward(tt["x"], tt["w0"], tt["s0"], tt["b0"], tt["wl"], tt["sl"], L)
        return float((host(o).astype(np.float64) * g64).sum())

    names = dict(w0="dw0", s0="ds0", b0="db0", wl="dwl", sl="dsl")
    for name, gname in names.items():
        base = t[name]
        flat = base.view(-1)
        fd = np.zeros(flat.numel())
        for i in range(flat.numel()):
            old = float(flat[i])
            flat[i] = old + 1.0
            lp = loss(t)
            flat[i] = old - 1.0
            lm = loss(t)
            flat[i] = old
            fd[i] = (lp - lm) / 2.0
        got = host(gr[gname]).ravel()
        assert rel_err(got, fd) <= 1e-3, (name, rel_err(got, fd))
    # dx at the four corners and at random pixels
    xf = t["x"].view(-1)
    H, W = wl_.H, wl_.W
    idxs = [0, W - 1, (H - 1) * W, H * W - 1] + list(np.random.default_rng(0).integers(0, xf.numel(), 12))
    gdx = host(gr["dx"]).ravel()
    rms = np.sqrt(np.mean(gdx ** 2))
    for i in idxs:
        old = float(xf[i])
        xf[i] = old + 1.0
        lp = loss(t)
        xf[i] = old - 1.0
        lm = loss(t)
        xf[i] = old
        assert abs((lp - lm) / 2.0 - gdx[i]) <= 1e-3 * rms, i


FULL = ["stage1_b32c96_64x64_L3", "bf16_b64c192_32x32_L3", "odd_b128c384_14x14_L2", "odd_b128c768_7x7_L1",
        "large_b8c64_224x224_L3"]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize_weight_grads.npz")


@functools.lru_cache(maxsize=1)
def _golden_file():
    return np.load(GOLDEN)   # written by tests/golden/make_fullsize_grads.py (oracle only)


def _golden(case):
    z = _golden_file()
    out = {k: z[f"{case}|{k}"] for k in ("dw0", "ds0", "db0", "dwl", "dsl") if f"{case}|{k}" in z.files}
    return out, str(z[f"{case}|inputs_sha256"])


def _inputs_sha256(d, L):
    h = hashlib.sha256()
    for key in ("x", "g", "w0", "s0", "b0", "wl", "sl"):
        v = d[key]
        if key in ("wl", "sl"):
            v = v[:L] if (v is not None and L > 0) else None
        h.update(key.encode())
        if v is not None:
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


def _full_size(wl_, L):
    """Full-size launch in the benchmark's launch configuration, with the real
    upstream gradient over the whole batch.  out and dx are compared with the
    oracle on two sampled batch entries; the weight gradients -- reductions
    over all B*H*W positions of every channel -- with the oracle's values for
    the whole batch (tests/golden/fullsize_weight_grads.npz, computed from the
    same seeded inputs, whose hash is checked first)."""
    d = workload_inputs(wl_)
    case = f"{wl_.name}_L{L}"
    ref_w, sha = _golden(case)
    assert _inputs_sha256(d, L) == sha, f"{case}: seeded inputs differ from the ones the golden values came from"
    rng = np.random.default_rng(7)
    batch = np.sort(rng.choice(wl_.B, size=2, replace=False))
    t = to_dev(d, wl_.dtype, L)
    if L < (t["wl"].shape[0] if t["wl"] is not None else 0):
        t["wl"], t["sl"] = t["wl"][:L].contiguous(), t["sl"][:L].contiguous()
    out, gr = run_fused(t, L)
    o = host(out)[batch]
    dxs = host(gr["dx"])[batch]
    del out, t
    dd = dict(d)
    dd["x"], dd["g"] = d["x"][batch], d["g"][batch]
    ref_out, ref_gr = oracle_ref(dd, L)
    tol = 1e-4 if wl_.dtype == "fp32" else 2e-2
    errs = {"out": rel_err(o, ref_out), "dx": rel_err(dxs, ref_gr["dx"])}
    for k, ref in ref_w.items():
        errs[k] = rel_err(host(gr[k]), ref)
    assert set(errs) >= {"dw0", "ds0", "db0"} and (L == 0 or {"dwl", "dsl"} <= set(errs)), errs
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{case}: {bad} (all {errs})"


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    wl_ = WORKLOADS[name]
    _full_size(wl_, wl_.L)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 5])
def test_full_size_sweep(L):
    _full_size(WORKLOADS["sweep_b64c96_128x128"], L)


@pytest.mark.parametrize("k", [5, 7])
def test_full_size_dwconv(k):
    """The plain depthwise-conv paths that WTConv is timed against: L = 0 at the
    headline block shape, k = 5 and k = 7, in the benchmark's launch configuration."""
    import dataclasses
    wl_ = dataclasses.replace(WORKLOADS["stage1_b32c96_64x64_L3"], name=f"stage1_L0_k{k}", L=0, k=k, L_max=0,
                              sweep=())
    _full_size(wl_, 0)


# Kernel sizes 9..31: no fused kernel holds their k^2 weights and accumulators
# in registers, so the fused entry points run the level-by-level kernels with
# the taps looped at run time.  Both entry points, small and large planes (the
# 64 x 64-tile threshold), bf16, L = 0, a kernel larger than the plane.
LARGE_K = [
    (2, 3, 32, 32, 2, 9, 120, "fp32"),
    (1, 2, 50, 60, 3, 11, 121, "fp32"),
    (2, 2, 20, 14, 1, 9, 122, "bf16"),
    (2, 3, 16, 16, 0, 13, 123, "fp32"),
    (1, 2, 9, 7, 3, 15, 124, "fp32"),
    (1, 1, 40, 33, 1, 31, 125, "fp32"),
]


@pytest.mark.parametrize("impl", ["fused", "unfused"])
@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", LARGE_K)
def test_large_kernel_sizes(impl, B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype, impl)


# Planes beyond the on-chip pipeline: level 1 and the base conv level by level,
# the LL band recursively (fused once it fits).
LARGE = [
    (2, 3, 200, 150, 3, 5, 80, "fp32"),    # one peel, LL 100x75 fused with 2 levels
    (1, 2, 300, 260, 4, 3, 81, "fp32"),    # two peels (150x130 is still too large), k = 3
    (2, 2, 160, 144, 2, 5, 82, "bf16"),    # bf16 storage at the top, fp32 LL below
    (1, 2, 260, 130, 0, 7, 83, "fp32"),    # L = 0: the plain depthwise conv
    (2, 2, 140, 141, 1, 5, 84, "fp32"),    # L = 1: nothing below the peeled level, ragged side
    (1, 2, 257, 129, 9, 5, 85, "fp32"),    # levels deeper than the plane (tail), odd sides
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", LARGE)
def test_large_planes(B, C, H, W, L, k, seed, dtype):
    _case(B, C, H, W, L, k, seed, dtype)


# Channels-last (NHWC) tensors: through NCHW copies in the workspace (layout 1,
# both implementations), or read and written in place by the fused plane
# pipeline for every plane it holds (layout 2: one (batch chunk, channel) unit
# per workgroup; planes beyond it are adapted).  Every staging path of the pipeline: DMA rows
# (fp32, fixed and runtime geometry), register prefetch and synchronous
# staging (bf16, rows not a multiple of 4 pixels), two blocks per quad.
CHANNELS_LAST = [
    (2, 6, 64, 64, 3, 5, 90, "fp32"),      # fixed geometry, DMA rows
    (2, 5, 32, 32, 3, 5, 91, "bf16"),      # bf16: staged through registers
    (3, 7, 14, 14, 2, 5, 92, "fp32"),      # several planes per workgroup, rows of 14 pixels
    (5, 20, 7, 7, 1, 5, 93, "fp32"),       # the 7 x 7 class in the plane pipeline
    (1, 3, 200, 150, 2, 5, 94, "fp32"),    # peeled plane: adapted through NCHW copies
    (3, 4, 48, 48, 3, 5, 96, "fp32"),      # runtime geometry, DMA rows
    (2, 3, 13, 10, 3, 3, 97, "fp32"),      # ragged, k = 3
    (1, 2, 128, 128, 2, 5, 98, "fp32"),    # two blocks per quad
    (2, 4, 64, 64, 2, 5, 99, "bf16"),      # bf16 64 x 64
    (4, 3, 24, 24, 0, 7, 100, "fp32"),     # L = 0, k = 7
    (35, 17, 8, 8, 2, 5, 101, "fp32"),     # many units, odd channel count
    (2, 8, 32, 32, 3, 5, 102, "bf16"),     # 16-byte transposes of bf16 (channels a multiple of 8)
]


@pytest.mark.parametrize("impl", ["fused", "fused_in_place", "unfused"])
@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", CHANNELS_LAST)
def test_channels_last(impl, B, C, H, W, L, k, seed, dtype):
    d = inputs(B, C, H, W, L, k, seed, dtype)
    t = to_dev(d, dtype, L)
    for key in ("x", "g"):
        t[key] = t[key].contiguous(memory_format=torch.channels_last)
    if impl == "fused_in_place":
        out = binding.wtconv_forward(t["x"], t["w0"], t["s0"], t["b0"], t["wl"], t["sl"], L, in_place=True)
        gr = binding.wtconv_backward(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L, in_place=True)
        torch.cuda.synchronize()
    else:
        out, gr = run_fused(t, L, impl)
    if C > 1 and H * W > 1:
        assert not out.is_contiguous() and out.is_contiguous(memory_format=torch.channels_last)
    ref_out, ref_gr = oracle_ref(d, L)
    check_all(out, gr, ref_out, ref_gr, dtype, f"channels-last {impl} B{B} C{C} {H}x{W} L{L} {dtype}")


def test_mixed_layouts_rejected():
    d = inputs(1, 3, 16, 16, 1, 5, 95)
    t = to_dev(d, "fp32", 1)
    g_cl = t["g"].contiguous(memory_format=torch.channels_last)
    with pytest.raises(ValueError):
        binding.wtconv_backward(t["x"], g_cl, t["w0"], t["s0"], t["wl"], t["sl"], 1)


def test_channels_last_full_size():
    """The 32 x 96 x 64 x 64, L = 3 block in channels-last at full size, through
    NCHW copies and in place: out and dx bit-identical to the NCHW call (same
    arithmetic per plane, only the addressing differs), weight gradients
    against the whole-batch oracle."""
    wl_ = WORKLOADS["stage1_b32c96_64x64_L3"]
    L = wl_.L
    d = workload_inputs(wl_)
    ref_w, sha = _golden(f"{wl_.name}_L{L}")
    assert _inputs_sha256(d, L) == sha
    t = to_dev(d, wl_.dtype, L)
    out_n, gr_n = run_fused(t, L)
    tc = dict(t)
    for key in ("x", "g"):
        tc[key] = t[key].contiguous(memory_format=torch.channels_last)
    for in_place in (False, True):
        out_c = binding.wtconv_forward(tc["x"], t["w0"], t["s0"], t["b0"], t["wl"], t["sl"], L, in_place=in_place)
        gr_c = binding.wtconv_backward(tc["x"], tc["g"], t["w0"], t["s0"], t["wl"], t["sl"], L, in_place=in_place)
        torch.cuda.synchronize()
        assert out_c.is_contiguous(memory_format=torch.channels_last)
        assert torch.equal(out_c.contiguous(), out_n), in_place
        assert torch.equal(gr_c["dx"].contiguous(), gr_n["dx"]), in_place
        errs = {k: rel_err(host(gr_c[k]), ref) for k, ref in ref_w.items()}
        assert all(v <= 1e-4 for v in errs.values()), (in_place, errs)
