"""C-ABI checks that need no GPU: the library loads, exports every function
that include/wtconv.h declares, rejects bad arguments before any HIP call,
and reports workspace sizes, the I/O model and flop counts."""

import ctypes
import os
import re

import pytest

from memory_bound_cnn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "wtconv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wtconv_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    names = _declared()
    assert "wtconv_forward" in names and "wtconv_backward" in names
    for n in names:
        assert hasattr(lib, n), n


def _desc(**kw):
    a = dict(B=2, C=3, H=16, W=16, L=2, k=5, dtype=0, layout=0)
    a.update(kw)
    return binding.wtc_desc(a["B"], a["C"], a["H"], a["W"], a["L"], a["k"], a["dtype"], a["layout"])


FAKE = ctypes.c_void_p(16)   # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(k=4), binding.WTC_EINVAL), (dict(k=0), binding.WTC_EINVAL), (dict(L=-1), binding.WTC_EINVAL),
    (dict(B=0), binding.WTC_EINVAL), (dict(H=0), binding.WTC_EINVAL), (dict(dtype=7), binding.WTC_EDTYPE),
    (dict(layout=3), binding.WTC_EDTYPE),
    (dict(layout=1, H=512, W=512), binding.WTC_EWORKSPACE),   # channels-last beyond the pipeline: adapted
    (dict(H=512, W=512), binding.WTC_EWORKSPACE),
    (dict(k=33), binding.WTC_ESHAPE),
    (dict(k=9), binding.WTC_EWORKSPACE),   # k = 9..31 runs the level-by-level kernels: it needs a workspace
])
def test_forward_rejects(kw, status):
    lib = binding.load_library()
    d = _desc(**kw)
    st = lib.wtconv_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == status


def test_null_pointers_rejected():
    lib = binding.load_library()
    d = _desc()
    assert lib.wtconv_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == binding.WTC_EINVAL
    assert lib.wtconv_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == binding.WTC_EINVAL
    d0 = _desc(L=0)   # wl/sl may be NULL when L == 0 -- but here x is NULL
    assert lib.wtconv_forward(ctypes.byref(d0), None, FAKE, FAKE, FAKE, None, None, FAKE, None, 0, None) == binding.WTC_EINVAL
    assert lib.wtconv_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, FAKE, FAKE, 1 << 30, None) == binding.WTC_EINVAL
    assert lib.wtconv_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == binding.WTC_EINVAL


def test_backward_workspace_checked():
    lib = binding.load_library()
    d = _desc()
    need = lib.wtconv_backward_workspace(ctypes.byref(d))
    assert need > 0
    st = lib.wtconv_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, FAKE, need - 1, None)
    assert st == binding.WTC_EWORKSPACE
    st = lib.wtconv_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, None, need, None)
    assert st == binding.WTC_EWORKSPACE


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert binding.wtconv_status_string(s)
    assert "unknown" in binding.wtconv_status_string(42)


def test_io_model_fused_is_minimal_traffic():
    B, C, H, W, L, k = 32, 96, 64, 64, 3, 5
    N = B * C * H * W
    fwd = binding.wtconv_io_model_bytes(B, C, H, W, L, k, "fp32", 0, 0)
    bwd = binding.wtconv_io_model_bytes(B, C, H, W, L, k, "fp32", 0, 1)
    assert 2 * N * 4 <= fwd <= 2 * N * 4 * 1.01
    assert 3 * N * 4 <= bwd <= 3 * N * 4 * 1.03
    bf = binding.wtconv_io_model_bytes(B, C, H, W, L, k, "bf16", 0, 0)
    assert 2 * N * 2 <= bf <= 2 * N * 2 * 1.02
    assert binding.wtconv_io_model_bytes(B, C, H, W, L, 4, "fp32", 0, 0) < 0


def test_flop_count_closed_form():
    # forward FMAs per pixel at k=5, L=3 on a 64x64 plane: 25 + 100 (1/4 + 1/16 + 1/64)
    B, C, H, W, L, k = 1, 1, 64, 64, 3, 5
    N = H * W
    f = binding.wtconv_flops(B, C, H, W, L, k, "fp32", 0)
    fma = 25 + 100 * (1 / 4 + 1 / 16 + 1 / 64)
    adds = 2 + 16 * (1 / 4 + 1 / 16 + 1 / 64)
    assert abs(f - N * (2 * fma + adds)) < 1e-6 * f


def test_unfused_workspace_and_limits():
    lib = binding.load_library()
    B, C, H, W, L, k = 2, 3, 16, 10, 3, 5
    # forward: S_i, Y_i (4 bands each) and Z_i (the finer grid) per level, float32, 256-byte aligned
    sizes = [(16, 10), (8, 5), (4, 3), (2, 2)]
    want = 0
    for i in range(1, L + 1):
        n4 = B * C * 4 * sizes[i][0] * sizes[i][1] * 4
        nz = B * C * sizes[i - 1][0] * sizes[i - 1][1] * 4
        want += 2 * (-(-n4 // 256) * 256) + (-(-nz // 256) * 256)
    assert binding.wtconv_forward_unfused_workspace(B, C, H, W, L, k) == want
    assert binding.wtconv_forward_unfused_workspace(B, C, H, W, 0, k) == 0
    assert binding.wtconv_backward_unfused_workspace(B, C, H, W, L, k) > want
    # any plane size is accepted (no LDS limit) ...
    assert binding.wtconv_forward_unfused_workspace(1, 1, 512, 512, 2, 5) > 0
    # ... but not more than 30 levels, k > 31, or tensors beyond 32-bit indexing
    d = _desc(L=31)
    assert lib.wtconv_forward_unfused(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      1 << 40, None) == binding.WTC_ESHAPE
    d = _desc(k=33)
    assert lib.wtconv_forward_unfused(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      1 << 40, None) == binding.WTC_ESHAPE
    d = _desc(B=4096, C=1024, H=32, W=32)
    assert lib.wtconv_forward_unfused(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      1 << 40, None) == binding.WTC_ESHAPE
    d = _desc()
    need = lib.wtconv_forward_unfused_workspace(ctypes.byref(d))
    assert lib.wtconv_forward_unfused(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      need - 1, None) == binding.WTC_EWORKSPACE


def test_io_model_unfused_counts_intermediates():
    # forward at L = 1 on a 64x64 fp32 plane, per plane (N = 4096 pixels, bands 4 x 1024):
    # analysis reads N, writes N; conv reads N, writes N; synthesis reads N, writes N;
    # base reads x and Z_1, writes out: 9 N floats
    B, C, H, W, k = 1, 1, 64, 64, 5
    N = H * W
    params = 4 * (C * k * k * (1 + 4) + C * (2 + 4))
    f1 = binding.wtconv_io_model_bytes(B, C, H, W, 1, k, "fp32", 1, 0)
    assert abs(f1 - (9 * N * 4 + params)) < 1e-6 * f1
    # each level adds traffic, and the unfused path always moves more than the fused one
    prev = f1
    for L in range(2, 6):
        f = binding.wtconv_io_model_bytes(B, C, H, W, L, k, "fp32", 1, 0)
        assert f > prev
        prev = f
    for L in range(0, 6):
        for dr in (0, 1):
            fu = binding.wtconv_io_model_bytes(32, 96, 64, 64, L, k, "fp32", 1, dr)
            fz = binding.wtconv_io_model_bytes(32, 96, 64, 64, L, k, "fp32", 0, dr)
            assert fu >= fz * (0.99 if L == 0 else 1.5), (L, dr)


def test_large_planes_take_the_peeled_path():
    """Planes beyond the on-chip pipeline run their LL band recursively and
    level 1 with the base conv fused over tiles: a workspace for the LL band,
    the deeper result and (backward) the per-tile records there; none
    (forward) or only the partial records (backward) where the fused kernels
    fit."""
    assert binding.wtconv_forward_workspace(32, 96, 64, 64, 3, 5) == 0
    small_b = binding.wtconv_backward_workspace(32, 96, 64, 64, 3, 5)
    assert 0 < small_b < 4 * 32 * 96 * 64 * 64
    for H, W, L in [(200, 150, 3), (300, 260, 4), (512, 512, 5), (260, 130, 0), (140, 140, 1)]:
        f = binding.wtconv_forward_workspace(2, 3, H, W, L, 5)
        b = binding.wtconv_backward_workspace(2, 3, H, W, L, 5)
        h1, w1 = (H + 1) // 2, (W + 1) // 2
        if L == 0:
            assert f == 0 and b > 0
        elif L == 1:
            # the tile kernels need no forward workspace; the backward holds
            # the per-tile correlation records only
            assert f == 0 and 0 < b < 2 * 3 * H * W * 4, (H, W, L, f, b)
        else:
            # at least the LL band and the deeper result, in float32
            assert f >= 2 * 2 * 3 * h1 * w1 * 4 and b > f, (H, W, L, f, b)
    # the analytic traffic of the peeled forward exceeds the fused one's 2 N e
    n = 2 * 3 * 200 * 150 * 4
    assert binding.wtconv_io_model_bytes(2, 3, 200, 150, 3, 5, impl=0, direction=0) > 2 * n
    assert binding.wtconv_io_model_bytes(2, 3, 200, 150, 3, 5, impl=0, direction=0) < \
        binding.wtconv_io_model_bytes(2, 3, 200, 150, 3, 5, impl=1, direction=0)
    # limits that no path lifts
    assert binding.wtconv_forward_workspace(2, 3, 64, 64, 2, 33) == 0


def test_channels_last_workspace_and_model():
    """Channels-last tensors: layout 1 goes through NCHW copies at the front of
    the workspace (forward two tensors, backward three; four / six extra
    tensor passes of traffic); layout 2 reads and writes them in place for
    planes the on-chip pipeline holds (the NCHW workspace -- none forward, the
    partial records backward -- and the NCHW traffic), and is adapted like
    layout 1 beyond them.  The level-by-level baseline always adapts."""
    B, C, H, W, L, k = 4, 6, 64, 64, 3, 5
    t = B * C * H * W * 4
    for Hx, Wx in ((H, W), (200, 200)):
        tx = B * C * Hx * Wx * 4
        assert binding.wtconv_forward_workspace(B, C, Hx, Wx, L, k, layout=1) == \
            2 * tx + binding.wtconv_forward_workspace(B, C, Hx, Wx, L, k)
        assert binding.wtconv_backward_workspace(B, C, Hx, Wx, L, k, layout=1) == \
            3 * tx + binding.wtconv_backward_workspace(B, C, Hx, Wx, L, k)
        for direction, extra in ((0, 4), (1, 6)):
            assert binding.wtconv_io_model_bytes(B, C, Hx, Wx, L, k, impl=0, direction=direction, layout=1) == \
                binding.wtconv_io_model_bytes(B, C, Hx, Wx, L, k, impl=0, direction=direction) + extra * tx
    # in place
    assert binding.wtconv_forward_workspace(B, C, H, W, L, k, layout=2) == 0
    nb = binding.wtconv_backward_workspace(B, C, H, W, L, k, layout=2)
    assert 0 < nb < t
    for direction in (0, 1):
        assert binding.wtconv_io_model_bytes(B, C, H, W, L, k, impl=0, direction=direction, layout=2) <= \
            binding.wtconv_io_model_bytes(B, C, H, W, L, k, impl=0, direction=direction) * 1.01
    tb = B * C * 200 * 200 * 4   # beyond the pipeline: adapted
    assert binding.wtconv_forward_workspace(B, C, 200, 200, L, k, layout=2) == \
        2 * tb + binding.wtconv_forward_workspace(B, C, 200, 200, L, k)
    # the baseline adapts every layout
    for lay in (1, 2):
        assert binding.wtconv_backward_unfused_workspace(B, C, H, W, L, k, "bf16", layout=lay) == \
            3 * (t // 2) + binding.wtconv_backward_unfused_workspace(B, C, H, W, L, k, "bf16")
    assert binding.wtconv_forward_workspace(B, C, H, W, L, k, layout=3) == 0


def test_base_correlation_limits_checked_before_any_hip_call():
    lib = binding.load_library()
    bf = dict(dtype=binding.WTC_BF16, L=0, H=32, W=32)
    for impl in (binding.CORR_VALU, binding.CORR_MFMA):
        d = _desc(**bf)
        need = lib.wtconv_base_correlation_workspace(ctypes.byref(d), impl)
        assert need >= 4 * d.C * (d.k * d.k + 1)
        assert lib.wtconv_base_correlation(ctypes.byref(d), FAKE, FAKE, FAKE, impl, FAKE, need - 1,
                                           None) == binding.WTC_EWORKSPACE
        assert lib.wtconv_base_correlation(ctypes.byref(d), FAKE, None, FAKE, impl, FAKE, need,
                                           None) == binding.WTC_EINVAL
    cases = [
        (dict(dtype=0), binding.CORR_MFMA, binding.WTC_EDTYPE),        # matrix cores: bf16 only
        (dict(k=9), binding.CORR_MFMA, binding.WTC_ESHAPE),            # k <= 7
        (dict(H=65), binding.CORR_MFMA, binding.WTC_ESHAPE),           # planes up to 64 x 64
        (dict(layout=1), binding.CORR_VALU, binding.WTC_EDTYPE),       # NCHW only
        (dict(k=33), binding.CORR_VALU, binding.WTC_ESHAPE),
        (dict(), 2, binding.WTC_EINVAL),
    ]
    for kw, impl, status in cases:
        a = dict(bf)
        a.update(kw)
        d = _desc(**a)
        assert lib.wtconv_base_correlation_workspace(ctypes.byref(d), impl) == 0
        assert lib.wtconv_base_correlation(ctypes.byref(d), FAKE, FAKE, FAKE, impl, FAKE, 1 << 30,
                                           None) == status, (kw, impl)
