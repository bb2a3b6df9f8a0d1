"""The base level's weight-gradient correlation on its own -- on the vector
units (impl CORR_VALU) and on the gfx950 matrix cores (impl CORR_MFMA) --
against the float64 oracle's correlation, through the C ABI.

bf16 products are exact in the fp32 accumulators of both paths, so the two
differ from the oracle only by fp32 summation rounding: they are held to the
fp32 bar (max|err| <= 1e-4 * RMS), not the looser bf16 one."""

import numpy as np
import pytest
import torch

import oracle
from memory_bound_cnn_amd import binding
from memory_bound_cnn_amd.inputs import WORKLOADS, workload_inputs
from tests.gpu_helpers import TOL, host, inputs, rel_err, to_dev

pytestmark = pytest.mark.gpu

VALU, MFMA = binding.CORR_VALU, binding.CORR_MFMA

# (B, C, H, W, k, seed): a tile-sized plane, ragged widths (one and two
# 32-pixel segments), the largest plane (64 x 64), a plane smaller than the
# window, a single pixel, more channels than compute units, and batch chunks
# of 10 planes (a partial last round of the four waves)
SHAPES = [
    (3, 5, 32, 32, 5, 1),
    (2, 3, 17, 45, 7, 2),
    (2, 4, 31, 13, 3, 3),
    (4, 2, 64, 64, 3, 4),
    (9, 4, 5, 6, 7, 5),
    (1, 1, 1, 1, 1, 6),
    (2, 300, 8, 8, 5, 7),
    (40, 256, 8, 8, 3, 8),
]


def _run(d, dtype, k, impl):
    t = to_dev(d, dtype, L=0)
    got = binding.wtconv_base_correlation(t["x"], t["g"], k, impl)
    torch.cuda.synchronize()
    return host(got)


@pytest.mark.parametrize("impl", [VALU, MFMA], ids=["valu", "mfma"])
@pytest.mark.parametrize("B,C,H,W,k,seed", SHAPES)
def test_base_correlation_bf16(B, C, H, W, k, seed, impl):
    print(f"base correlation bf16 impl={impl} B={B} C={C} {H}x{W} k={k}", flush=True)
    d = inputs(B, C, H, W, 0, k, seed, "bf16")
    ref = oracle.corr(d["g"], d["x"], k)
    err = rel_err(_run(d, "bf16", k, impl), ref)
    assert err <= TOL["fp32"], err


@pytest.mark.parametrize("B,C,H,W,k,seed", [(3, 5, 32, 32, 5, 11), (2, 3, 17, 45, 7, 12), (2, 3, 20, 21, 9, 13),
                                             (1, 2, 3, 40, 1, 14)])
def test_base_correlation_fp32_valu(B, C, H, W, k, seed):
    print(f"base correlation fp32 B={B} C={C} {H}x{W} k={k}", flush=True)
    d = inputs(B, C, H, W, 0, k, seed, "fp32")
    ref = oracle.corr(d["g"], d["x"], k)
    assert rel_err(_run(d, "fp32", k, VALU), ref) <= TOL["fp32"]


def test_base_correlation_full_size_bf16():
    """The bf16 workload at its full size (64 x 192 planes of 32 x 32,
    k = 5): 65,536 terms per tap and channel, both paths against the oracle."""
    w = WORKLOADS["bf16_b64c192_32x32_L3"]
    print(f"base correlation full size {w.name}", flush=True)
    d = workload_inputs(w)
    ref = oracle.corr(d["g"], d["x"], w.k)
    t = to_dev({"x": d["x"], "g": d["g"]}, "bf16")
    for impl in (VALU, MFMA):
        got = binding.wtconv_base_correlation(t["x"], t["g"], w.k, impl)
        torch.cuda.synchronize()
        err = rel_err(host(got), ref)
        assert err <= TOL["fp32"], (impl, err)


def test_base_correlation_deterministic():
    d = inputs(8, 16, 32, 32, 0, 5, 21, "bf16")
    t = to_dev(d, "bf16", L=0)
    for impl in (VALU, MFMA):
        a = binding.wtconv_base_correlation(t["x"], t["g"], 5, impl)
        b = binding.wtconv_base_correlation(t["x"], t["g"], 5, impl)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
