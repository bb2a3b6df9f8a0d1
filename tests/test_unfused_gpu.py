"""Parity of the level-by-level HIP baseline (the "_unfused" entry points)
with the float64 oracle, at reduced sizes and at two full benchmark shapes.  Same tolerances as the fused path: max|err| <= 1e-4 * RMS
(float32 storage), 2e-2 * RMS (bfloat16 storage)."""

import pytest
import torch

from memory_bound_cnn_amd.inputs import WORKLOADS, workload_inputs
from tests.gpu_helpers import check_all, host, inputs, oracle_ref, rel_err, run_fused, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (1, 8, 32, 32, 2, 5, 100, "fp32"),
    (2, 6, 64, 64, 3, 5, 101, "fp32"),
    (3, 8, 32, 32, 3, 5, 102, "bf16"),
    (1, 2, 128, 128, 5, 5, 103, "fp32"),
    (5, 8, 14, 14, 2, 5, 104, "fp32"),
    (9, 8, 7, 7, 1, 5, 105, "fp32"),
    (2, 3, 16, 16, 0, 5, 106, "fp32"),     # L = 0
    (2, 3, 13, 10, 3, 3, 107, "fp32"),     # odd sides, k = 3
    (1, 2, 3, 3, 5, 3, 108, "fp32"),       # levels past the 1x1 grid
    (1, 2, 9, 17, 2, 7, 109, "fp32"),      # k = 7
    (2, 4, 24, 24, 2, 1, 110, "fp32"),     # k = 1
    (1, 1, 200, 72, 2, 5, 111, "fp32"),    # larger than the fused path's LDS plane limit in one side
    # planes with both sides >= 48 take the 64 x 64 tiled stencil kernels
    # (level 0 here, and level 1 too for the 100-wide one): every kernel size,
    # ragged tiles, bf16 storage
    (1, 2, 96, 100, 1, 7, 112, "fp32"),
    (1, 2, 70, 66, 1, 1, 113, "fp32"),
    (2, 2, 80, 72, 2, 3, 114, "bf16"),
    (1, 3, 130, 97, 2, 5, 115, "fp32"),
]


@pytest.mark.parametrize("B,C,H,W,L,k,seed,dtype", CASES)
def test_unfused_matches_oracle(B, C, H, W, L, k, seed, dtype):
    d = inputs(B, C, H, W, L, k, seed, dtype)
    t = to_dev(d, dtype, L)
    out, gr = run_fused(t, L, "unfused")
    ref_out, ref_gr = oracle_ref(d, L)
    check_all(out, gr, ref_out, ref_gr, dtype, f"unfused B{B} C{C} {H}x{W} L{L} k{k} {dtype}")


@pytest.mark.parametrize("name", ["stage1_b32c96_64x64_L3", "bf16_b64c192_32x32_L3"])
def test_unfused_full_size(name):
    """The baseline at full benchmark size against the oracle: out and dx on
    two sampled batch entries, every weight gradient over the whole batch
    (the stored float64 oracle values of tests/golden/fullsize_weight_grads.npz)."""
    import numpy as np

    from tests.test_parity_gpu import _golden, _inputs_sha256
    wl_ = WORKLOADS[name]
    L = wl_.L
    d = workload_inputs(wl_)
    ref_w, sha = _golden(f"{name}_L{L}")
    assert _inputs_sha256(d, L) == sha
    t = to_dev(d, wl_.dtype, L)
    out, gr = run_fused(t, L, "unfused")
    batch = np.array([3, wl_.B - 1])
    dd = dict(d)
    dd["x"], dd["g"] = d["x"][batch], d["g"][batch]
    ref_out, ref_gr = oracle_ref(dd, L)
    tol = 1e-4 if wl_.dtype == "fp32" else 2e-2
    errs = {"out": rel_err(host(out)[batch], ref_out), "dx": rel_err(host(gr["dx"])[batch], ref_gr["dx"])}
    for key, ref in ref_w.items():
        errs[key] = rel_err(host(gr[key]), ref)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"unfused {name}: {bad} (all {errs})"
    torch.cuda.synchronize()
