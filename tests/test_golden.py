"""The stored full-size oracle weight gradients (tests/golden/fullsize_weight_grads.npz)
against the oracle itself: every parity case is present, and one case -- the
32 x 96 x 64 x 64, L = 3 block -- is recomputed here from the seeded inputs and
must match to float64 rounding, so a stale or hand-edited file fails."""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))

import make_fullsize_grads as mk  # noqa: E402
import oracle  # noqa: E402
from memory_bound_cnn_amd.inputs import WORKLOADS, workload_inputs  # noqa: E402


def _load():
    return np.load(mk.OUT)


def test_every_case_present():
    z = _load()
    for case, w, L in mk.cases():
        for key in ("dw0", "ds0", "db0") + (("dwl", "dsl") if L > 0 else ()):
            a = z[f"{case}|{key}"]
            assert a.dtype == np.float64 and np.all(np.isfinite(a)), (case, key)
        assert z[f"{case}|dw0"].shape == (w.C, w.k, w.k)
        if L > 0:
            assert z[f"{case}|dwl"].shape == (L, 4 * w.C, w.k, w.k)
            assert z[f"{case}|dsl"].shape == (L, 4 * w.C)
        assert len(str(z[f"{case}|inputs_sha256"])) == 64


def test_stage1_case_recomputed():
    w = WORKLOADS["stage1_b32c96_64x64_L3"]
    d = workload_inputs(w)
    case = f"{w.name}_L{w.L}"
    z = _load()
    sub = dict(d)
    assert mk.inputs_sha256(sub) == str(z[f"{case}|inputs_sha256"])
    gr = oracle.backward(d["x"], d["g"], d["w0"], d["s0"], d["b0"], d["wl"], d["sl"], w.L, batch_chunk=8)
    for key in ("dw0", "ds0", "db0", "dwl", "dsl"):
        ref = z[f"{case}|{key}"]
        scale = np.sqrt(np.mean(ref ** 2))
        assert np.max(np.abs(gr[key] - ref)) <= 1e-12 * scale, key
