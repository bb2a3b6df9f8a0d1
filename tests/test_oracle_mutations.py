"""The oracle's pins are sensitive: plant plausible mistakes in a copy of the
oracle (on the CPU, in a temporary directory) and check that the pins in
``test_oracle`` reject every one of them."""

import importlib.util
import os
import shutil

import pytest

import tests.test_oracle as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                          "wtconv_oracle.py")

# (description, original text, mutated text)
MUTATIONS = [
    ("wrong sign in one analysis band", "hx = 0.5 * (a - b + c - d)", "hx = 0.5 * (a - b - c + d)"),
    ("wrong sign in one synthesis phase", "out[..., 0::2, 1::2] = 0.5 * (t0 - t1 + t2 - t3)",
     "out[..., 0::2, 1::2] = 0.5 * (t0 + t1 + t2 - t3)"),
    ("missing normalisation", "ll = 0.5 * (a + b + c + d)", "ll = (a + b + c + d)"),
    ("no 180-degree rotation in dX", "dwconv(g, _rot180(w0))", "dwconv(g, w0)"),
    ("deeper level added to the wrong band", "T[:, :, 0] += Z", "T[:, :, 1] += Z"),
    ("scale gradient scaled twice", 'dsl[i - 1] = np.einsum("bchw,bchw->c", dYf, V)',
     'dsl[i - 1] = sl[i - 1] * np.einsum("bchw,bchw->c", dYf, V)'),
    ("transposed kernel", "Xp[:, :, ky:ky + h, kx:kx + w]\n    return out",
     "Xp[:, :, kx:kx + h, ky:ky + w]\n    return out"),
    ("dropped bias", "out = out + b0[None, :, None, None]", "out = out"),
    ("convolved LL fed to the next level", "LL = bands[:, :, 0]", "LL = bands[:, :, 0] * 0.999"),
    ("dropped base convolution in dX", "dx = dx + dLL", "dx = dLL"),
]

# Pins run against each mutant (fast ones; each mutation must fail at least one).
PIN_CALLS = [
    ("test_golden_haar_2x2", {}),
    ("test_golden_operator_2x2", {}),
    ("test_haar_perfect_reconstruction", dict(h=7, w=5)),
    ("test_haar_parseval", dict(h=7, w=5)),
    ("test_L0_equals_depthwise_conv", dict(k=3)),
    ("test_L0_backward_equals_autograd", {}),
    ("test_delta_kernels_unit_scales", dict(H=7, W=5, L=3)),
    ("test_cascade_equals_closed_form", dict(H=7, W=5, L=3, k=5)),
    ("test_adjoint_dot", dict(H=7, W=5, L=3)),
    ("test_finite_differences_exact", dict(H=7, W=5, L=2, k=3)),
    ("test_scale_gradient_identity", {}),
]


def _load_mutant(tmp_path, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    d = tmp_path / "mut"
    d.mkdir()
    shutil.copy(ORACLE_SRC, d / "wtconv_oracle.py")
    (d / "wtconv_oracle.py").write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mutant_oracle", d / "wtconv_oracle.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_mutant(tmp_path, monkeypatch, desc, old, new):
    mutant = _load_mutant(tmp_path, old, new)
    monkeypatch.setattr(pins, "oracle", mutant)
    caught = []
    for name, kwargs in PIN_CALLS:
        try:
            getattr(pins, name)(**kwargs)
        except AssertionError:
            caught.append(name)
    assert caught, f"no pin rejected the mutant: {desc}"


def test_unmutated_oracle_passes_all_listed_pins():
    for name, kwargs in PIN_CALLS:
        getattr(pins, name)(**kwargs)
