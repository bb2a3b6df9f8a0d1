"""wtconv_backward_noalloc (the backward pass with no workspace and no
allocation, its scratch a fixed per-GPU device array) against
wtconv_backward, through the C ABI: two calls in a row, the second with a
smaller input, each bit-identical to the workspace entry point on the same
inputs (same kernels, deterministic reduction order); a call that needs more
scratch than the array holds is refused before any launch."""

import pytest
import torch

from memory_bound_cnn_amd import binding
from tests.gpu_helpers import host, inputs, oracle_ref, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _buffers(t, L):
    x = t["x"]
    C, k = x.shape[1], t["w0"].shape[-1]
    f32 = dict(dtype=torch.float32, device=x.device)
    grads = dict(dw0=torch.empty(C, k, k, **f32), ds0=torch.empty(C, **f32), db0=torch.empty(C, **f32),
                 dwl=torch.empty(L, 4 * C, k, k, **f32) if L else None,
                 dsl=torch.empty(L, 4 * C, **f32) if L else None)
    return torch.empty_like(x), grads


CALLS = [
    (4, 24, 64, 64, 3, 5, 300, "fp32"),    # 64x64 planes, direct-load backward
    (3, 10, 32, 32, 2, 5, 301, "bf16"),    # smaller, bf16 storage
    (2, 5, 14, 14, 2, 5, 302, "fp32"),     # smaller again, several planes per workgroup
]


def test_noalloc_matches_workspace_entry_point():
    for B, C, H, W, L, k, seed, dtype in CALLS:
        d = inputs(B, C, H, W, L, k, seed, dtype)
        t = to_dev(d, dtype, L)
        dx, grads = _buffers(t, L)
        binding.wtconv_backward_noalloc(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L, dx=dx, grads=grads)
        ref = binding.wtconv_backward(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L)
        torch.cuda.synchronize()
        assert torch.equal(dx, ref["dx"]), (B, C, H, W, L)
        for key, v in grads.items():
            if v is not None:
                assert torch.equal(v, ref[key]), (key, B, C, H, W, L)
        # and within the oracle tolerance on its own
        _, ref_gr = oracle_ref(d, L)
        gr = dict(grads)
        gr["dx"] = dx
        tol = 1e-4 if dtype == "fp32" else 2e-2
        for key in ("dx", "dw0", "ds0", "db0", "dwl", "dsl"):
            if ref_gr.get(key) is not None:
                assert rel_err(host(gr[key]), ref_gr[key]) <= tol, key


def test_noalloc_refuses_more_than_its_scratch():
    # planes beyond the on-chip pipeline need far more than the fixed array
    B, C, H, W, L, k = 8, 64, 224, 224, 3, 5
    assert binding.wtconv_backward_workspace(B, C, H, W, L, k) > binding.NOALLOC_SCRATCH_BYTES
    d = inputs(B, C, H, W, L, k, 303)
    t = to_dev(d, "fp32", L)
    with pytest.raises(binding.WTCError) as e:
        binding.wtconv_backward_noalloc(t["x"], t["g"], t["w0"], t["s0"], t["wl"], t["sl"], L)
    assert e.value.status == binding.WTC_ESCRATCH
