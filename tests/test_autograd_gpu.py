"""The PyTorch autograd wrapper on the GPU: gradients of a training-style step
(loss = <out, g>) through WTConvFunction, for the fused kernels and for the
level-by-level baseline, against the float64 oracle."""

import pytest
import torch

from memory_bound_cnn_amd.autograd import WTConv2d, wtconv
from tests.gpu_helpers import check_all, inputs, oracle_ref, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("impl", ["fused", "unfused"])
@pytest.mark.parametrize("B,C,H,W,L,dtype", [(2, 4, 32, 32, 2, "fp32"), (3, 5, 14, 14, 2, "fp32"),
                                             (2, 4, 32, 32, 3, "bf16")])
def test_autograd_matches_oracle(impl, B, C, H, W, L, dtype):
    d = inputs(B, C, H, W, L, 5, 90 + L, dtype)
    t = to_dev(d, dtype, L)
    x = t["x"].clone().requires_grad_(True)
    params = {k: t[k].clone().requires_grad_(True) for k in ("w0", "s0", "b0", "wl", "sl")}
    out = wtconv(x, params["w0"], params["s0"], params["b0"], params["wl"], params["sl"], L, impl=impl)
    out.backward(t["g"])
    gr = {"dx": x.grad, "dw0": params["w0"].grad, "ds0": params["s0"].grad, "db0": params["b0"].grad,
          "dwl": params["wl"].grad, "dsl": params["sl"].grad}
    ref_out, ref_gr = oracle_ref(d, L)
    check_all(out.detach(), gr, ref_out, ref_gr, dtype, f"autograd {impl} {B}x{C}x{H}x{W} L{L} {dtype}")


def test_module_step_updates_all_parameters():
    torch.manual_seed(0)
    m = WTConv2d(6, kernel_size=5, levels=2, device="cuda")
    x = torch.randn(2, 6, 16, 16, device="cuda", requires_grad=True)
    y = m(x)
    assert y.shape == x.shape
    (y * y).sum().backward()
    for name, p in m.named_parameters():
        assert p.grad is not None and torch.isfinite(p.grad).all(), name
        assert p.grad.abs().sum() > 0, name
    assert x.grad is not None and torch.isfinite(x.grad).all()


def test_bad_impl_rejected():
    x = torch.zeros(1, 1, 8, 8, device="cuda")
    w = torch.zeros(1, 5, 5, device="cuda")
    s = torch.ones(1, device="cuda")
    with pytest.raises(ValueError):
        wtconv(x, w, s, s, None, None, 0, impl="other")


def test_channels_last_stays_channels_last():
    """A channels-last input goes through the wrapper without an NCHW copy:
    out and dx keep its layout, and the gradients match the NCHW call."""
    d = inputs(2, 6, 32, 32, 2, 5, 95)
    t = to_dev(d, "fp32", 2)
    res = {}
    for fmt in (torch.contiguous_format, torch.channels_last):
        x = t["x"].detach().clone(memory_format=fmt).requires_grad_(True)
        p = {k: t[k].clone().requires_grad_(True) for k in ("w0", "s0", "b0", "wl", "sl")}
        out = wtconv(x, p["w0"], p["s0"], p["b0"], p["wl"], p["sl"], 2)
        out.backward(t["g"])
        res[fmt] = (out.detach(), x.grad, {k: v.grad for k, v in p.items()})
    out_cl, dx_cl, gp_cl = res[torch.channels_last]
    assert out_cl.is_contiguous(memory_format=torch.channels_last) and not out_cl.is_contiguous()
    assert dx_cl.is_contiguous(memory_format=torch.channels_last)
    out_n, dx_n, gp_n = res[torch.contiguous_format]
    assert torch.equal(out_cl.contiguous(), out_n) and torch.equal(dx_cl.contiguous(), dx_n)
    for k in gp_n:
        assert torch.equal(gp_cl[k], gp_n[k]), k


def test_parameters_with_more_levels_than_used():
    """wl / sl with more rows than L (a module built for more levels): the
    gradients have the parameters' shapes, zero beyond level L."""
    d = inputs(2, 4, 16, 16, 3, 5, 96)
    t = to_dev(d, "fp32", 3)
    p = {k: t[k].clone().requires_grad_(True) for k in ("w0", "s0", "b0", "wl", "sl")}
    out = wtconv(t["x"], p["w0"], p["s0"], p["b0"], p["wl"], p["sl"], 2)
    out.backward(t["g"])
    assert p["wl"].grad.shape == p["wl"].shape and p["sl"].grad.shape == p["sl"].shape
    assert torch.count_nonzero(p["wl"].grad[2]) == 0 and torch.count_nonzero(p["sl"].grad[2]) == 0
    ref = wtconv(t["x"], t["w0"], t["s0"], t["b0"], t["wl"][:2].contiguous(), t["sl"][:2].contiguous(), 2)
    assert torch.equal(out.detach(), ref)
    _, ref_gr = oracle_ref(d, 2)
    from tests.gpu_helpers import host, rel_err
    assert rel_err(host(p["wl"].grad[:2]), ref_gr["dwl"]) <= 1e-4
    assert rel_err(host(p["sl"].grad[:2]), ref_gr["dsl"]) <= 1e-4
