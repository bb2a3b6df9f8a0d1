"""bfloat16 outputs are rounded on the device exactly as the host helper
rounds them (round to nearest, ties to even; overflow to infinity; NaN stays
NaN).  The kernels round through one shared helper, which on gfx950 is the
hardware pair conversion; this pins its results bit for bit against the
independent reference of the CPU helper test.

The operator with L = 0, k = 1, scale 1 and bias 0 is out = c * x per
channel.  With x in bfloat16 (8 significant bits) and c of at most 16
significant bits the product is exact in float32, so the float32 value the
kernel rounds is known on the host, and the c below put many of them exactly
halfway between two bfloat16 values."""

import numpy as np
import pytest
import torch

from memory_bound_cnn_amd import binding
from tests.test_numeric_helpers import _ref_bf16

pytestmark = pytest.mark.gpu

# per-channel multipliers: identity, and products whose bits past the bfloat16
# mantissa are the multiplicand's own bits (ties where x is a power of two)
C_VALUES = [1.0, 1.0 + 2.0 ** -8, 1.0 - 2.0 ** -9, 1.5 + 2.0 ** -8, 0.75 + 2.0 ** -10, 1.0 + 3.0 * 2.0 ** -9,
            1.0 + 2.0 ** -8 + 2.0 ** -15, 1.2529296875]


def _x_bits(rng, shape):
    """bfloat16 bit patterns: random finite values, powers of two, and in
    every plane values near the largest finite one (their products overflow
    the bfloat16 range), zeros, infinities and NaNs."""
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, n, dtype=np.uint32) << 15
    expo = rng.integers(100, 155, n, dtype=np.uint32) << 7
    mant = rng.integers(0, 128, n, dtype=np.uint32)
    mant[rng.random(n) < 0.3] = 0                      # powers of two: ties under c = 1 + 2^-8
    b = sign | expo | mant
    special = np.array([0x0000, 0x7F7F, 0xFF7F, 0x7F7E, 0x7F00, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80],
                       dtype=np.uint32)
    b = b.reshape(shape[0] * shape[1], -1)
    b[:, :special.size] = special
    return b.astype(np.uint16).reshape(shape)


def exp_all(want):
    return np.array([-1 if v is None else v for v in want], dtype=np.int64)


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_bf16_output_rounding_matches_host(impl):
    rng = np.random.default_rng(7)
    B, C, H, W = 2, len(C_VALUES), 32, 32
    xb = _x_bits(rng, (B, C, H, W))
    x32 = (xb.astype(np.uint32) << 16).view(np.float32)
    c = np.array(C_VALUES, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        want32 = x32 * c[None, :, None, None] + np.float32(0.0)   # exact products; -0 + 0 = +0 as on the device
    want = np.array(_ref_bf16(want32.view(np.uint32).ravel()), dtype=object)

    d = torch.device("cuda", 0)
    x = torch.from_numpy(xb.view(np.int16).copy()).to(d).view(torch.bfloat16)
    w0 = torch.from_numpy(c.reshape(C, 1, 1).copy()).to(d)
    s0 = torch.ones(C, dtype=torch.float32, device=d)
    b0 = torch.zeros(C, dtype=torch.float32, device=d)
    fwd = binding.wtconv_forward if impl == "fused" else binding.wtconv_forward_unfused
    out = fwd(x, w0, s0, b0, None, None, 0)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.int64).ravel()

    nan = np.array([v is None for v in want])
    assert nan.any() and (~nan).sum() > 0
    g_nan = got[nan]
    assert np.all((g_nan & 0x7F80) == 0x7F80) and np.all((g_nan & 0x007F) != 0), "NaN in, NaN out"
    exp = np.array([v for v in want if v is not None], dtype=np.int64)
    bad = np.nonzero(got[~nan] != exp)[0]
    assert bad.size == 0, [(hex(int(want32.view(np.uint32).ravel()[~nan][i])), hex(int(got[~nan][i])),
                            hex(int(exp[i]))) for i in bad[:8]]
    # the case was worth running: ties and overflows were among the values
    w32 = want32.view(np.uint32).ravel()
    assert np.count_nonzero((w32 & 0xFFFF) == 0x8000) > 100
    assert np.count_nonzero(np.isinf(want32.ravel())) > 0
    assert np.count_nonzero(np.isfinite(want32.ravel()) & (exp_all(want) == 0x7F80)) > 0   # rounded up to infinity
