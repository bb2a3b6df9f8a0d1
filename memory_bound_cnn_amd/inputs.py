"""Seeded synthetic inputs for WTConv, shared by the tests and the benchmark.

This module holds no arithmetic of the method: it only draws random tensors
and, for the bf16-storage workload, rounds them to bfloat16 values.  Both the
HIP library and the CPU oracle consume exactly the arrays returned here.

Draw order (NumPy PCG64, one generator per workload seed):
  1. x ~ N(0, 1)            [B, C, H, W]   (drawn as float32)
  2. g ~ N(0, 1)            [B, C, H, W]   (upstream gradient, float32)
  3. W0 = N(0, 1) / k       [C, k, k]      (variance 1/k^2)
  4. b0 = 0.1 * N(0, 1)     [C]            (variance 0.01)
  5. s0 ~ U[0.05, 0.5]      [C]
  6. for i = 1..L_max:  W_i = N(0, 1) / k [4C, k, k],  then  s_i ~ U[0.05, 0.5] [4C]
Parameters are drawn in float64 and rounded to float32.  For bf16 storage, x
and g are rounded to the nearest bfloat16 (ties to even) and kept as float32
values that are exactly representable in bfloat16.
"""

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_round", "bf16_bits", "bf16_bits_to_f32"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    H: int
    W: int
    L: int
    k: int
    dtype: str  # "fp32" or "bf16": storage type of x / out / g / dx
    seed: int
    L_max: int = 0  # levels drawn (>= L); 0 means L
    sweep: tuple = field(default_factory=tuple)  # extra L values run on one draw

    @property
    def levels_drawn(self):
        return max(self.L, self.L_max, *(self.sweep or (0,)))

    def at_level(self, L):
        return Workload(self.name, self.B, self.C, self.H, self.W, L, self.k, self.dtype,
                        self.seed, self.levels_drawn, ())


# The benchmark workloads: WTConvNeXt-like block shapes at several levels.
WORKLOADS = {
    # small parity / finite-difference case
    "tiny_b1c8_32x32_L2": Workload("tiny_b1c8_32x32_L2", 1, 8, 32, 32, 2, 5, "fp32", 0),
    # stage-1-like WTConvNeXt block: the headline workload
    "stage1_b32c96_64x64_L3": Workload("stage1_b32c96_64x64_L3", 32, 96, 64, 64, 3, 5, "fp32", 10),
    # bf16 storage, fp32 weights and accumulation
    "bf16_b64c192_32x32_L3": Workload("bf16_b64c192_32x32_L3", 64, 192, 32, 32, 3, 5, "bf16", 20),
    # level sweep on one draw (L = 1..5)
    "sweep_b64c96_128x128": Workload("sweep_b64c96_128x128", 64, 96, 128, 128, 1, 5, "fp32", 30,
                                     5, (1, 2, 3, 4, 5)),
    # odd / small spatial shapes
    "odd_b128c384_14x14_L2": Workload("odd_b128c384_14x14_L2", 128, 384, 14, 14, 2, 5, "fp32", 40),
    "odd_b128c768_7x7_L1": Workload("odd_b128c768_7x7_L1", 128, 768, 7, 7, 1, 5, "fp32", 41),
    # planes beyond the on-chip pipeline (a high-resolution first stage): level 1
    # level by level, the LL band (112 x 112) fused
    "large_b8c64_224x224_L3": Workload("large_b8c64_224x224_L3", 8, 64, 224, 224, 3, 5, "fp32", 50),
}


def bf16_bits(a):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(a):
    """Round float32 values to the nearest bfloat16 value (ties to even), as float32."""
    return bf16_bits_to_f32(bf16_bits(a))


def make_inputs(B, C, H, W, L, k, seed, dtype="fp32", L_max=None):
    """Draw one seeded input set.  Returns a dict of NumPy arrays.

    Keys: x, g (float32, bf16-exact when dtype == "bf16"), w0 [C,k,k], s0 [C],
    b0 [C], wl [Lmax,4C,k,k], sl [Lmax,4C] (float32; wl/sl are None if Lmax == 0).
    """
    Lmax = L if L_max is None else max(L, L_max)
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, C, H, W), dtype=np.float32)
    g = rng.standard_normal((B, C, H, W), dtype=np.float32)
    w0 = (rng.standard_normal((C, k, k)) / k).astype(np.float32)
    b0 = (0.1 * rng.standard_normal(C)).astype(np.float32)
    s0 = rng.uniform(0.05, 0.5, C).astype(np.float32)
    wl, sl = [], []
    for _ in range(Lmax):
        wl.append((rng.standard_normal((4 * C, k, k)) / k).astype(np.float32))
        sl.append(rng.uniform(0.05, 0.5, 4 * C).astype(np.float32))
    if dtype == "bf16":
        x = bf16_round(x)
        g = bf16_round(g)
    elif dtype != "fp32":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    return dict(
        x=x, g=g, w0=w0, s0=s0, b0=b0,
        wl=np.stack(wl) if Lmax else None,
        sl=np.stack(sl) if Lmax else None,
    )


def workload_inputs(wl: Workload):
    return make_inputs(wl.B, wl.C, wl.H, wl.W, wl.L, wl.k, wl.seed, wl.dtype, wl.levels_drawn)
