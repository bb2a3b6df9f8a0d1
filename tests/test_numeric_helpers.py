"""The numeric helpers every kernel shares (memory_bound_cnn_amd/csrc/wtc_numeric.h),
compiled on the host from the very header the kernels include:

* bf16_rne, float32 -> bfloat16 round to nearest even, against an
  independent reference (the nearest of the two neighbouring bfloat16 values,
  compared in float64, ties to the even one) on edge cases and random bit
  patterns; NaN must stay NaN, infinities and overflow give infinity;
* FastDiv, integer division through a biased float reciprocal, exhaustively
  over the range the kernels use it in (e < 2^16 with d <= 32768, e < d with
  d < 2^16), with the reciprocal also one ulp off either way."""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bound_cnn_amd", "csrc")

PROGRAM = r"""
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>
#include "wtc_numeric.h"

static long check_div(int d0, int d1) {
    long bad = 0;
    for (int d = d0; d < d1; ++d) {
        const wtc::FastDiv f = wtc::make_div(d);
        const float rs[3] = {f.r, std::nextafter(f.r, 0.f), std::nextafter(f.r, 2.f)};
        const int emax = d <= 32768 ? 65536 : d;
        for (int v = 0; v < 3; ++v) {
            wtc::FastDiv g = f;
            g.r = rs[v];
            for (int e = 0; e < emax; ++e) bad += wtc::fdiv(e, g) != e / d;
        }
    }
    return bad;
}

int main(int argc, char** argv) {
    if (argc > 1 && !strcmp(argv[1], "div")) {
        const int nt = 8;
        std::vector<long> bad(nt, 0);
        std::vector<std::thread> th;
        for (int t = 0; t < nt; ++t)   // interleaved blocks of divisors: even load
            th.emplace_back([t, &bad] { for (int d0 = 1 + 256 * t; d0 < 65536; d0 += 256 * 8)
                                           bad[t] += check_div(d0, d0 + 256 < 65536 ? d0 + 256 : 65536); });
        for (auto& x : th) x.join();
        long tot = 0;
        for (long b : bad) tot += b;
        printf("%ld\n", tot);
        return 0;
    }
    // bf16: one float32 bit pattern per line on stdin -> the bfloat16 bits
    unsigned int u;
    while (scanf("%x", &u) == 1) {
        float v;
        memcpy(&v, &u, 4);
        printf("%04x\n", (unsigned)wtc::bf16_rne(v));
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("numeric")
    src, exe = d / "t.cpp", d / "t"
    src.write_text(PROGRAM)
    subprocess.run([cxx, "-O2", "-std=c++17", "-pthread", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    return str(exe)


def _ref_bf16(bits):
    """Independent float32 -> bfloat16 (round to nearest, ties to even)."""
    out = []
    for u in bits:
        u = int(u)
        v = np.array([u], dtype=np.uint32).view(np.float32)[0]
        if np.isnan(v):
            out.append(None)
            continue
        if np.isinf(v):
            out.append(u >> 16)
            continue
        lo = u >> 16                       # truncation: the neighbour towards zero
        hi = lo + 1                        # the next one away from zero
        # a neighbour with the all-ones exponent is the overflow case: IEEE rounding
        # compares with the value it would have with an unbounded exponent, 2^128
        f = lambda b: float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0]) if (b & 0x7F80) != 0x7F80 \
            else 2.0 ** 128 * (1 if b < 0x8000 else -1)
        x, a, b = float(v), f(lo), f(hi)
        da, db = abs(x - a), abs(b - x)
        if da < db or (da == db and lo % 2 == 0):
            out.append(lo)
        else:
            out.append(hi)
    return out


def test_bf16_rounding(prog):
    rng = np.random.default_rng(0)
    edge = [0x00000000, 0x80000000, 0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF,
            0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F800000, 0xFF800000, 0x00000001, 0x00008000,
            0x00018000, 0x007FFFFF, 0x7F800001, 0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFF800001, 0x7F80FFFF,
            0x7FBF0000]
    bits = np.concatenate([np.array(edge, dtype=np.uint64), rng.integers(0, 2 ** 32, 200000, dtype=np.uint64)])
    r = subprocess.run([prog], input="\n".join(f"{int(b):08x}" for b in bits), capture_output=True, text=True,
                       check=True)
    got = [int(t, 16) for t in r.stdout.split()]
    ref = _ref_bf16(bits)
    assert len(got) == len(ref)
    for b, g, want in zip(bits, got, ref):
        if want is None:   # NaN in, NaN out (exponent all ones, mantissa non-zero), sign kept
            assert (g & 0x7F80) == 0x7F80 and (g & 0x007F) != 0 and (g >> 15) == (int(b) >> 31), hex(int(b))
        else:
            assert g == want, (hex(int(b)), hex(g), hex(want))


def test_fastdiv_exhaustive(prog):
    r = subprocess.run([prog, "div"], capture_output=True, text=True, check=True, timeout=600)
    assert int(r.stdout.strip()) == 0
