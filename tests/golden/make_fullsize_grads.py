"""Write the float64 oracle's weight gradients at the full benchmark shapes.

    python tests/golden/make_fullsize_grads.py [--procs N]

Output: tests/golden/fullsize_weight_grads.npz.  For every full-size workload
(and every level of the level sweep) it holds the oracle's dw0 [C,k,k],
ds0 [C], db0 [C], dwl [L,4C,k,k] and dsl [L,4C], summed over the WHOLE batch
(no masking of the upstream gradient), plus a SHA-256 of the seeded inputs
they were computed from.  The GPU parity test compares the library's
full-length reductions (up to B*H*W = 1,048,576 terms per channel) with
these values and refuses to run if its own inputs hash differently.

Only the oracle (oracle/) and the seeded input generator
(memory_bound_cnn_amd/inputs.py, which holds no arithmetic of the method)
are used here; nothing from the HIP library.  The oracle's backward is linear
in the batch, so per-chunk results are summed in float64 in a fixed order.
"""

import argparse
import dataclasses
import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from memory_bound_cnn_amd.inputs import WORKLOADS, workload_inputs  # noqa: E402

OUT = os.path.join(HERE, "fullsize_weight_grads.npz")
GRAD_KEYS = ("dw0", "ds0", "db0", "dwl", "dsl")


def cases():
    """(case name, workload, L) for every full-size parity case."""
    out = []
    for name in ("stage1_b32c96_64x64_L3", "bf16_b64c192_32x32_L3", "odd_b128c384_14x14_L2",
                 "odd_b128c768_7x7_L1", "large_b8c64_224x224_L3"):
        w = WORKLOADS[name]
        out.append((f"{name}_L{w.L}", w, w.L))
    sw = WORKLOADS["sweep_b64c96_128x128"]
    for L in sw.sweep:
        out.append((f"{sw.name}_L{L}", sw, L))
    # the plain depthwise convolutions WTConv is compared with (L = 0, k = 5 and 7)
    st = WORKLOADS["stage1_b32c96_64x64_L3"]
    for k in (5, 7):
        w = dataclasses.replace(st, name=f"stage1_L0_k{k}", L=0, k=k, L_max=0, sweep=())
        out.append((f"{w.name}_L0", w, 0))
    return out


def inputs_sha256(d):
    """Hash of the arrays a full-size case consumes (x, g and every parameter)."""
    h = hashlib.sha256()
    for key in ("x", "g", "w0", "s0", "b0", "wl", "sl"):
        v = d[key]
        h.update(key.encode())
        if v is not None:
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


_D = {}   # workload name -> inputs (shared with forked workers)


def _task(args):
    name, L, b0, b1 = args
    d = _D[name]
    wl = d["wl"][:L] if L > 0 else None
    sl = d["sl"][:L] if L > 0 else None
    gr = oracle.backward(d["x"][b0:b1], d["g"][b0:b1], d["w0"], d["s0"], d["b0"], wl, sl, L)
    return {k: gr[k] for k in GRAD_KEYS if gr[k] is not None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--chunk", type=int, default=4, help="batch entries per task")
    a = ap.parse_args()
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    result = {}
    ctx = mp.get_context("fork")
    for case, w, L in cases():
        t0 = time.time()
        if w.name not in _D:
            _D.clear()
            _D[w.name] = workload_inputs(w)
        d = _D[w.name]
        tasks = [(w.name, L, b, min(b + a.chunk, w.B)) for b in range(0, w.B, a.chunk)]
        with ctx.Pool(a.procs) as pool:
            parts = pool.map(_task, tasks, chunksize=1)
        tot = {}
        for p in parts:   # fixed order: batch chunk order
            for k, v in p.items():
                tot[k] = v if k not in tot else tot[k] + v
        for k, v in tot.items():
            result[f"{case}|{k}"] = np.asarray(v, dtype=np.float64)
        sub = dict(d)
        if L > 0:
            sub["wl"], sub["sl"] = d["wl"][:L], d["sl"][:L]
        else:
            sub["wl"] = sub["sl"] = None
        result[f"{case}|inputs_sha256"] = np.array(inputs_sha256(sub))
        print(f"{case}: {len(tasks)} tasks, {time.time() - t0:.1f} s", flush=True)
    np.savez_compressed(OUT, **result)
    print(f"wrote {OUT} ({os.path.getsize(OUT)} bytes)")


if __name__ == "__main__":
    main()
