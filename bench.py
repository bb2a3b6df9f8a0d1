"""Benchmark of the fused WTConv forward + backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--level L]
                    [--impl fused|unfused] [--no-cpu-baseline] [--no-summary]

One step = one wtconv_forward + one wtconv_backward (every kernel of the hot
path) over one batch of synthetic, seeded inputs already resident in HBM.
Input buffer sets are rotated so that the working set of consecutive steps
exceeds the 256 MB Infinity Cache.  Prints ONE JSON line.

Default workload: the level sweep block, B=64, C=96, 128 x 128, k=5, fp32, at
L=3 (the largest single-GPU configuration; the other levels and every other
workload are timed in `per_workload`).

value    = achieved HBM throughput of the step in GB/s: the fused I/O model's
           bytes (forward: read x, write out; backward: read x and g, write
           dx; plus parameters and partial sums) / measured step time.
roofline = the dominant call, wtconv_backward (the fused backward kernel and
           its small finalize), against the 8 TB/s HBM peak: algorithmic bytes
           per call (3 e N: read x and g, write dx) / its duration, timed live
           with HIP events on the launch stream over the timed steps; beside
           it the same call against the VALU peaks.
cpu_baseline = the float64 CPU oracle on the host's cores (a baseline, not a target).
"""

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Published fp32 vector peak of MI355X (packed FP32 FMA): 157.3 TFLOP/s.  The
# library is built with packed-FP32 instructions disabled, so the peak its
# code can reach is half of it: 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA)
# x 2.4 GHz = 78.6 TFLOP/s.
VALU_PACKED_PEAK_TFLOPS = 157.3
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
HEADLINE = "sweep_b64c96_128x128"
HEADLINE_L = 3
MALL_BYTES = 256 * 2 ** 20
COPY_PROBE_MIB = 1024


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--level", type=int, default=None, help="override L (sweep workload)")
    p.add_argument("--impl", default="fused", choices=["fused", "unfused"])
    p.add_argument("--layout", default="nchw", choices=["nchw", "nhwc", "nhwc_inplace"],
                   help="activation memory layout: nhwc = torch.channels_last tensors through NCHW copies "
                        "(layout 1), nhwc_inplace = read and written in place (layout 2)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-summary", action="store_true")
    p.add_argument("--torch-dwconv", action="store_true",
                   help="also time PyTorch's depthwise k x k convolution (MIOpen) at the headline shape")
    p.add_argument("--profile-steps", type=int, default=None,
                   help="run only this many calls, no summary / CPU baseline (for rocprofv3)")
    p.add_argument("--profile-only", default="both", choices=["both", "fwd", "bwd"],
                   help="with --profile-steps: call only the forward or only the backward entry point, so "
                        "that every library kernel of the run belongs to that direction")
    p.add_argument("--corr-calls", type=int, default=None,
                   help="run only the base-correlation comparison with this many calls per path (kernel traces)")
    p.add_argument("--copy-probe-mib", type=int, default=None,
                   help="run a plain device copy (read N + write N bytes) 3 times, to calibrate "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE against known traffic")
    p.add_argument("--stats-summary", nargs=2, metavar=("PROFILE_DIR", "OUT_TXT"), default=None,
                   help="format the kernel_stats.csv of a rocprofv3 --kernel-trace --stats --output-format csv "
                        "run as a text summary (no GPU needed)")
    p.add_argument("--pmc-summary", nargs=7, default=None,
                   metavar=("FWD_FETCH_DIR", "FWD_WRITE_DIR", "BWD_FETCH_DIR", "BWD_WRITE_DIR", "COPY_FETCH_DIR",
                            "COPY_WRITE_DIR", "OUT_TXT"),
                   help="turn FETCH_SIZE / WRITE_SIZE counter runs of --profile-steps --profile-only fwd|bwd and "
                        "of --copy-probe-mib into calibrated HBM bytes per call: writes OUT_TXT and "
                        "profiles/pmc_traffic.json")
    p.add_argument("--cmd", default="", help="command line recorded in a summary")
    p.add_argument("--source-hash", default=None,
                   help="with --pmc-summary: the kernel-source hash the profiled run printed (default: the "
                        "current sources')")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_bound_cnn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


class Runner:
    """Device buffers for one workload and one implementation."""

    def __init__(self, wl, L, impl, torch, binding, rotate=True, layout="nchw"):
        from memory_bound_cnn_amd.inputs import workload_inputs
        self.torch, self.b = torch, binding
        self.wl, self.L, self.impl = wl, L, impl
        dev = torch.device("cuda", 0)
        d = workload_inputs(wl)
        sd = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        e = 2 if wl.dtype == "bf16" else 4
        N = wl.B * wl.C * wl.H * wl.W
        set_bytes = 4 * N * e
        R = max(1, min(8, math.ceil(4 * MALL_BYTES / set_bytes))) if rotate else 1
        self.R = R
        x = torch.from_numpy(d["x"]).to(dev).to(sd)
        g = torch.from_numpy(d["g"]).to(dev).to(sd)
        if layout != "nchw":
            x = x.contiguous(memory_format=torch.channels_last)
            g = g.contiguous(memory_format=torch.channels_last)
        self.sets = []
        for r in range(R):
            fmt = torch.channels_last if layout != "nchw" else torch.contiguous_format
            xs = x if r == 0 else x.roll(r, dims=0).contiguous(memory_format=fmt)
            gs = g if r == 0 else g.roll(r, dims=0).contiguous(memory_format=fmt)
            self.sets.append(dict(x=xs, g=gs, out=torch.empty_like(x), dx=torch.empty_like(x)))
        f = lambda a: torch.from_numpy(a).to(dev)
        self.w0, self.s0, self.b0 = f(d["w0"]), f(d["s0"]), f(d["b0"])
        self.wl_ = f(d["wl"][:L]).contiguous() if L > 0 else None
        self.sl_ = f(d["sl"][:L]).contiguous() if L > 0 else None
        C, k = wl.C, wl.k
        f32 = dict(dtype=torch.float32, device=dev)
        self.grads = dict(dw0=torch.empty(C, k, k, **f32), ds0=torch.empty(C, **f32), db0=torch.empty(C, **f32),
                          dwl=torch.empty(L, 4 * C, k, k, **f32) if L > 0 else None,
                          dsl=torch.empty(L, 4 * C, **f32) if L > 0 else None)
        shp = (wl.B, wl.C, wl.H, wl.W, L, k, wl.dtype)
        lay = {"nchw": 0, "nhwc": 1, "nhwc_inplace": 2}[layout]
        self.in_place = layout == "nhwc_inplace"
        if impl == "fused":
            self.fwd, self.bwd = binding.wtconv_forward, binding.wtconv_backward
            wsf = binding.wtconv_forward_workspace(*shp, layout=lay)
            wsb = binding.wtconv_backward_workspace(*shp, layout=lay)
        else:
            self.fwd, self.bwd = binding.wtconv_forward_unfused, binding.wtconv_backward_unfused
            wsf = binding.wtconv_forward_unfused_workspace(*shp, layout=lay)
            wsb = binding.wtconv_backward_unfused_workspace(*shp, layout=lay)
        self.ws_f = torch.empty(max(wsf, 1), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        self.N, self.e = N, e

    def step(self, i, ev=None, only="both"):
        s = self.sets[i % self.R]
        if ev is not None:
            ev[0].record()
        kw = {"in_place": True} if self.in_place else {}
        if only != "bwd":
            self.fwd(s["x"], self.w0, self.s0, self.b0, self.wl_, self.sl_, self.L, out=s["out"],
                     workspace=self.ws_f, **kw)
        if ev is not None:
            ev[1].record()
        if only != "fwd":
            self.bwd(s["x"], s["g"], self.w0, self.s0, self.wl_, self.sl_, self.L, dx=s["dx"], grads=self.grads,
                     workspace=self.ws_b, **kw)
        if ev is not None:
            ev[2].record()

    def time(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            self.step(i, evs[i])
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        return total_ms / steps, fwd_ms, bwd_ms


def dwconv_comparison(wl, torch, binding, with_torch):
    """WTConv against the plain depthwise convolution it replaces, at one
    shape: this library's L-level k x k operator, its L = 0 path (a k x k
    depthwise conv with scale and bias) at k = 5 and at k = 7 (the ConvNeXt
    block's kernel), and optionally PyTorch's depthwise conv (MIOpen) with
    autograd for the backward (dx, dW, db).  fwd+bwd ms per call pair."""
    import dataclasses
    res = {"shape": {"B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W, "storage": wl.dtype}}
    cases = {f"wtconv_L{wl.L}_k{wl.k}": (wl.L, wl.k), "dwconv_L0_k5": (0, 5), "dwconv_L0_k7": (0, 7)}
    for label, (Lc, kc) in cases.items():
        ww = dataclasses.replace(wl, name=f"{wl.name}_{label}", L=Lc, k=kc, L_max=Lc, sweep=())
        rr = Runner(ww, Lc, "fused", torch, binding)
        m, mf, mb = rr.time(50, 5)
        del rr
        res[label] = {"ms": round(m, 5), "fwd_ms": round(mf, 5), "bwd_ms": round(mb, 5)}
    if with_torch:
        import torch.nn.functional as F
        sd = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        x = torch.randn(wl.B, wl.C, wl.H, wl.W, device="cuda", dtype=sd, requires_grad=True)
        g = torch.randn_like(x)
        w = torch.randn(wl.C, 1, 7, 7, device="cuda", dtype=sd, requires_grad=True)
        b = torch.randn(wl.C, device="cuda", dtype=sd, requires_grad=True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        fw, bw = [], []
        for i in range(25):
            ev[0].record()
            y = F.conv2d(x, w, b, padding=3, groups=wl.C)
            ev[1].record()
            y.backward(g)
            ev[2].record()
            torch.cuda.synchronize()
            if i >= 5:
                fw.append(ev[0].elapsed_time(ev[1]))
                bw.append(ev[1].elapsed_time(ev[2]))
            x.grad = w.grad = b.grad = None
        res["torch_dwconv_k7"] = {"ms": round(sum(fw) / len(fw) + sum(bw) / len(bw), 5),
                                  "fwd_ms": round(sum(fw) / len(fw), 5), "bwd_ms": round(sum(bw) / len(bw), 5)}
    base = res["dwconv_L0_k7"]["ms"]
    res["wtconv_over_dwconv_k7"] = round(res[f"wtconv_L{wl.L}_k{wl.k}"]["ms"] / base, 3)
    return res


def channels_last_comparison(torch, binding):
    """Fused forward + backward on channels-last tensors -- through NCHW copies
    (layout 1) and in place (layout 2) -- against the same workload in NCHW,
    ms per step."""
    from memory_bound_cnn_amd.inputs import WORKLOADS
    res = []
    for name in ("stage1_b32c96_64x64_L3", "bf16_b64c192_32x32_L3", "odd_b128c384_14x14_L2"):
        w = WORKLOADS[name]
        row = {"workload": name, "L": w.L}
        for layout in ("nchw", "nhwc", "nhwc_inplace"):
            rr = Runner(w, w.L, "fused", torch, binding, layout=layout)
            m, mf, mb = rr.time(50, 5)
            del rr
            row[layout] = {"ms": round(m, 5), "fwd_ms": round(mf, 5), "bwd_ms": round(mb, 5)}
        row["nhwc_over_nchw"] = round(row["nhwc"]["ms"] / row["nchw"]["ms"], 3)
        row["nhwc_inplace_over_nchw"] = round(row["nhwc_inplace"]["ms"] / row["nchw"]["ms"], 3)
        res.append(row)
        torch.cuda.empty_cache()
    return res


def base_correlation_comparison(torch, binding, calls=50, profile=False):
    """The base level's weight-gradient correlation on its own, on the bf16
    workload's shape (64 x 192 planes of 32 x 32, k = 5): the vector-unit
    correlation tiles of the level-by-level path against the matrix-core
    kernel, us per call and the rate of reading x and g once.  profile: just
    run the calls (for a kernel trace)."""
    from memory_bound_cnn_amd.inputs import WORKLOADS
    w = WORKLOADS["bf16_b64c192_32x32_L3"]
    gen = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(w.B, w.C, w.H, w.W, device="cuda", generator=gen).to(torch.bfloat16)
    g = torch.randn(w.B, w.C, w.H, w.W, device="cuda", generator=gen).to(torch.bfloat16)
    res = {"shape": {"B": w.B, "C": w.C, "H": w.H, "W": w.W, "k": w.k, "storage": "bf16"},
           "bytes_per_call": 2 * x.numel() * 2}
    outs = {}
    for label, impl in (("valu", binding.CORR_VALU), ("mfma", binding.CORR_MFMA)):
        out = torch.empty(w.C, w.k, w.k, device="cuda")
        ws = torch.empty(binding.wtconv_base_correlation_workspace(w.B, w.C, w.H, w.W, w.k, "bf16", impl),
                         dtype=torch.uint8, device="cuda")
        for _ in range(3 if not profile else 0):
            binding.wtconv_base_correlation(x, g, w.k, impl, out=out, workspace=ws)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(calls):
            binding.wtconv_base_correlation(x, g, w.k, impl, out=out, workspace=ws)
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / calls * 1e3
        res[label] = {"us": round(us, 2), "gbps": round(res["bytes_per_call"] / (us * 1e-6) / 1e9, 1)}
        outs[label] = out
    ref = outs["valu"]
    res["mfma_over_valu_max_rel_diff"] = float((outs["mfma"] - ref).abs().max() / ref.pow(2).mean().sqrt())
    res["mfma_speedup"] = round(res["valu"]["us"] / res["mfma"]["us"], 2)
    return res


def memory_comparison(wl, L, torch, binding):
    """Peak device memory of one training-style step (forward, then backward
    of <out, g>) through the autograd wrapper, above the memory already held
    by the inputs and parameters: the fused kernels against the level-by-level
    baseline."""
    from memory_bound_cnn_amd.autograd import wtconv
    from memory_bound_cnn_amd.inputs import workload_inputs
    d = workload_inputs(wl)
    sd = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda", 0)
    x0 = torch.from_numpy(d["x"]).to(dev).to(sd)
    g = torch.from_numpy(d["g"]).to(dev).to(sd)
    prm = {k: torch.from_numpy(d[k][:L] if k in ("wl", "sl") else d[k]).to(dev).contiguous()
           for k in ("w0", "s0", "b0", "wl", "sl")}
    shp = (wl.B, wl.C, wl.H, wl.W, L, wl.k, wl.dtype)
    res = {"workload": wl.name, "L": L, "input_bytes": x0.numel() * x0.element_size()}
    for impl in ("fused", "unfused"):
        x = x0.clone().requires_grad_(True)
        p = {k: v.clone().requires_grad_(True) for k, v in prm.items()}
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        y = wtconv(x, p["w0"], p["s0"], p["b0"], p["wl"], p["sl"], L, impl=impl)
        y.backward(g)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        if impl == "fused":
            ws = (binding.wtconv_forward_workspace(*shp), binding.wtconv_backward_workspace(*shp))
        else:
            ws = (binding.wtconv_forward_unfused_workspace(*shp), binding.wtconv_backward_unfused_workspace(*shp))
        res[impl] = {"peak_bytes_above_inputs": int(peak), "fwd_workspace_bytes": ws[0],
                     "bwd_workspace_bytes": ws[1]}
        del y, x, p
    res["unfused_over_fused_peak"] = round(res["unfused"]["peak_bytes_above_inputs"] /
                                           res["fused"]["peak_bytes_above_inputs"], 3)
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores
# ---------------------------------------------------------------------------
def _oracle_task(args):
    os.environ["OMP_NUM_THREADS"] = "1"
    x, g, w0, s0, b0, wl_, sl_, L = args
    import oracle
    t0 = time.perf_counter()
    oracle.forward(x, w0, s0, b0, wl_, sl_, L)
    oracle.backward(x, g, w0, s0, b0, wl_, sl_, L)
    return time.perf_counter() - t0


def host_cores():
    """Host cores this process may use, capped at the 16 host CPUs a one-GPU
    share of the box provides (whatever the affinity mask lists)."""
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return max(1, min(16, ncpu)), ncpu


def cpu_baseline(wl, L, bytes_per_batch_entry, budget_s=20.0):
    """Time the float64 oracle (forward + backward) on a bounded sample of the
    workload: whole batch entries, one per task, on a pool of host processes
    (one per usable core, one thread each), about `budget_s` seconds of CPU
    work in total (the batch is cycled through when one pass over it is
    shorter than that).  Also the warm one-core time of one entry (after a
    first call has paid the imports and page faults)."""
    from memory_bound_cnn_amd.inputs import workload_inputs
    cores, ncpu = host_cores()
    d = workload_inputs(wl)
    wl_ = d["wl"][:L] if L > 0 else None
    sl_ = d["sl"][:L] if L > 0 else None
    task = lambda b: (d["x"][b:b + 1], d["g"][b:b + 1], d["w0"], d["s0"], d["b0"], wl_, sl_, L)
    _oracle_task(task(0))                           # cold call: imports, page faults
    t1 = _oracle_task(task(1 % wl.B))               # warm: one entry, one core
    n_entries = int(max(cores, math.ceil(budget_s / max(t1, 1e-3))))
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_task, [task(0)] * cores)   # warm the workers (imports)
        t0 = time.perf_counter()
        pool.map(_oracle_task, [task(b % wl.B) for b in range(n_entries)], chunksize=1)
        wall = time.perf_counter() - t0
    value = n_entries * bytes_per_batch_entry / wall / 1e9
    return dict(value=value, unit="GB/s", cores=cores, kind="oracle",
                sample=f"{n_entries} batch entries of {wl.name} at L={L} (B={wl.B}; entries cycled), "
                       f"{n_entries * t1:.0f} s of CPU work at the warm one-core rate: float64 NumPy oracle, forward + "
                       f"backward, one batch entry per task on a pool of {cores} processes (1 thread each; affinity "
                       f"lists {ncpu} CPUs, a one-GPU share is 16); wall {wall:.2f} s",
                wall_s=round(wall, 3), entries=n_entries,
                one_core=dict(value=round(bytes_per_batch_entry / t1 / 1e9, 4), unit="GB/s",
                              seconds_per_entry=round(t1, 3)))


# ---------------------------------------------------------------------------
# rocprofv3 summaries (CSV output) -> committed text summaries
# ---------------------------------------------------------------------------
def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for fn in sorted(files):
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise SystemExit(f"no *{suffix} under {d}")


def _rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def is_library_kernel(name):
    """Kernels of libwtconv (namespace wtc); torch's own set-up kernels and
    runtime copies are not."""
    return "wtc::" in name


def _short(name, n=96):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= n else name[:n - 3] + "..."


def stats_summary(prof_dir, out_txt, cmd):
    rows = _rows(_find_csv(prof_dir, "kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}", "",
             f"{'kernel':96s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s} {'pct':>6s}"]
    for r in rows:
        calls = int(_col(r, "Calls"))
        lines.append(f"{_short(_col(r, 'Name', 'KernelName')):96s} {calls:6d} "
                     f"{float(_col(r, 'AverageNs')) / 1e3:9.2f} {float(_col(r, 'MinNs')) / 1e3:9.2f} "
                     f"{float(_col(r, 'MaxNs')) / 1e3:9.2f} {float(_col(r, 'TotalDurationNs')) / 1e3:10.1f} "
                     f"{float(_col(r, 'Percentage')):6.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_totals(d, counter):
    """Per kernel name: (sum of the counter over its dispatches in KiB, dispatches)."""
    acc = {}
    for r in _rows(_find_csv(d, "counter_collection.csv")):
        if _col(r, "Counter_Name", "counter_name") != counter:
            continue
        k = _col(r, "Kernel_Name", "kernel_name")
        v = acc.setdefault(k, [0.0, 0])
        v[0] += float(_col(r, "Counter_Value", "value"))
        v[1] += 1
    return acc


def pmc_summary(dirs, out_txt, cmd, wl_name, L, source_hash=None, layout="nchw"):
    """Calibrated HBM bytes per call of each direction from FETCH_SIZE and
    WRITE_SIZE runs (one counter per run) that called only that direction.
    Every library kernel of such a run belongs to the direction; the calls
    are counted as the fewest dispatches of any library kernel (each kernel
    of a call runs at least once per call)."""
    from memory_bound_cnn_amd.inputs import WORKLOADS
    fwd_f, fwd_w, bwd_f, bwd_w, cfetch_dir, cwrite_dir = dirs
    cf, cw = _pmc_totals(cfetch_dir, "FETCH_SIZE"), _pmc_totals(cwrite_dir, "WRITE_SIZE")
    # the copy probe's kernel is the kernel moving the most bytes per dispatch
    ck = max(cf, key=lambda k: cf[k][0] / cf[k][1])
    copy_bytes = float(COPY_PROBE_MIB * 2 ** 20)
    f_fac = copy_bytes / (cf[ck][0] / cf[ck][1] * 1024.0)
    w_fac = copy_bytes / (cw[ck][0] / cw[ck][1] * 1024.0)
    wl = WORKLOADS[wl_name]
    shp = (wl.B, wl.C, wl.H, wl.W, L, wl.k, wl.dtype)
    tot, per_kernel = {}, {}
    for role, fd, wd in (("fwd", fwd_f, fwd_w), ("bwd", bwd_f, bwd_w)):
        fetch = {k: v for k, v in _pmc_totals(fd, "FETCH_SIZE").items() if is_library_kernel(k)}
        write = {k: v for k, v in _pmc_totals(wd, "WRITE_SIZE").items() if is_library_kernel(k)}
        calls_f = min(v[1] for v in fetch.values())
        calls_w = min(v[1] for v in write.values())
        rb = sum(v[0] for v in fetch.values()) * 1024.0 * f_fac / calls_f
        wb = sum(v[0] for v in write.values()) * 1024.0 * w_fac / calls_w
        tot[role] = rb + wb
        for k in sorted(set(fetch) | set(write)):
            fv, wv = fetch.get(k, (0.0, 1)), write.get(k, (0.0, 1))
            per_kernel[f"{role}: {_short(k)}"] = {
                "read_bytes_per_call": fv[0] * 1024.0 * f_fac / calls_f,
                "write_bytes_per_call": wv[0] * 1024.0 * w_fac / calls_w,
                "dispatches_per_call": fv[1] / calls_f}
    from memory_bound_cnn_amd import binding
    lay = {"nchw": 0, "nhwc": 1, "nhwc_inplace": 2}[layout]
    model = {"fwd": binding.wtconv_io_model_bytes(*shp, impl=0, direction=0, layout=lay),
             "bwd": binding.wtconv_io_model_bytes(*shp, impl=0, direction=1, layout=lay)}
    rec = {"source_hash": source_hash or kernel_source_hash(),
           "calibration": {"copy_kernel": _short(ck), "copy_bytes_each_way": copy_bytes,
                           "fetch_factor": f_fac, "write_factor": w_fac},
           "workloads": {f"{wl_name}_L{L}" + ("" if layout == "nchw" else "_" + layout): {"fwd_bytes": tot["fwd"], "bwd_bytes": tot["bwd"],
                                             "model_fwd_bytes": model["fwd"], "model_bwd_bytes": model["bwd"],
                                             "command": cmd, "kernels": per_kernel}}}
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    old = {}
    if os.path.exists(path):
        try:
            old = json.load(open(path))
        except ValueError:
            old = {}
    if old.get("source_hash") == rec["source_hash"]:
        old["workloads"].update(rec["workloads"])
        rec["workloads"] = old["workloads"]
    json.dump(rec, open(path, "w"), indent=1)
    lines = ["# rocprofv3 FETCH_SIZE / WRITE_SIZE per call, calibrated against a plain copy",
             f"# command: {cmd}", "",
             f"copy probe: {_short(ck)} moving {copy_bytes:.0f} B each way; FETCH_SIZE reads "
             f"{cf[ck][0] / cf[ck][1]:.1f} KiB -> factor {f_fac:.4f}; WRITE_SIZE reads "
             f"{cw[ck][0] / cw[ck][1]:.1f} KiB -> factor {w_fac:.4f}",
             f"workload {wl_name} L={L} layout {layout}", ""]
    for k, v in per_kernel.items():
        lines.append(f"{k:104s} x{v['dispatches_per_call']:.0f}/call: read {v['read_bytes_per_call'] / 1e6:9.2f} MB, "
                     f"write {v['write_bytes_per_call'] / 1e6:9.2f} MB")
    for r in ("fwd", "bwd"):
        lines.append(f"{r}: measured {tot[r] / 1e6:.2f} MB per call vs I/O model {model[r] / 1e6:.2f} MB "
                     f"(ratio {tot[r] / model[r]:.3f})")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_from_profiles(wl, L, layout="nchw"):
    """HBM bytes per call (fwd_bytes, bwd_bytes) from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except ValueError:
        return None
    key = f"{wl.name}_L{L}" + ("" if layout == "nchw" else "_" + layout)
    r = rec.get("workloads", {}).get(key)
    if not r or rec.get("source_hash") != kernel_source_hash():
        return None
    return r


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the operator has no multi-GPU path "
                                   "(batch sharding needs only an all-reduce of the tiny weight gradients); "
                                   "run with --gpus 1"}))
        sys.exit(2)
    from memory_bound_cnn_amd import binding
    from memory_bound_cnn_amd.inputs import WORKLOADS
    binding.load_library()
    wl = WORKLOADS[a.workload]
    L = (HEADLINE_L if wl.name == HEADLINE else wl.L) if a.level is None else a.level
    if a.stats_summary:
        stats_summary(a.stats_summary[0], a.stats_summary[1], a.cmd)
        return
    if a.pmc_summary:
        pmc_summary(a.pmc_summary[:6], a.pmc_summary[6], a.cmd, wl.name, L, a.source_hash, a.layout)
        return
    shp = (wl.B, wl.C, wl.H, wl.W, L, wl.k, wl.dtype)
    lay = {"nchw": 0, "nhwc": 1, "nhwc_inplace": 2}[a.layout]
    io_f = binding.wtconv_io_model_bytes(*shp, impl=0, direction=0, layout=lay)
    io_b = binding.wtconv_io_model_bytes(*shp, impl=0, direction=1, layout=lay)

    # The CPU baseline runs first, before this process touches the GPU.
    cpu = None
    if not a.no_cpu_baseline and a.profile_steps is None and a.copy_probe_mib is None and a.corr_calls is None:
        cpu = cpu_baseline(wl, L, (io_f + io_b) / wl.B)
        cpu["value"] = round(cpu["value"], 4)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    if a.corr_calls is not None:
        print(json.dumps({"base_correlation_comparison":
                          base_correlation_comparison(torch, binding, calls=a.corr_calls, profile=True)}))
        return

    if a.copy_probe_mib is not None:
        if a.copy_probe_mib != COPY_PROBE_MIB:
            raise SystemExit(f"--copy-probe-mib must be {COPY_PROBE_MIB} (the size the calibration assumes)")
        n = a.copy_probe_mib * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}))
        return

    if a.profile_steps is not None:
        r = Runner(wl, L, a.impl, torch, binding, layout=a.layout)
        for i in range(a.profile_steps):
            r.step(i, only=a.profile_only)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": wl.name, "L": L, "impl": a.impl, "calls": a.profile_steps,
                          "only": a.profile_only, "layout": a.layout, "source_hash": kernel_source_hash()}))
        return

    r = Runner(wl, L, a.impl, torch, binding, layout=a.layout)
    ms, fwd_ms, bwd_ms = r.time(a.steps, a.warmup)
    fl_f = binding.wtconv_flops(*shp, direction=0)
    fl_b = binding.wtconv_flops(*shp, direction=1)
    gbps = (io_f + io_b) / (ms * 1e-3) / 1e9
    tflops_b = fl_b / (bwd_ms * 1e-3) / 1e12
    tflops_f = fl_f / (fwd_ms * 1e-3) / 1e12
    line = {
        "metric": "WTConv fwd+bwd ms/iter and achieved HBM GB/s (% of MI355X peak) per level L",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "fp32" else "bf16-storage/f32-compute",
        "data": "synthetic (seeded N(0,1) inputs and gradients, N(0,1/k^2) weights, U[0.05,0.5] scales)",
        "config": {"workload": wl.name, "B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W, "L": L, "k": wl.k,
                   "storage": wl.dtype, "impl": a.impl, "layout": a.layout},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "io_model_bytes": {"fwd": io_f, "bwd": io_b},
        "flops": {"fwd": fl_f, "bwd": fl_b},
        "buffer_sets_rotated": r.R,
    }
    tr = traffic_from_profiles(wl, L, a.layout)
    # dominant call: wtconv_backward; algorithmic bytes per call = 3 e N
    alg_b = 3.0 * r.e * r.N
    alg_f = 2.0 * r.e * r.N
    gbps_b = alg_b / (bwd_ms * 1e-3) / 1e9
    gbps_f = alg_f / (fwd_ms * 1e-3) / 1e9
    line["roofline"] = {
        "bound": "hbm",
        "kernel": "wtconv_backward: the fused backward kernel and its finalize (the dominant call of the step)",
        "achieved": round(gbps_b, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(gbps_b / HBM_PEAK_GBPS, 4),
        "traffic": tr["bwd_bytes"] if tr else None,
        "algorithmic_bytes_per_launch": alg_b,
        "algorithmic_bytes_per_pixel": 3 * r.e,
        "pixels_per_launch": r.N,
        "launch_ms": round(bwd_ms, 5),
        "timing": "HIP events on the launch stream around each wtconv_backward call of the timed steps, averaged",
        "alu": {"achieved_tflops": round(tflops_b, 3),
                "frac_of_published_fp32_peak": round(tflops_b / VALU_PACKED_PEAK_TFLOPS, 4),
                "published_fp32_peak_tflops": VALU_PACKED_PEAK_TFLOPS,
                "frac_of_nonpacked_peak": round(tflops_b / VALU_PEAK_TFLOPS, 4),
                "nonpacked_peak_tflops": round(VALU_PEAK_TFLOPS, 1),
                "note": "the library is built without packed-FP32 instructions, so 78.6 TFLOP/s is the "
                        "highest VALU rate its code can reach"},
        "forward": {"achieved": round(gbps_f, 1), "frac": round(gbps_f / HBM_PEAK_GBPS, 4),
                    "launch_ms": round(fwd_ms, 5), "algorithmic_bytes_per_launch": alg_f,
                    "traffic": tr["fwd_bytes"] if tr else None,
                    "alu_frac_of_nonpacked_peak": round(tflops_f / VALU_PEAK_TFLOPS, 4)},
    }
    if tr:
        line["measured_bytes_over_model"] = {"fwd": tr["fwd_bytes"] / io_f, "bwd": tr["bwd_bytes"] / io_b}

    if not a.no_summary:
        summary = []
        for name, w in WORKLOADS.items():
            levels = w.sweep if w.sweep else (w.L,)
            for Lw in levels:
                ww = w.at_level(Lw)
                sh = (ww.B, ww.C, ww.H, ww.W, Lw, ww.k, ww.dtype)
                row = {"workload": name, "L": Lw}
                for impl in ("fused", "unfused"):
                    try:
                        rr = Runner(ww, Lw, impl, torch, binding)
                        steps = max(10, min(100, int(2e5 / max(1, ww.B * ww.C * ww.H * ww.W / 1e3))))
                        m, mf, mb = rr.time(steps, 5)
                        del rr
                        torch.cuda.empty_cache()
                    except Exception as ex:  # noqa: BLE001 - report and continue
                        row[impl] = {"error": str(ex)[:200]}
                        continue
                    model = binding.wtconv_io_model_bytes(*sh, impl=0, direction=0) + \
                        binding.wtconv_io_model_bytes(*sh, impl=0, direction=1)
                    fl = binding.wtconv_flops(*sh, direction=0) + binding.wtconv_flops(*sh, direction=1)
                    row[impl] = {"ms": round(m, 5), "fwd_ms": round(mf, 5), "bwd_ms": round(mb, 5),
                                 "gbps_fused_model": round(model / (m * 1e-3) / 1e9, 1),
                                 "pct_hbm_peak": round(100 * model / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                                 "pct_valu_peak": round(100 * fl / (m * 1e-3) / 1e12 / VALU_PEAK_TFLOPS, 2)}
                trw = traffic_from_profiles(ww, Lw)
                if trw and "ms" in row.get("fused", {}):
                    mf_ = binding.wtconv_io_model_bytes(*sh, impl=0, direction=0)
                    mb_ = binding.wtconv_io_model_bytes(*sh, impl=0, direction=1)
                    row["fused"]["measured_bytes_over_model"] = {"fwd": round(trw["fwd_bytes"] / mf_, 4),
                                                                 "bwd": round(trw["bwd_bytes"] / mb_, 4)}
                    row["fused"]["gbps_measured_bytes"] = round(
                        (trw["fwd_bytes"] + trw["bwd_bytes"]) / (row["fused"]["ms"] * 1e-3) / 1e9, 1)
                if "ms" in row.get("fused", {}) and "ms" in row.get("unfused", {}):
                    row["speedup_vs_unfused"] = round(row["unfused"]["ms"] / row["fused"]["ms"], 3)
                    row["unfused_model_bytes"] = binding.wtconv_io_model_bytes(*sh, impl=1, direction=0) + \
                        binding.wtconv_io_model_bytes(*sh, impl=1, direction=1)
                summary.append(row)
        line["per_workload"] = summary
        line["dwconv_comparison"] = dwconv_comparison(wl.at_level(L), torch, binding, a.torch_dwconv)
        line["channels_last_comparison"] = channels_last_comparison(torch, binding)
        line["base_correlation_comparison"] = base_correlation_comparison(torch, binding)
        line["training_step_memory"] = memory_comparison(wl, L, torch, binding)

    if cpu is not None:
        line["cpu_baseline"] = cpu
        line["gpu_over_cpu"] = round(gbps / cpu["value"], 1)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
