"""Build libwtconv.so (HIP kernels + C ABI) for gfx950, in place.

    python -m memory_bound_cnn_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled; the
objects are linked into memory_bound_cnn_amd/libwtconv.so.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libwtconv.so")
OBJDIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("WTC_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function", "-Wno-uninitialized",
    "-Wno-unknown-warning-option", "-Wno-sometimes-uninitialized",
]

SOURCES = ["wtconv_fused.hip", "wtconv_fused_k1.hip", "wtconv_fused_k3.hip", "wtconv_fused_k5.hip",
           "wtconv_fused_k7.hip", "wtconv_fused_s_p64.hip", "wtconv_fused_s_p32.hip",
           "wtconv_fused_s_p128a.hip", "wtconv_fused_s_p128b.hip", "wtconv_fused_s_small.hip", "wtconv_fused_s_p112.hip",
           "wtconv_fused_s_dw.hip",
           "wtconv_tiny.hip", "wtconv_lane.hip", "wtconv_unfused.hip", "wtconv_top.hip", "wtconv_layout.hip", "wtconv_noalloc.hip", "wtconv_corr.hip", "wtconv_api.cpp", "wtconv_plan.cpp"]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
