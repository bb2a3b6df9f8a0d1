"""The library's host side -- argument checks, launch planning, level peeling,
workspace layout, the channels-last adapter, the I/O and flop models
(wtconv_api.cpp, wtconv_plan.cpp) -- built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through a sweep of shapes
(tests/host/planner_sweep.cpp) with buffers of exactly the sizes the library
asks for.  The kernel launchers are host stand-ins (tests/host/planner_stubs.cpp)
that check each launch shape and touch every byte the kernels would read or
write, so a tensor, workspace region or record array sized too small fails here."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bound_cnn_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


def test_host_side_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "sweep"
    srcs = [os.path.join(CSRC, "wtconv_api.cpp"), os.path.join(CSRC, "wtconv_plan.cpp"),
            os.path.join(HOST, "planner_stubs.cpp"), os.path.join(HOST, "planner_sweep.cpp")]
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    subprocess.run([cxx] + flags + [f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}"] + srcs + ["-o", str(exe)],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "600"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "fails=0" in r.stdout
