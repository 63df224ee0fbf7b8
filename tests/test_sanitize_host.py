"""The library's pure C++ planners (varlen tile scheduler, congestion-free communication
planner, pipeline stage planner) built for the CPU with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by randomized pair, stage and copy tables
(tests/sanitize/plan_check.cpp): no sanitizer report, and every accepted plan keeps its
promises (tables inside the workspace, one send and one receive per worker and stage,
max-degree stages)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_wise_varlen_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp")] + \
    [os.path.join(CSRC, f) for f in ("fcp_plan.cpp", "fcp_comm.cpp", "fcp_pipeline.cpp")]


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path_factory.mktemp("sanitize") / "plan_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC] + SOURCES + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planners_under_sanitizers(plan_check, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([plan_check, str(seed), "1500"], capture_output=True, text=True,
                       timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failed checks" in r.stdout
