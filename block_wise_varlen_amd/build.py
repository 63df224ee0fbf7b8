"""Builds libfcp.so in-tree with hipcc for gfx950.

Every HIP/C++ source under csrc/ is compiled to an object (in parallel) and linked into
block_wise_varlen_amd/libfcp.so. Usage: ``python -m block_wise_varlen_amd.build``.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfcp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # No packed fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: every kernel runs two waves per SIMD (256 registers each).
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


# Per-source extra flags: the dQ kernel measured 1.6% faster with LLVM's max-ilp
# scheduling strategy (the forward and dK/dV kernels were no faster with it).
EXTRA_FLAGS = {
    "fcp_bwd_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = FLAGS + EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC] + flags + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + flags + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
