"""Builds libslide.so (HIP kernels for gfx950 + host runtime) in-tree, next to this file.

    python -m layer_sliding_offloaded_fwd_amd.build

Every call recompiles every source. Device code: hipcc --offload-arch=gfx950 with packed-fp32
instructions disabled. The CPU optimizer (adamw.cpp) is compiled by g++ with
-ffp-contract=off and no fast-math, which its bit-exact operation order relies on.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libslide.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["gemm.hip", "attention.hip", "pointwise.hip", "ce.hip", "layer.hip",
               "adamw_gpu.hip"]
HIP_HOST_SOURCES = ["common.cpp", "ring.cpp", "linkprobe.cpp"]   # host code on the HIP runtime
CPU_SOURCES = ["adamw.cpp", "tier.cpp"]

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
# the GPU AdamW matches the CPU one's rounding only without fused multiply-adds
PER_FILE_FLAGS = {"adamw_gpu.hip": ["-ffp-contract=off"]}
CPU_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-pthread",
             "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src in CPU_SOURCES:
        cmd = ["g++", *CPU_FLAGS, "-c", path, "-o", obj]
    elif src in HIP_HOST_SOURCES:
        cmd = [HIPCC, "-x", "hip", *HIP_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *HIP_FLAGS, *PER_FILE_FLAGS.get(src, []), "-c", path, "-o", obj]
    _run(cmd)
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    sources = HIP_SOURCES + HIP_HOST_SOURCES + CPU_SOURCES
    jobs = jobs or min(len(sources), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread",
          "-lhsa-runtime64"])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
