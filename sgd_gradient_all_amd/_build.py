"""Build libddl.so in-tree with hipcc for gfx950.

Flags: no fast-math, no fp contraction, fp32 denormals kept, HIP's correctly
rounded fp32 division (the default), and packed fp32 instructions disabled.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libddl.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("schedule.cpp", "plan.cpp", "step_kernels.hip", "fused_kernel.hip",
                     "lars_kernels.hip")]

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
