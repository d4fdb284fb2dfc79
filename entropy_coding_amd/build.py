"""Builds libkvc.so in-tree with hipcc for gfx950.

Flags that matter for bit-exactness of the shared CDF: no floating-point
contraction (-ffp-contract=off), float32 denormals kept
(-fno-gpu-flush-denormals-to-zero), and no packed-fp32 instructions.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvc.so")
ARCH = os.environ.get("KVC_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
DEVICE = [
    "-x", "hip", f"--offload-arch={ARCH}", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    rocm = os.path.dirname(os.path.dirname(cc))
    host_cxx = shutil.which("g++") or "g++"
    steps = [
        (cc, "kvc_kernels.hip", DEVICE),
        # the C ABI layer is host code only: plain g++ against the HIP runtime API
        (host_cxx, "kvc_api.cpp", ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
                                   "-Wall", "-Wextra"]),
    ]
    for comp, src, extra in steps:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [comp, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
