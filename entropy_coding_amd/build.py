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


CHECKED_DIR = os.path.join(HERE, "_build", "checked")
CHECKED_LIB = os.path.join(CHECKED_DIR, "libkvc_checked.so")


def build_checked(verbose: bool = False) -> str:
    """A second build for the CPU tests only: the C ABI layer compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer (g++; any finding aborts
    the process), linked with the same device code into
    _build/checked/libkvc_checked.so.  The host tests load it in a child
    process that preloads the sanitizer runtime (the Python interpreter is
    not built with it).  It is never loaded on a GPU."""
    cc = hipcc()
    os.makedirs(CHECKED_DIR, exist_ok=True)
    rocm = os.path.dirname(os.path.dirname(cc))
    kern = os.path.join(HERE, "_build", "kvc_kernels.o")     # the device code of build()
    api = os.path.join(CHECKED_DIR, "kvc_api.o")
    host_cxx = shutil.which("g++") or "g++"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    cmds = [] if os.path.exists(kern) else [[cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, "kvc_kernels.hip"), "-o", kern]]
    cmds += [
        [host_cxx, *[f for f in COMMON if f != "-O3"], "-O1", *san, "-D__HIP_PLATFORM_AMD__",
         "-I" + os.path.join(rocm, "include"), "-Wall", "-Wextra", "-c", os.path.join(CSRC, "kvc_api.cpp"), "-o", api],
        [host_cxx, "-shared", *san, kern, api, "-o", CHECKED_LIB + ".tmp", "-L" + os.path.join(rocm, "lib"),
         "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64"],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
    os.replace(CHECKED_LIB + ".tmp", CHECKED_LIB)
    return CHECKED_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    if "--checked" in sys.argv:
        print(build_checked(verbose=True))
