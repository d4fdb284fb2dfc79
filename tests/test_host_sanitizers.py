"""The C ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is built a second time with
kvc_api.cpp compiled by g++ -fsanitize=address,undefined (any finding
aborts), and the host-logic tests (test_library_abi.py, test_host_validation.py)
run against that build in a child process that preloads the sanitizer
runtime.  Header parsing, CRC, size queries, parameter and buffer checks,
table exports and every early error path are covered; device code is the
same object as in the product build and is not instrumented."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    gxx = shutil.which("g++")
    if not gxx:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def checked_lib():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only checks (stand-in device pointers): kept off GPUs")
    if not _runtime("libasan.so"):
        pytest.skip("g++ AddressSanitizer runtime not installed")
    from entropy_coding_amd import build
    if not os.path.exists(os.path.join(build.HERE, "_build", "kvc_kernels.o")):
        build.build()
    return build.build_checked()


def test_host_logic_under_address_and_undefined_behaviour_sanitizers(checked_lib):
    env = dict(os.environ)
    env["KVC_LIBRARY"] = checked_lib
    # the interpreter is not built with the sanitizer: its runtime goes first
    env["LD_PRELOAD"] = ":".join(p for p in [_runtime("libasan.so"), env.get("LD_PRELOAD", "")] if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    probe = ("import ctypes; from entropy_coding_amd import kvc; "
             "assert kvc.LIB_PATH.endswith('libkvc_checked.so'), kvc.LIB_PATH; "
             "ctypes.CDLL(None).__asan_report_load8; print('sanitized', kvc.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_library_abi.py", "tests/test_host_validation.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
