"""The host-validation tests of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The ABI layer (``csrc/abi.cpp``) is compiled for the host alone with g++ and both sanitizers,
linked with launcher stand-ins that never run anything (``tests/asan/launch_stubs.cpp``; no
validation test reaches a launch), and ``tests/test_abi_cpu.py`` runs against that library in a
child process with the ASan runtime preloaded.  Any out-of-bounds access, use of freed memory,
signed overflow, misaligned access or other undefined behaviour on the host side of the ABI ends
that run with an error.  Host code only: nothing here is built for or runs on a GPU.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    return gxx


def test_abi_host_validation_under_sanitizers(tmp_path):
    gxx = _gxx()
    lib = str(tmp_path / "libdiffattn_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    asan_rt = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.isabs(asan_rt) and os.path.exists(asan_rt), asan_rt
    env = dict(os.environ)
    env.update({
        "DIFFATTN_SANITIZED_LIB": lib,
        "LD_PRELOAD": asan_rt,
        # the Python interpreter itself is not built for leak checking
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=97",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "failed" not in r.stdout, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
