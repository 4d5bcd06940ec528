"""The C-ABI layer (api.cpp: argument checks, routing and slicing, mxq_pack;
workspace.cpp: the split workspace cache) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU.

The HIP runtime and the kernel-side launchers are host stand-ins
(tests/sanitize/): each launch touches every byte range the real kernel would
read or write, computed from its arguments, on exact-size host buffers, so a
wrong pointer or size in the C-ABI layer is a sanitizer report.  Device code
is not part of this build (no GPU sanitizer is used).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_matmul_qmv_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "workspace.cpp"),
           os.path.join(SAN, "hip_stub.cpp"), os.path.join(SAN, "kernel_stub.cpp"), os.path.join(SAN, "driver.cpp")]


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("sanitize") / "mxq_sanitize")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *SOURCES, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stderr[-4000:]}"
    return exe


def test_c_abi_layer_under_asan_and_ubsan(sanitized_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "sanitize driver: ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
