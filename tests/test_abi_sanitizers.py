"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (host only).

api.cpp is built with g++ and -fsanitize=address,undefined next to host stand-ins
for the kernel launchers (tests/asan/launch_stubs.cpp: every launcher refuses), and
the ABI test suite (tests/test_abi.py) runs against that build in a child process
with the sanitizer runtimes preloaded.  Any out-of-bounds access, overflow or other
undefined behaviour on the validation paths aborts the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_attention_v2_amd", "csrc")


def _runtime(gxx, name):
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_suite_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    lib = tmp_path / "libdiffattn_asan.so"
    build = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
             os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan, ubsan = _runtime(gxx, "libasan.so"), _runtime(gxx, "libubsan.so")
    assert asan and ubsan, "sanitizer runtimes not found"
    env = dict(os.environ, DIFFATTN_LIBRARY=str(lib), LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
