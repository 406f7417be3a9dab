"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp (every argument check and the dispatch) is compiled for the host
with g++ -fsanitize=address,undefined, linked with stand-in launchers that
touch no device (tests/hostcheck/abi_stubs.cpp), and the whole of
tests/test_abi.py runs against that library in a child process with the
sanitizer runtimes preloaded.  Any sanitizer report fails the run.  CPU
only; no GPU and no HIP runtime calls are involved.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "hostcheck")
LIB = os.path.join(OUT, "libfa_hostcheck.so")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"],
                          stdout=subprocess.PIPE, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build():
    os.makedirs(OUT, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "exact_io_aware_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "tests", "hostcheck", "abi_stubs.cpp"),
           "-o", LIB]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    assert r.returncode == 0, "host-check build failed:\n" + r.stdout


@pytest.mark.timeout(600)
def test_abi_suite_under_asan_ubsan():
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    _build()
    env = dict(os.environ)
    env.update(FA_ABI_TEST_LIB=LIB, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=540)
    print(r.stdout[-3000:])
    assert r.returncode == 0, "ABI tests failed under the sanitizers"
    assert "ERROR: AddressSanitizer" not in r.stdout
    assert "runtime error" not in r.stdout
    assert " passed" in r.stdout
