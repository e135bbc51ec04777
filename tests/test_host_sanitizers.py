"""The library's host C++ (expand.cpp, index.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer and run through every expander, the class table
and the 47-bit rank (tests/sanitizer_driver.py), with results checked against
the oracle's unpackers.  CPU only: g++ builds the host sources alone (no HIP
file), and the driver runs in a child process with the sanitizer runtimes
preloaded, so any report aborts it with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_gemv_lvq_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("no sanitizer runtimes in this toolchain")
    lib = str(tmp_path / "liblvq_host_san.so")
    build = (["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared"] + SAN +
             [os.path.join(CSRC, "expand.cpp"), os.path.join(CSRC, "index.cpp"), "-o", lib])
    b = subprocess.run(build, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan + " " + ubsan,
        # the interpreter itself is not instrumented: its own allocations at
        # exit are not this library's leaks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1",
    })
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitizer_driver.py"), lib],
                       capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "SANITIZED OK" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
