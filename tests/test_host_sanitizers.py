"""The library's host code under sanitizers (CPU).

api.cpp (argument validation of every entry point) and lowrank_split.cpp (the threaded offline
split) are compiled with g++ for the host, once with AddressSanitizer + UndefinedBehaviorSanitizer
and once with ThreadSanitizer, linked with host stand-ins for the kernel launchers
(tests/sanitize/launch_stub.cpp: no GPU is involved), and the C-ABI tests, the offline-split tests
and the multi-threaded tests run against each build in a child process with the sanitizer runtime
preloaded.  Any report fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a4_bit_quantized_amd", "csrc")
TESTS = ["tests/test_abi.py", "tests/test_lowrank_split.py", "tests/test_abi_threads.py"]
SANITIZERS = {
    "asan_ubsan": (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"], "libasan.so",
                   {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}),
    # numpy's BLAS threads synchronise outside the instrumented code: keep them to one
    "tsan": (["-fsanitize=thread"], "libtsan.so", {"TSAN_OPTIONS": "halt_on_error=1", "OPENBLAS_NUM_THREADS": "1"}),
}


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.parametrize("kind", sorted(SANITIZERS))
def test_host_code_under_sanitizer(kind, tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    flags, runtime, env_extra = SANITIZERS[kind]
    rt = _runtime(runtime)
    if rt is None:
        pytest.skip(f"{runtime} not available")
    lib = str(tmp_path / f"libw4a4_host_{kind}.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + flags +
           ["-shared", "-fPIC", "-Wl,-Bsymbolic", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "lowrank_split.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"), "-pthread", "-o", lib])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt, W4A4_LIBRARY=lib, **env_extra)
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider"] + TESTS, cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in out
