"""Build libw4a4.so in-tree with hipcc for gfx950.

Usage: ``python -m w4a4_bit_quantized_amd.build`` (or ``build()`` from Python).
The library lands next to this file, where the binding loads it from.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/api.cpp", "csrc/quantize.hip", "csrc/gemm.hip", "csrc/gemm_skinny.hip", "csrc/hadamard.hip",
           "csrc/lowrank_split.cpp", "csrc/noalloc.hip", "csrc/gemm_mx.hip"]
# Sources whose kernel choice reads the path-forcing test hooks (see csrc/launch.h).
HOOKED = ("csrc/gemm.hip", "csrc/gemm_skinny.hip", "csrc/gemm_mx.hip")
TEST_LIB = "libw4a4_test.so"
ARCH = os.environ.get("W4A4_ARCH", "gfx950")


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",                      # keep every float32 rounding step explicit
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        "-Wall", "-Wno-unused-function",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise))


def build(verbose=False, out=None, test_lib=True, jobs=None):
    """Compile every HIP/C++ source (in parallel, one object each) and link the shared library;
    returns its path.  With test_lib, also link libw4a4_test.so: the same objects, except the
    sources with test hooks, which are compiled a second time with W4A4_TEST_HOOKS (tests use it
    to force kernel variants; nothing else loads it)."""
    out = out or os.path.join(HERE, "libw4a4.so")
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    base = [f for f in flags() if f != "-shared"]
    objs, tobjs, cmds = [], [], []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(obj)
        cmds.append([hipcc()] + base + ["-c", os.path.join(HERE, s), "-o", obj])
        if test_lib and s in HOOKED:
            tobj = os.path.join(objdir, os.path.basename(s) + ".hooks.o")
            tobjs.append(tobj)
            cmds.append([hipcc()] + base + ["-DW4A4_TEST_HOOKS", "-c", os.path.join(HERE, s), "-o", tobj])
        else:
            tobjs.append(obj)
    # the largest translation units first, so that they do not start last
    cmds.sort(key=lambda c: -os.path.getsize(c[-3]))
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"]
    targets = [(out, objs)] + ([(os.path.join(HERE, TEST_LIB), tobjs)] if test_lib else [])
    for path, ob in targets:
        tmp = path + ".tmp"
        _run(link + ob + ["-o", tmp], verbose)
        os.replace(tmp, path)
    return out


def build_probe(verbose=False):
    """Compile the matrix-core throughput probe (a standalone program, not part of the library)."""
    out = os.path.join(HERE, "mfma_peak")
    cmd = [hipcc()] + [f for f in flags() if f not in ("-fPIC", "-shared")] + [
        os.path.join(HERE, "csrc", "mfma_peak.cpp"), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
