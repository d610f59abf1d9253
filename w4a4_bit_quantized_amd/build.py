"""Build libw4a4.so in-tree with hipcc for gfx950.

Usage: ``python -m w4a4_bit_quantized_amd.build`` (or ``build()`` from Python).
The library lands next to this file, where the binding loads it from.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/api.cpp", "csrc/quantize.hip", "csrc/gemm.hip", "csrc/gemm_skinny.hip", "csrc/hadamard.hip",
           "csrc/lowrank_split.cpp"]
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


def build(verbose=False, out=None):
    """Compile every HIP/C++ source into one shared library; returns its path."""
    out = out or os.path.join(HERE, "libw4a4.so")
    tmp = out + ".tmp"
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, out)
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
