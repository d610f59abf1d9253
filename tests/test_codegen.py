"""Code-generation checks of the GEMM kernels (CPU: compiles gemm.hip to gfx950 assembly).

The persistent kernels rely on every wave issuing exactly ST = FM * FN * 2 buffer stores per tile,
and ST dropped placeholder stores before the first tile, so that each tile's first vmcnt waits
count the stores in flight behind the K-steps they wait for.  If the compiler merged or removed
any of them (it once merged identical placeholder stores into one), the waits would be too loose
and a K-step could be read before it landed; this counts the store instructions in the compiled
code of every persistent kernel instantiation.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    import sys
    sys.path.insert(0, os.path.join(ROOT, "w4a4_bit_quantized_amd"))
    import build
    flags = [f for f in build.flags() if f not in ("-fPIC", "-shared")]
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [hipcc] + flags + ["--cuda-device-only", "-S", os.path.join(ROOT, "w4a4_bit_quantized_amd", "csrc", "gemm.hip"),
                             "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read().split("\n")


def _kernels(lines, pattern):
    """(name, body lines) of every kernel whose symbol matches pattern."""
    out = []
    for i, line in enumerate(lines):
        m = re.match(r"(_Z\S*" + pattern + r"\S*):", line)
        if m:
            j = i
            while not lines[j].startswith(".Lfunc_end"):
                j += 1
            out.append((m.group(1), lines[i:j]))
    return out


def test_persistent_kernels_issue_exactly_st_stores_per_tile(gemm_asm):
    ks = _kernels(gemm_asm, r"_persist_kernel")
    assert len(ks) >= 10, f"expected the persistent kernel instantiations, found {len(ks)}"
    for name, body in ks:
        fm, fn = map(int, re.search(r"ILi\d+ELi\d+ELi(\d+)ELi(\d+)ELb", name).groups())
        st = fm * fn * 2
        n = sum(1 for line in body if "buffer_store_dwordx4" in line)
        assert n == 2 * st, f"{name}: {n} buffer stores, expected {st} placeholders + {st} per tile"
        # (other vector-memory operations, such as register spills, issued after the prefetched
        # K-steps only make those waits stricter: completion is in issue order)
