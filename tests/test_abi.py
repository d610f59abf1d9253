"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments before any launch (no GPU is touched: validation
returns before the first HIP call, and M == 0 / N == 0 calls launch nothing)."""

import ctypes
import os
import re

import pytest

import w4a4_bit_quantized_amd as w4
from w4a4_bit_quantized_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
P = 0x10000  # a fake, well-aligned device address; never dereferenced by the validation paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from w4a4_bit_quantized_amd import build
        build.build()
    return w4.load_library()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "w4a4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"defined"})


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"svdq_quantize_act", "svdq_gemm_lowrank", "svdq_linear", "svdq_quantize_weight",
            "svdq_linear_workspace_bytes", "w4a4_status_string", "w4a4_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/w4a4.h but not exported"
    assert set(binding.SIGNATURES) == set(names)


def test_status_strings(lib):
    for s in range(6):
        assert lib.w4a4_status_string(s)
    assert lib.w4a4_status_string(99) == b"unknown status"
    assert lib.w4a4_version() >= 100


def _qa(lib, x=P, lam=P, pd=P, M=16, K=64, R=32, hb=0, q=P, s=P, lo=P):
    return lib.svdq_quantize_act(x, lam, pd, M, K, R, hb, q, s, lo, None)


def test_quantize_act_validation(lib):
    assert _qa(lib, x=None) == ERR_NULL
    assert _qa(lib, pd=None) == ERR_NULL
    assert _qa(lib, pd=None, lo=None, R=0, M=0) == OK  # R == 0 needs no proj_down; M == 0 launches nothing
    assert _qa(lib, K=24) == ERR_SHAPE
    assert _qa(lib, K=0) == ERR_SHAPE
    assert _qa(lib, M=-1) == ERR_SHAPE
    assert _qa(lib, R=-1) == ERR_SHAPE
    assert _qa(lib, R=65) == ERR_UNSUPPORTED
    assert _qa(lib, K=(1 << 24) + 16) == ERR_UNSUPPORTED
    assert _qa(lib, hb=8) == ERR_UNSUPPORTED
    assert _qa(lib, hb=256) == ERR_UNSUPPORTED
    assert _qa(lib, K=48, hb=32) == ERR_SHAPE
    assert _qa(lib, x=P + 8) == ERR_ALIGN
    assert _qa(lib, lam=P + 2) == ERR_ALIGN
    assert _qa(lib, q=P + 2) == ERR_ALIGN
    assert _qa(lib, M=0) == OK


def test_quantize_weight_validation(lib):
    f = lib.svdq_quantize_weight
    assert f(None, P, 8, 64, 0, P, P, None) == ERR_NULL
    assert f(P, P, 8, 40, 0, P, P, None) == ERR_SHAPE
    assert f(P, P, 8, 64, 12, P, P, None) == ERR_UNSUPPORTED
    assert f(P + 4, P, 8, 64, 0, P, P, None) == ERR_ALIGN
    assert f(P, P, 0, 64, 0, P, P, None) == OK


def _gemm(lib, qa=P, sa=P, lo=P, qw=P, sw=P, pu=P, wc=P, wt=P, M=16, N=32, K=64, R=32, y=P):
    return lib.svdq_gemm_lowrank(qa, sa, lo, qw, sw, pu, wc, wt, M, N, K, R, y, None)


def test_gemm_validation(lib):
    assert _gemm(lib, y=None) == ERR_NULL
    assert _gemm(lib, lo=None) == ERR_NULL
    assert _gemm(lib, lo=None, pu=None, R=0, M=0) == OK
    assert _gemm(lib, K=8) == ERR_SHAPE
    assert _gemm(lib, N=-3) == ERR_SHAPE
    assert _gemm(lib, R=100) == ERR_UNSUPPORTED
    assert _gemm(lib, K=(1 << 24) + 16) == ERR_UNSUPPORTED
    assert _gemm(lib, qa=P + 4) == ERR_ALIGN
    assert _gemm(lib, qw=P + 8) == ERR_ALIGN
    assert _gemm(lib, y=P + 1) == ERR_ALIGN
    assert _gemm(lib, N=0) == OK


def test_workspace_size(lib):
    f = lib.svdq_linear_workspace_bytes
    a256 = lambda v: (v + 255) // 256 * 256
    assert f(4096, 3072, 32) == a256(4096 * 1536) + a256(192 * 4096) + a256(4096 * 32 * 4)
    assert f(1, 16, 0) == 256 + 256
    assert f(-1, 64, 0) == 0 and f(4, 40, 0) == 0 and f(4, 64, 65) == 0


def _lin(lib, x=P, qw=P, sw=P, pd=P, pu=P, lam=P, wc=P, wt=P, M=16, N=32, K=64, R=32, hb=0, y=P, ws=P, wsb=None):
    if wsb is None:
        wsb = lib.svdq_linear_workspace_bytes(max(M, 0), K, max(R, 0))
    return lib.svdq_linear(x, qw, sw, pd, pu, lam, wc, wt, M, N, K, R, hb, y, ws, wsb, None)


def test_linear_validation(lib):
    assert _lin(lib, x=None) == ERR_NULL
    assert _lin(lib, ws=None) == ERR_NULL
    assert _lin(lib, wsb=100) == ERR_SHAPE
    assert _lin(lib, ws=P + 16) == ERR_ALIGN
    assert _lin(lib, hb=24) == ERR_UNSUPPORTED
    assert _lin(lib, K=48, hb=32) == ERR_SHAPE
    assert _lin(lib, M=0) == OK
    assert _lin(lib, N=0, ws=None) == OK


def test_binding_signatures_match_header(lib):
    for name, (res, args) in binding.SIGNATURES.items():
        fn = getattr(lib, name)
        assert fn.argtypes == args and fn.restype == res
    assert ctypes.sizeof(ctypes.c_size_t) == 8


# ---- MXFP4 entry points -----------------------------------------------------------------------

def test_mx_validation(lib):
    qa = lambda **k: lib.svdq_quantize_act_mx(k.get("x", P), P, P, k.get("M", 16), k.get("K", 128), k.get("R", 32),
                                               k.get("hb", 32), P, P, P, None)
    assert qa(K=48) == ERR_SHAPE           # K % 32
    assert qa(hb=16) == ERR_UNSUPPORTED    # rotation in blocks of 32 or none
    assert qa(hb=128) == ERR_UNSUPPORTED
    assert qa(x=None) == ERR_NULL
    assert qa(M=0, x=None) == OK
    qw = lambda **k: lib.svdq_quantize_weight_mx(P, P, k.get("N", 8), k.get("K", 64), k.get("hb", 0), P, P, None)
    assert qw(K=80) == ERR_SHAPE and qw(hb=64) == ERR_UNSUPPORTED and qw(N=0) == OK
    g = lambda **k: lib.svdq_gemm_lowrank_mx(P, k.get("sa", P), P, P, k.get("sw", P), P, P, P, k.get("M", 16),
                                              k.get("N", 64), k.get("K", 256), k.get("R", 32), P, None)
    assert g(K=96) == ERR_SHAPE            # whole 128-column K-steps
    assert g(N=66) == ERR_SHAPE            # N % 4
    assert g(sa=P + 2) == ERR_ALIGN and g(sw=P + 1) == ERR_ALIGN
    assert g(M=0) == OK
    assert lib.svdq_linear_mx_workspace_bytes(6, 256, 32) == 768 + 256 + 768  # codes, scales (8 x 8 rows), lora
    assert lib.svdq_linear_mx_workspace_bytes(6, 48, 32) == 0


# ---- standalone block Hadamard transform --------------------------------------------------------

def test_hadamard_validation(lib):
    def h(x=P, ldx=64, y=P + 0x1000, ldy=64, rows=4, cols=64, block=16, dtype=0):
        return lib.w4a4_hadamard_transform(x, ldx, y, ldy, rows, cols, block, dtype, None)
    assert h(block=3) == ERR_UNSUPPORTED and h(block=1) == ERR_UNSUPPORTED
    assert h(block=8192, cols=8192, ldx=8192, ldy=8192) == ERR_UNSUPPORTED  # above W4A4_HADAMARD_MAX_BLOCK
    assert h(dtype=3) == ERR_UNSUPPORTED and h(dtype=-1) == ERR_UNSUPPORTED
    assert h(cols=72) == ERR_SHAPE                 # cols % block
    assert h(ldx=32) == ERR_SHAPE and h(ldy=48) == ERR_SHAPE
    assert h(rows=-1) == ERR_SHAPE and h(cols=-16) == ERR_SHAPE
    assert h(y=P, ldy=128) == ERR_SHAPE            # in place needs equal row strides
    assert h(rows=0, x=None, y=None) == OK and h(cols=0, x=None, y=None) == OK
    assert h(x=None) == ERR_NULL and h(y=None) == ERR_NULL
    assert h(x=P + 1) == ERR_ALIGN                 # bf16 needs 2-byte alignment
    assert h(y=P + 2, dtype=2) == ERR_ALIGN        # f32 needs 4-byte alignment
    assert binding.HADAMARD_MAX_BLOCK == 4096


def test_bias_validation(lib):
    g = lambda b, **k: lib.svdq_gemm_lowrank_bias(P, P, P, P, P, P, P, P, b, k.get("M", 16), 64, 256, 32, P, None)
    assert g(P + 1) == ERR_ALIGN          # bf16 bias needs 2-byte alignment
    assert g(None, M=0) == OK and g(P + 1, M=0) == OK  # nothing to do: no pointer is looked at
    gm = lambda b: lib.svdq_gemm_lowrank_mx_bias(P, P, P, P, P, P, P, P, b, 16, 64, 256, 32, P, None)
    assert gm(P + 1) == ERR_ALIGN
    lin = lambda b, ws=P: lib.svdq_linear_bias(P, P, P, P, P, P, P, P, b, 16, 64, 256, 32, 0, P, ws, 1 << 20, None)
    assert lin(P + 3) == ERR_ALIGN
    assert lin(P, ws=None) == ERR_NULL
    linm = lambda b: lib.svdq_linear_mx_bias(P, P, P, P, P, P, P, P, b, 16, 64, 256, 32, 32, P, P, 1 << 20, None)
    assert linm(P + 1) == ERR_ALIGN


def test_linear_noalloc_validation(lib):
    """The entry point without allocation: svdq_linear's checks and statuses, then the limit of its
    static buffer (W4A4_ERR_SCRATCH), all before any HIP call."""
    f = lib.svdq_linear_noalloc

    def call(x=P, M=16, N=16, K=64, R=8, hb=0, y=P, bias=None):
        return f(x, P, P, P, P, P, P, P, bias, M, N, K, R, hb, y, None)

    assert call(K=40) == ERR_SHAPE
    assert call(R=65) == ERR_UNSUPPORTED
    assert call(hb=8) == ERR_UNSUPPORTED
    assert call(x=None) == ERR_NULL
    assert call(y=None) == ERR_NULL
    assert call(x=P + 8) == ERR_ALIGN
    assert call(bias=P + 1) == ERR_ALIGN
    assert call(M=0) == OK and call(N=0) == OK
    # 64 MiB holds M * K / 2 + M * K / 16 + 4 M R bytes (each part 256-byte aligned)
    assert call(M=4096, K=12288, R=32) != 6          # 28.9 MB: fits
    assert call(M=8192, K=16384, R=32) == 6          # 77 MB: refused
    assert call(M=8192, K=16384, R=32, x=None) == ERR_NULL  # other errors are reported first
    assert lib.w4a4_status_string(6)
