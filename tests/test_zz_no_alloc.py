"""svdq_linear_noalloc (the layer with the library's static device workspace) against svdq_linear
with a caller-provided workspace: bit-identical outputs, on two calls in a row with the second
one smaller (the buffer keeps the first call's contents), through the C ABI (needs an MI355X)."""

import numpy as np
import pytest

import helpers as H
from w4a4_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import w4a4_bit_quantized_amd as w
    w.load_library()
    return w


def _case(M, K, N, R, B, seed, bias):
    lay = synth.make_layer("tiny", seed=seed, M=M, K=K, N=N, R=R, B=B, wcs="uniform")
    qw, ws = H.oracle_weights(lay)
    layer = H.device_layer(lay, qw, ws)
    if bias:
        layer["bias"] = H.to_dev_bf16(H.seeded_bias(N, M))
    return H.to_dev_bf16(lay["x"]), layer


@pytest.mark.parametrize("first,second", [
    ((600, 1024, 520, 32, 64, True), (37, 256, 260, 16, 16, False)),   # tiled GEMM, then a smaller tiled call
    ((2048, 3072, 1024, 32, 0, False), (16, 2048, 8200, 32, 0, True)),  # large, then the skinny path (K split)
])
def test_noalloc_matches_workspace_entry_point(w4, first, second):
    import torch
    for M, K, N, R, B, bias in (first, second):
        print(f"\nnoalloc case M={M} K={K} N={N} R={R} B={B} bias={bias}", flush=True)
        x, layer = _case(M, K, N, R, B, seed=M + K, bias=bias)
        ref = w4.svdq_linear(x, layer, hadamard_block=B)
        y = w4.svdq_linear_noalloc(x, layer, hadamard_block=B)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"differs at M={M} K={K} N={N}"


def test_noalloc_refuses_sizes_beyond_its_buffer(w4):
    import torch
    from w4a4_bit_quantized_amd import binding
    lay = synth.make_layer("tiny", seed=3, M=4, K=64, N=8, R=4)
    qw, ws = H.oracle_weights(lay)
    layer = H.device_layer(lay, qw, ws)
    # 8192 x 16384 needs 77 MB of workspace: refused before any launch (no device memory is read)
    lib = w4.load_library()
    P = layer["qweight"].data_ptr()
    st = lib.svdq_linear_noalloc(P, P, P, P, P, P, P, P, None, 8192, 64, 16384, 32, 0, P, None)
    assert st == 6, binding.STATUS_NAMES.get(st)
    torch.cuda.synchronize()
