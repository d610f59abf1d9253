"""CPU tests of the binding's shape checks: every tensor handed to the C ABI is checked against
the sizes (M, N, K, R) before the call, because the library sees raw pointers and a mis-sized
tensor would be read or written past its end.  The checks take any torch tensor, so CPU tensors
stand in for device ones here."""

import pytest
import torch

from w4a4_bit_quantized_amd import binding as b

M, N, K, R = 6, 40, 64, 8


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _gemm_args(group=16, scale_rows=M):
    return dict(qact=_u8(M, K // 2), ascales=_u8(K // group, scale_rows), lora_act=torch.zeros(M, R),
                qweight=_u8(N, K // 2), wscales=_u8(K // group, N), proj_up=_bf(N, R), wcscales=_bf(N),
                wtscale=_bf(1))


def _layer(group=16):
    return dict(qweight=_u8(N, K // 2), wscales=_u8(K // group, N), proj_down=_bf(K, R), proj_up=_bf(N, R),
                smooth_factor=_bf(K), wcscales=_bf(N), wtscale=_bf(1))


def test_consistent_shapes_pass():
    assert b.check_quantize_act_shapes(_bf(M, K), _bf(K), _bf(K, R)) == (M, K, R)
    assert b.check_gemm_shapes(**_gemm_args(), y=_bf(M, N), bias=_bf(N)) == (M, N, K, R)
    assert b.check_gemm_shapes(**_gemm_args(32, 8), group=32, scale_rows=8) == (M, N, K, R)
    assert b.check_layer_shapes(M, K, dict(_layer(), bias=_bf(N)), y=_bf(M, N)) == (N, R)
    assert b.check_layer_shapes(M, K, _layer(32), group=32) == (N, R)


@pytest.mark.parametrize("name,bad", [("smooth_factor", _bf(K + 16)), ("proj_down", _bf(K - 16, R))])
def test_quantize_act_mismatch(name, bad):
    args = dict(x=_bf(M, K), smooth_factor=_bf(K), proj_down=_bf(K, R))
    args[name] = bad
    with pytest.raises(ValueError, match=name):
        b.check_quantize_act_shapes(**args)


@pytest.mark.parametrize("name,bad", [
    ("ascales", _u8(K // 16, M + 1)), ("ascales", _u8(K // 16 + 1, M)), ("lora_act", torch.zeros(M, R + 1)),
    ("lora_act", torch.zeros(M + 1, R)), ("qweight", _u8(N, K // 2 + 8)), ("wscales", _u8(K // 16, N - 1)),
    ("wcscales", _bf(N + 1)), ("wtscale", _bf(2)), ("proj_up", _bf(N, R, 1)),
])
def test_gemm_mismatch(name, bad):
    args = _gemm_args()
    args[name] = bad
    with pytest.raises(ValueError, match=name):
        b.check_gemm_shapes(**args)


def test_gemm_out_and_bias_mismatch():
    with pytest.raises(ValueError, match="out"):
        b.check_gemm_shapes(**_gemm_args(), y=_bf(M, N - 1))
    with pytest.raises(ValueError, match="bias"):
        b.check_gemm_shapes(**_gemm_args(), bias=_bf(N + 1))


def test_gemm_mx_scale_rows():
    """MX activation scales have M rounded up to 4 rows: an (K/32, M) tensor is refused."""
    with pytest.raises(ValueError, match="ascales"):
        b.check_gemm_shapes(**_gemm_args(32, M), group=32, scale_rows=b.mx_scale_rows(M))


@pytest.mark.parametrize("name,bad", [
    ("wscales", _u8(K // 16, N + 1)), ("proj_down", _bf(K, R + 1)), ("proj_down", _bf(K + 16, R)),
    ("smooth_factor", _bf(K - 16)), ("wcscales", _bf(N - 1)), ("wtscale", _bf(3)), ("qweight", _u8(N, K // 2 - 8)),
    ("bias", _bf(N + 2)),
])
def test_layer_mismatch(name, bad):
    layer = _layer()
    layer[name] = bad
    with pytest.raises(ValueError, match=name):
        b.check_layer_shapes(M, K, layer)


def test_layer_out_mismatch():
    with pytest.raises(ValueError, match="out"):
        b.check_layer_shapes(M, K, _layer(), y=_bf(M + 1, N))


def test_checks_run_before_the_library_call(monkeypatch):
    """A wrapper raises on a mismatch before touching the library (no library call is made)."""
    calls = []

    class Spy:
        def __getattr__(self, name):
            calls.append(name)
            raise AssertionError(f"library called: {name}")

    monkeypatch.setattr(b, "load_library", lambda: Spy())
    monkeypatch.setattr(b, "_dev", lambda t, *a, **k: t)  # CPU tensors pass the device checks
    with pytest.raises(ValueError, match="proj_down"):
        b.svdq_quantize_act(_bf(M, K), _bf(K), _bf(K + 16, R))
    args = _gemm_args()
    args["wscales"] = _u8(K // 16, N + 1)
    with pytest.raises(ValueError, match="wscales"):
        b.svdq_gemm_lowrank(**args)
    layer = _layer()
    layer["proj_up"] = _bf(N, R + 1)
    with pytest.raises(ValueError, match="proj_down"):
        b.svdq_linear(_bf(M, K), layer)
    assert calls == []
