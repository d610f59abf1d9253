"""Pins of the oracle's quantizers.

* Rotate notes, section 1: the signed/unsigned INT4 absmax worked examples,
  with and without the Hadamard rotation (values in tests/golden).
* "SVDQuant W4A4" page, "Checkpoint contract": FP4 pairs per byte, one e4m3
  scale per 16 along K, scale tensors laid out (K/16, rows).
* Reconstruction bound, exact reproduction of grid values and special cases of
  the per-16 group quantizer.
"""

import math

import numpy as np
import pytest

from oracle import formats, hadamard, quant


# ---- INT4 worked examples (rotate notes, section 1) -------------------------------------------

def test_unsigned_background_example(golden):
    ex = golden["unsigned_background"]
    q, scale, xh = quant.int4_absmax(ex["x"], signed=False)
    assert scale == pytest.approx(100.0 / 15.0)
    assert q.tolist() == ex["q"]
    assert np.allclose(xh, ex["x_hat"])


def test_extreme_outlier_example(golden):
    ex = golden["extreme_outlier"]
    q, scale, xh = quant.int4_absmax(ex["x"])
    assert q.tolist() == ex["no_rotation_q"]
    assert np.allclose(xh, ex["no_rotation_x_hat"])
    assert np.mean((np.float64(ex["x"]) - xh) ** 2) == pytest.approx(ex["no_rotation_mse"], abs=1e-3)
    xr = hadamard.fwht_blocks(np.float32(ex["x"]), 4).astype(np.float64)
    qr, sr, xrh = quant.int4_absmax(xr)
    assert qr.tolist() == ex["rotated_q"]
    # inverse rotation (H = H^T = H^-1 once normalised): recovery [0, 0, 0, 81]
    rec = hadamard.fwht_blocks(np.float32(xrh), 4).astype(np.float64)
    assert np.allclose(rec, ex["rotated_recovery"], atol=1e-4)


def test_realistic_example(golden):
    ex = golden["realistic"]
    x = np.float64(ex["x"])
    q, scale, xh = quant.int4_absmax(x)
    assert q.tolist() == ex["no_rotation_q"]
    assert np.allclose(xh, ex["no_rotation_x_hat"], atol=1e-3)
    mse0 = np.mean((x - xh) ** 2)
    assert mse0 == pytest.approx(ex["no_rotation_mse"], abs=1e-3)
    assert np.max(np.abs(x - xh)) == pytest.approx(ex["no_rotation_max_abs_err"], abs=1e-3)
    xr = hadamard.fwht_blocks(np.float32(x), 4).astype(np.float64)
    qr, sr, xrh = quant.int4_absmax(xr)
    assert qr.tolist() == ex["rotated_q"]
    assert np.allclose(xrh, ex["rotated_dequant"], atol=1e-3)
    rec = hadamard.fwht_blocks(np.float32(xrh), 4).astype(np.float64)
    assert np.allclose(rec, ex["rotated_recovery"], atol=1e-3)
    mse1 = np.mean((x - rec) ** 2)
    assert mse1 == pytest.approx(ex["rotated_mse"], abs=1e-3)
    assert np.max(np.abs(x - rec)) == pytest.approx(ex["rotated_max_abs_err"], abs=1e-3)
    # the page derives "-69%" from its 3-decimal MSEs (1 - 0.073/0.237 = 69.2%);
    # the exact ratio is 69.6%, so the printed figure is the truncated percentage
    assert math.floor(100 * (1 - mse1 / mse0)) == ex["mse_reduction_percent"]
    assert math.floor(100 * (1 - ex["rotated_mse"] / ex["no_rotation_mse"])) == ex["mse_reduction_percent"]
    assert np.ptp(x) == pytest.approx(ex["range_no_rotation"], abs=1e-6)
    assert np.ptp(xr) == pytest.approx(ex["range_rotated"], abs=1e-5)


# ---- per-16 group FP4 quantizer ----------------------------------------------------------------

def test_grid_values_reproduced_exactly_for_every_scale():
    grid = np.float32([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6, 6])  # 16 = one group
    codes_all = formats.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    rows = (grid[None, :] * codes_all[:, None]).astype(np.float32)  # max |v| = 6 * sd  ->  scale = sd
    codes, s8 = quant.group_quantize(rows)
    assert np.array_equal(s8[:, 0], np.arange(1, 0x7F, dtype=np.uint8))
    back = formats.e2m1_decode(codes) * codes_all[:, None]
    assert np.array_equal(back, rows)


def test_reconstruction_bound():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((400, 64)) * np.exp2(rng.integers(-12, 8, (400, 1)))).astype(np.float32)
    codes, s8 = quant.group_quantize(v)
    sd = np.repeat(formats.e4m3_decode(s8), 16, axis=1).astype(np.float64)
    q = formats.e2m1_decode(codes).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = v.astype(np.float64) / sd
    unsat = np.abs(t) <= 6.0
    step = np.where(np.abs(q) < 2, 0.5, np.where(np.abs(q) < 4, 1.0, 2.0))
    step = np.where((np.abs(q) == 2) & (np.abs(t) < 2), 0.5, step)
    step = np.where((np.abs(q) == 4) & (np.abs(t) < 4), 1.0, step)
    err = np.abs(t - q)
    assert np.all(err[unsat] <= step[unsat] / 2 + 1e-6)
    # the stored scale is the e4m3 rounding of amax/6
    amax = np.abs(v.reshape(400, 4, 16)).max(-1)
    assert np.array_equal(s8, formats.e4m3_encode(amax / np.float32(6)))


def test_zero_and_tiny_groups():
    v = np.zeros((3, 32), np.float32)
    v[1, :16] = 2.0 ** -14  # amax/6 < 2^-10: rounds to scale 0
    v[2, :16] = np.float32(6 * 2.0 ** -10)  # amax/6 == 2^-10: tie between 0 and 2^-9 -> even (0)
    v[2, 16:] = -0.0
    codes, s8 = quant.group_quantize(v)
    assert s8.tolist() == [[0, 0], [0, 0], [0, 0]]
    assert not codes.any()


def test_saturation_of_large_groups():
    v = np.full((1, 16), 1e6, np.float32)
    v[0, 1] = -1e6
    codes, s8 = quant.group_quantize(v)
    assert s8.tolist() == [[0x7E]]
    assert codes[0, 0] == 7 and codes[0, 1] == 15


def test_pack_layout_even_k_low_nibble():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    packed = quant.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(quant.unpack_nibbles(packed), codes)


# ---- activation and weight quantizers ---------------------------------------------------------

def _layer(M=8, K=64, N=5, R=4, seed=0):
    rng = np.random.default_rng(seed)
    bf = lambda a: ((np.asarray(a, np.float32).view(np.uint32) + 0x8000) & 0xFFFF0000).view(np.float32)
    x = bf(rng.standard_normal((M, K)))
    lam = bf(rng.uniform(0.5, 2.0, K))
    pd = bf(rng.standard_normal((K, R)) / np.sqrt(K))
    w = bf(rng.standard_normal((N, K)) / np.sqrt(K))
    return x, lam, pd, w


def test_quantize_act_shapes_and_layout():
    x, lam, pd, _ = _layer(M=8, K=64, R=4)
    qact, ascales, lora = quant.quantize_act(x, lam, pd)
    assert qact.shape == (8, 32) and qact.dtype == np.uint8
    assert ascales.shape == (4, 8) and ascales.dtype == np.uint8
    assert lora.shape == (8, 4)
    # row m, group g of the activation is quantized on its own
    xs = (x / lam).astype(np.float32)
    for m in (0, 5):
        for g in range(4):
            c, s = quant.group_quantize(xs[m:m + 1, 16 * g:16 * g + 16])
            assert ascales[g, m] == s[0, 0]
            assert np.array_equal(quant.unpack_nibbles(qact[m:m + 1, 8 * g:8 * g + 8]), c)


def test_quantize_act_smoothing_divides():
    x = np.ones((1, 16), np.float32)
    lam = np.full(16, 2.0, np.float32)
    qact, ascales, lora = quant.quantize_act(x, lam, np.ones((16, 1), np.float32))
    assert formats.e4m3_decode(ascales)[0, 0] == pytest.approx(0.5 / 6, rel=0.07)
    assert lora[0, 0] == pytest.approx(8.0)  # sum of 16 values of 1/2


def test_quantize_act_lora_uses_unrotated_input():
    x, lam, pd, _ = _layer(M=4, K=128, R=3, seed=5)
    _, _, l0 = quant.quantize_act(x, lam, pd, 0)
    _, _, l1 = quant.quantize_act(x, lam, pd, 64)
    assert np.array_equal(l0, l1)
    assert np.allclose(l0, (x.astype(np.float64) / lam) @ pd, rtol=1e-6)


def test_quantize_act_rotation_quantizes_rotated_values():
    x, lam, pd, _ = _layer(M=4, K=128, R=0, seed=6)
    qact, ascales, _ = quant.quantize_act(x, lam, pd[:, :0], 32)
    v = hadamard.fwht_blocks((x / lam).astype(np.float32), 32)
    c, s = quant.group_quantize(v)
    assert np.array_equal(qact, quant.pack_nibbles(c))
    assert np.array_equal(ascales, s.T)


def test_quantize_weight_folds_smoothing_and_rotation():
    _, lam, _, w = _layer(N=6, K=64, seed=8)
    qw, ws = quant.quantize_weight(w, lam, 16)
    assert qw.shape == (6, 32) and ws.shape == (4, 6)
    wq = hadamard.fwht_blocks((w * lam).astype(np.float32), 16)
    c, s = quant.group_quantize(wq)
    assert np.array_equal(qw, quant.pack_nibbles(c)) and np.array_equal(ws, s.T)
