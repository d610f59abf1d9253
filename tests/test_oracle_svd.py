"""Pins of the oracle's offline low-rank split ("SVDQuant W4A4" page, Overview and Checkpoint
contract: a small low-rank branch proj_down (K, R) / proj_up (N, R) beside the 4-bit weight)."""

import numpy as np
import pytest

from oracle import formats, svd


def _planted(N, K, R, noise, seed):
    """bf16 weight with a planted rank-R part (singular values 40 .. 10) plus Gaussian noise."""
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((N, R)))
    v, _ = np.linalg.qr(rng.standard_normal((K, R)))
    s = np.linspace(40.0, 10.0, R)
    w = (u * s) @ v.T / np.sqrt(K) + noise * rng.standard_normal((N, K)) / np.sqrt(K)
    lam = rng.uniform(0.5, 2.0, K)
    return formats.bf16_from_f64(w), formats.bf16_from_f64(lam)


def _f(bits):
    return formats.bf16_to_f32(bits).astype(np.float64)


def test_exact_low_rank_weight_is_reproduced():
    w, lam = _planted(96, 64, 8, 0.0, 1)
    pd, pu, resid, s, low = svd.lowrank_split(_f(w), _f(lam), 8)
    ws = svd.smoothed(_f(w), _f(lam))
    # the weight's own bf16 rounding makes it rank 64 in principle; beyond rank 8 only that remains
    assert s[8] < 1e-2 * s[7]
    assert np.linalg.norm(ws - low) <= 2.0 ** -7 * np.linalg.norm(ws)
    assert np.linalg.norm(_f(resid)) <= 2.0 ** -6 * np.linalg.norm(ws)


def test_eckart_young_identity():
    w, lam = _planted(80, 48, 6, 0.3, 2)
    ws = svd.smoothed(_f(w), _f(lam))
    _, _, _, s, low = svd.lowrank_split(_f(w), _f(lam), 6)
    assert np.isclose(np.linalg.norm(ws - low) ** 2, np.sum(s[6:] ** 2), rtol=1e-9)
    assert np.all(np.diff(s) <= 0)


def test_factors_are_scaled_orthonormal_columns():
    w, lam = _planted(64, 40, 5, 0.2, 3)
    pd, pu, _, s, _ = svd.lowrank_split(_f(w), _f(lam), 5)
    gu = _f(pu).T @ _f(pu)
    gd = _f(pd).T @ _f(pd)
    assert np.allclose(gu, np.diag(s[:5]), rtol=2e-2, atol=2e-2 * s[0])
    assert np.allclose(gd, np.diag(s[:5]), rtol=2e-2, atol=2e-2 * s[0])


def test_residual_is_taken_against_the_stored_factors():
    w, lam = _planted(48, 32, 4, 0.5, 4)
    pd, pu, resid, _, _ = svd.lowrank_split(_f(w), _f(lam), 4)
    ws = svd.smoothed(_f(w), _f(lam))
    stored = _f(pu) @ _f(pd).T
    assert np.array_equal(resid, formats.bf16_from_f64(ws - stored))


def test_rank_zero_keeps_everything_in_the_residual():
    w, lam = _planted(16, 32, 2, 0.5, 5)
    pd, pu, resid, _, _ = svd.lowrank_split(_f(w), _f(lam), 0)
    assert pd.shape == (32, 0) and pu.shape == (16, 0)
    assert np.array_equal(resid, formats.bf16_from_f64(svd.smoothed(_f(w), _f(lam))))


@pytest.mark.parametrize("R", [4, 16])
def test_split_reduces_the_fp4_error(R):
    """The reason for the branch: quantizing the residual instead of the whole weight lowers the
    weight's FP4 reconstruction error on a weight with a dominant low-rank part."""
    from oracle import linear, quant
    w, lam = _planted(64, 128, R, 0.2, 6 + R)
    ws = svd.smoothed(_f(w), _f(lam))
    pd, pu, resid, _, _ = svd.lowrank_split(_f(w), _f(lam), R)
    qw0, s0 = quant.quantize_weight(ws.astype(np.float32), np.ones(128, np.float32))
    err0 = np.linalg.norm(linear.dequant(qw0, s0) - ws)
    qw1, s1 = quant.quantize_weight(_f(resid).astype(np.float32), np.ones(128, np.float32))
    err1 = np.linalg.norm(linear.dequant(qw1, s1) + _f(pu) @ _f(pd).T - ws)
    assert err1 < 0.5 * err0
