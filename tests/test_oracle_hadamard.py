"""Pins of the oracle's block Sylvester Hadamard transform.

Source: rotate notes, section 1 (worked examples with the normalised H_4),
section 2.2 (Sylvester recursion, H H^T = n I, H = H^T) and section 3.1 (the
transform equals the dense product and is its own inverse).
"""

import numpy as np
import pytest

from oracle import hadamard


def _sylvester_dense(n):
    """Unnormalised Sylvester matrix built by the block recursion H_2n = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_worked_example_realistic(golden):
    ex = golden["realistic"]
    got = hadamard.fwht_blocks(np.float32(ex["x"]), 4)
    assert np.allclose(got, ex["rotated"], atol=1e-5)


def test_worked_example_extreme_outlier(golden):
    ex = golden["extreme_outlier"]
    got = hadamard.fwht_blocks(np.float32(ex["x"]), 4).astype(np.float64)
    # The page prints [40.50, -39.90, -39.70, 39.90]; its own arithmetic gives
    # [40.5, -40.0, -39.7, 39.8].  Entries 0 and 2 agree with the page.
    assert got[0] == pytest.approx(40.5, abs=1e-4)
    assert got[2] == pytest.approx(-39.7, abs=1e-4)
    assert np.allclose(got, [40.5, -40.0, -39.7, 39.8], atol=1e-4)


def test_h4_matches_page(golden):
    h = np.stack([hadamard.fwht_blocks(row, 4) for row in np.eye(4, dtype=np.float32)])
    assert np.array_equal(h, np.float32(golden["hadamard_4"]["H4"]))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128])
def test_equals_dense_sylvester_product(n):
    rng = np.random.default_rng(n)
    x = rng.integers(-8, 9, size=(5, 3 * n)).astype(np.float32)  # small integers: stages are exact
    got = hadamard.fwht_blocks(x, n).astype(np.float64)
    h = _sylvester_dense(n) / np.sqrt(n)
    ref = (x.astype(np.float64).reshape(5, 3, n) @ h.T).reshape(5, 3 * n)
    assert np.allclose(got, ref, rtol=2e-7, atol=1e-6)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128])
def test_orthogonal_and_symmetric(n):
    h = np.stack([hadamard.fwht_blocks(r, n) for r in np.eye(n, dtype=np.float32)]).astype(np.float64)
    assert np.allclose(h @ h.T, np.eye(n), atol=1e-6)
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("n", [4, 16, 64, 128])
def test_involution_and_roundtrip(n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 2 * n)).astype(np.float32)
    y = hadamard.fwht_blocks(x, n)
    back = hadamard.fwht_blocks(y, n)
    assert np.allclose(back, x, rtol=1e-5, atol=1e-6)
    if n in (4, 16, 64):  # power of 4: 1/sqrt(n) is exact, integer inputs round-trip exactly
        xi = rng.integers(-50, 50, size=(3, n)).astype(np.float32)
        assert np.array_equal(hadamard.fwht_blocks(hadamard.fwht_blocks(xi, n), n), xi)


def test_normalisation_constant_128():
    assert hadamard.norm_const(128).view(np.uint32) == np.uint32(0x3DB504F3)


def test_blocks_are_independent():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 256)).astype(np.float32)
    full = hadamard.fwht_blocks(x, 128)
    assert np.array_equal(full[:, :128], hadamard.fwht_blocks(x[:, :128], 128))
    assert np.array_equal(full[:, 128:], hadamard.fwht_blocks(x[:, 128:], 128))


def test_rejects_bad_blocks():
    with pytest.raises(ValueError):
        hadamard.fwht_blocks(np.zeros((1, 48), np.float32), 32)
    with pytest.raises(ValueError):
        hadamard.fwht_blocks(np.zeros((1, 48), np.float32), 24)
