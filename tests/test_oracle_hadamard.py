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


# ---- the standalone transform (rotate notes, section 3.1: Hadacore, in place, head_dim blocks,
# output partitions) -------------------------------------------------------------------------


def _stored(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32) * 3
    return hadamard.from_f32(x, dtype)


@pytest.mark.parametrize("dtype", hadamard.DTYPES)
@pytest.mark.parametrize("n", [2, 8, 64, 512, 2048])
def test_standalone_equals_rounded_dense_product(dtype, n):
    """The transform equals the float64 dense product rounded once to the storage type, except
    where the float32 butterflies land within a few float32 ulps of a rounding boundary."""
    rng = np.random.default_rng(n)
    x = _stored(rng, (3, 2 * n), dtype)
    got = hadamard.to_f32(hadamard.hadamard_transform(x, n, dtype), dtype).astype(np.float64)
    h = _sylvester_dense(n) / np.sqrt(n)
    exact = (hadamard.to_f32(x, dtype).astype(np.float64).reshape(3, 2, n) @ h.T).reshape(3, 2 * n)
    ref = hadamard.to_f32(hadamard.from_f32(exact.astype(np.float32), dtype), dtype).astype(np.float64)
    ulp = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -23}[dtype]
    # float32 butterflies differ from the exact product by about log2(n) float32 ulps of the
    # block's magnitude; one storage ulp covers the final rounding
    scale = np.abs(hadamard.to_f32(x, dtype)).reshape(3, 2, n).max(axis=2).repeat(n, axis=1)
    tol = ulp * np.abs(exact) + (np.log2(n) + 2) * 2.0 ** -23 * np.sqrt(n) * scale
    assert np.all(np.abs(got - exact) <= tol + 1e-30)
    if dtype != "f32":  # the storage rounding hides the butterflies' float32 error except near boundaries
        assert np.mean(got == ref) > 0.95


@pytest.mark.parametrize("dtype,n", [("bf16", 4), ("bf16", 16), ("bf16", 64), ("f16", 16), ("f16", 256),
                                     ("f16", 1024), ("f32", 64), ("f32", 1024), ("f32", 4096)])
def test_standalone_involution_exact_for_powers_of_four(dtype, n):
    """Sizes 4^k: 1/sqrt(n) is a power of two, and inputs in {-1, 0, 1} stay exact through both
    passes while the storage type holds every integer up to n (bf16: n <= 256, f16: n <= 2048)."""
    rng = np.random.default_rng(3)
    xi = rng.integers(-1, 2, size=(2, n)).astype(np.float32)
    x = hadamard.from_f32(xi, dtype)
    twice = hadamard.hadamard_transform(hadamard.hadamard_transform(x, n, dtype), n, dtype)
    assert np.array_equal(hadamard.to_f32(twice, dtype), xi)


def test_standalone_partition_leaves_other_columns():
    """An output partition [start, start + length) is transformed; everything else is copied."""
    rng = np.random.default_rng(5)
    x = _stored(rng, (4, 96), "bf16")
    y = hadamard.hadamard_transform(x, 16, "bf16", start=32, length=48)
    assert np.array_equal(y[:, :32], x[:, :32]) and np.array_equal(y[:, 80:], x[:, 80:])
    part = hadamard.hadamard_transform(x[:, 32:80], 16, "bf16")
    assert np.array_equal(y[:, 32:80], part)


def test_standalone_head_dim_blocks_equal_separate_rows():
    """Blocking by head_dim is the transform of each head's slice on its own."""
    rng = np.random.default_rng(6)
    x = _stored(rng, (3, 4 * 64), "f16")
    y = hadamard.hadamard_transform(x, 64, "f16")
    for h in range(4):
        assert np.array_equal(y[:, 64 * h:64 * h + 64], hadamard.hadamard_transform(x[:, 64 * h:64 * h + 64], 64, "f16"))


def test_storage_rounding_matches_torch():
    """bf16 and f16 rounding of the float32 result agree with torch's CPU conversions."""
    import torch
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))).astype(np.float32)
    b = hadamard.from_f32(v, "bf16")
    tb = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, tb)
    h = hadamard.from_f32(v, "f16")
    th = torch.from_numpy(v).to(torch.float16).numpy()
    assert np.array_equal(h.view(np.uint16), th.view(np.uint16))
