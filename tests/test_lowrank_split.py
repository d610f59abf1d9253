"""The library's offline low-rank split (host code, randomized range finder) against the
oracle's exact SVD ("SVDQuant W4A4" page, Overview and Checkpoint contract).

Singular vectors are unique only up to sign, so the comparison is on what is unique: the
singular values, the rank-R product of the stored factors, and the residual it leaves.  The
weights have a planted, well-separated rank-R part (the randomized method converges to the
exact top-R subspace there).  Host code only: these tests need no GPU.
"""

import numpy as np
import pytest

import w4a4_bit_quantized_amd as w4
from w4a4_bit_quantized_amd import binding
from oracle import formats, svd


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(binding.library_path()):
        from w4a4_bit_quantized_amd import build
        build.build()
    return w4.load_library()


def _planted(N, K, R, noise, seed):
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((N, R)))
    v, _ = np.linalg.qr(rng.standard_normal((K, R)))
    s = np.linspace(40.0, 10.0, R)
    w = (u * s) @ v.T / np.sqrt(K) + noise * rng.standard_normal((N, K)) / np.sqrt(K)
    return formats.bf16_from_f64(w), formats.bf16_from_f64(rng.uniform(0.5, 2.0, K))


def _f(bits):
    return formats.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("N,K,R,noise", [(96, 64, 8, 0.1), (200, 160, 32, 0.2), (64, 256, 16, 0.05), (33, 47, 5, 0.1)])
def test_split_matches_exact_svd(lib, N, K, R, noise):
    w, lam = _planted(N, K, R, noise, N + K)
    pd, pu, resid, sv = w4.svdq_lowrank_split(w, lam, R, oversample=10, power_iters=4, seed=1)
    pd_r, pu_r, resid_r, s_r, low_r = svd.lowrank_split(_f(w), _f(lam), R)
    assert np.allclose(sv.astype(np.float64), s_r[:R], rtol=1e-5)
    prod = _f(pu) @ _f(pd).T
    prod_r = _f(pu_r) @ _f(pd_r).T
    ws = svd.smoothed(_f(w), _f(lam))
    # both products round the same exact factors to bf16: they agree to bf16 level
    assert np.linalg.norm(prod - prod_r) <= 2.0 ** -6 * np.linalg.norm(low_r)
    assert np.linalg.norm(prod - low_r) <= 2.0 ** -6 * np.linalg.norm(low_r)
    # the residual is taken against the library's own stored factors, rounded once
    assert np.array_equal(resid, formats.bf16_from_f64(ws - prod))
    assert np.linalg.norm(_f(resid) - _f(resid_r)) <= 2.0 ** -5 * np.linalg.norm(_f(resid_r)) + 2.0 ** -6 * np.linalg.norm(low_r)


def test_deterministic_for_a_seed_and_thread_count_independent(lib):
    w, lam = _planted(80, 72, 6, 0.1, 9)
    a = w4.svdq_lowrank_split(w, lam, 6, seed=3, threads=1)
    b = w4.svdq_lowrank_split(w, lam, 6, seed=3, threads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rank_zero_and_errors(lib):
    w, lam = _planted(16, 24, 2, 0.3, 4)
    pd, pu, resid, sv = w4.svdq_lowrank_split(w, lam, 0)
    assert pd.shape == (24, 0) and pu.shape == (16, 0) and sv.shape == (0,)
    assert np.array_equal(resid, formats.bf16_from_f64(svd.smoothed(_f(w), _f(lam))))
    with pytest.raises(w4.W4A4Error):
        w4.svdq_lowrank_split(w, lam, 17)   # R > min(N, K)
    with pytest.raises(w4.W4A4Error):
        w4.svdq_lowrank_split(w, lam, 2, oversample=-1)
    P = 0x10000
    assert lib.svdq_lowrank_split(None, P, 4, 4, 1, 0, 0, 0, 1, P, P, P, None) == 1  # ERR_NULL
    assert lib.svdq_lowrank_split(P, P, 4, 4, 1, 0, 0, 0, 1, None, P, P, None) == 1
    assert lib.svdq_lowrank_split(P, P, 0, 4, 1, 0, 0, 0, 1, P, P, P, None) == 2  # ERR_SHAPE
    assert lib.svdq_lowrank_split(P, P, 200, 100, 65, 0, 0, 0, 1, P, P, P, None) == 2  # R > W4A4_MAX_RANK
