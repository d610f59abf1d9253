"""Pins of the oracle's MXFP4 variant (rotate notes, section 3.3: FP-Quant with
hadamard_group_size 32, forward_dtype mxfp4, forward_method abs_max).

* E8M0 values from the OCP microscaling table, and the doubling invariant.
* The block-scale exponent against a brute-force search over powers of two.
* Exact reproduction of grid values at every scale; reconstruction bound; the
  block maximum lands in the top binade of the E2M1 grid.
* The GEMM against a pure-Python block-scaled triple loop.
"""

import math

import numpy as np
import pytest

from oracle import formats, hadamard, mx, quant


def test_e8m0_table_values():
    # OCP MX v1.0 E8M0: bias 127, 0xFF NaN
    assert mx.e8m0_decode(0x7F) == 1.0
    assert mx.e8m0_decode(0x80) == 2.0
    assert mx.e8m0_decode(0x7E) == 0.5
    assert mx.e8m0_decode(0x00) == 2.0 ** -127
    assert mx.e8m0_decode(0xFE) == 2.0 ** 127
    assert np.isnan(mx.e8m0_decode(0xFF))


def test_e8m0_doubling():
    b = np.arange(0, 254)
    assert np.array_equal(mx.e8m0_decode(b + 1), 2.0 * mx.e8m0_decode(b))


def _brute_exponent(amax):
    q = float(np.float32(np.float32(amax) / np.float32(6.0)))
    if q == 0.0:
        return -127
    for e in range(-127, 128):
        if 2.0 ** e >= q:
            return e
    return 127


def test_scale_exponent_matches_brute_force():
    rng = np.random.default_rng(5)
    vals = [0.0, 6.0, 3.0, 12.0, 1e-40, 6.0 * 2.0 ** -127, 6.0 * 2.0 ** -126, 6.0 * 2.0 ** 100, 3.4e38]
    for k in range(-130, 126, 7):
        base = 6.0 * 2.0 ** k
        vals += [base, np.nextafter(np.float32(base), np.float32(0)), np.nextafter(np.float32(base), np.float32(np.inf))]
    vals += list((rng.uniform(0.5, 1.0, 300) * np.exp2(rng.integers(-140, 120, 300))).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    vals = vals[np.isfinite(vals)]
    got = mx.scale_exponent(vals)
    exp = np.array([_brute_exponent(v) for v in vals])
    assert np.array_equal(got, exp)


def test_grid_values_reproduced_at_every_scale():
    grid = formats.e2m1_decode(np.arange(16))
    for e in range(-120, 121, 3):
        blk = np.zeros((16, 32), np.float32)
        blk[:, 0] = 6.0 * 2.0 ** e  # amax = 6 * 2^e  ->  scale exactly 2^e
        blk[:, 1] = grid * 2.0 ** e
        codes, e8 = mx.group_quantize_mx(blk)
        assert np.all(e8 == e + 127)
        dec = formats.e2m1_decode(codes[:, 1]).astype(np.float64) * 2.0 ** e
        assert np.array_equal(dec, (grid * 2.0 ** e).astype(np.float64))


def test_reconstruction_bound_and_top_binade():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    codes, e8 = mx.group_quantize_mx(v)
    s = np.repeat(mx.e8m0_decode(e8), 32, axis=1)
    t = v.astype(np.float64) / s
    assert np.all(np.abs(t) <= 6.0 * (1 + 2.0 ** -23))  # the scale never clips
    half_step = np.where(np.abs(t) <= 2.0, 0.25, np.where(np.abs(t) <= 4.0, 0.5, 1.0))
    dec = formats.e2m1_decode(codes).astype(np.float64)
    assert np.all(np.abs(dec - t) <= half_step + 1e-12)
    # the block maximum maps into (3, 6]
    g = np.abs(t).reshape(64, 8, 32).max(axis=-1)
    assert np.all((g > 3.0) & (g <= 6.0 * (1 + 2.0 ** -23)))


def test_zero_block_and_sign_of_zero():
    blk = np.zeros((1, 32), np.float32)
    blk[0, 3] = -0.0
    codes, e8 = mx.group_quantize_mx(blk)
    assert e8[0, 0] == 0  # 2^-127
    assert codes[0, 3] == 0x8 and codes[0, 0] == 0


def test_act_layout_padding_and_rotation_group():
    rng = np.random.default_rng(7)
    M, K, R = 6, 128, 8
    x = rng.standard_normal((M, K)).astype(np.float32)
    lam = rng.uniform(0.5, 2, K).astype(np.float32)
    pd = rng.standard_normal((K, R)).astype(np.float32)
    qa, sa, lo = mx.quantize_act_mx(x, lam, pd, 32)
    assert qa.shape == (M, K // 2) and sa.shape == (K // 32, 8) and lo.shape == (M, R)
    assert np.all(sa[:, M:] == 0)
    v = hadamard.fwht_blocks(quant.smooth(x, lam), 32)
    codes, e8 = mx.group_quantize_mx(v)
    assert np.array_equal(qa, quant.pack_nibbles(codes)) and np.array_equal(sa[:, :M], e8.T)
    assert np.allclose(lo, quant.smooth(x, lam).astype(np.float64) @ pd.astype(np.float64))


def _triple_loop(qa, sa, qw, sw, M, N, K):
    ca, cw = quant.unpack_nibbles(qa), quant.unpack_nibbles(qw)
    tab = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    dec = lambda c: (-1.0 if c & 8 else 1.0) * tab[c & 7]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for g in range(K // 32):
                part = sum(dec(int(ca[m, k])) * dec(int(cw[n, k])) for k in range(32 * g, 32 * g + 32))
                tot += part * math.ldexp(1.0, int(sa[g, m]) - 127) * math.ldexp(1.0, int(sw[g, n]) - 127)
            out[m, n] = tot
    return out


@pytest.mark.parametrize("M,K,N,R", [(3, 64, 5, 4), (8, 96, 4, 0)])
def test_gemm_mx_matches_triple_loop(M, K, N, R):
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    lam = np.ones(K, np.float32)
    qa, sa, lo = mx.quantize_act_mx(x, lam, np.zeros((K, R), np.float32), 32)
    qw, sw = mx.quantize_weight_mx(w, lam, 32)
    pu = rng.standard_normal((N, R)).astype(np.float32)
    wcs = rng.uniform(0.9, 1.1, N).astype(np.float32)
    yb, y = mx.gemm_lowrank_mx(qa, sa, lo, qw, sw, pu, wcs, np.float32([1.0]))
    ref = _triple_loop(qa, sa, qw, sw, M, N, K) * wcs[None, :].astype(np.float64)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(yb, formats.bf16_from_f64(ref))
    bias = rng.uniform(-2, 2, N).astype(np.float32)  # the optional per-output offset, unscaled
    yb2, y2 = mx.gemm_lowrank_mx(qa, sa, lo, qw, sw, pu, wcs, np.float32([1.0]), bias)
    assert np.allclose(y2, ref + bias.astype(np.float64)[None, :], rtol=1e-12, atol=1e-12)


def test_identity_of_rotation_in_the_product():
    # with the rotation folded into the weights the unquantized product is unchanged (x R^T (W R^T)^T = x W^T);
    # the MX layer's quantized output stays within the FP4 noise band of it
    rng = np.random.default_rng(9)
    M, K, N = 16, 256, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    lam = np.ones(K, np.float32)
    qw, sw = mx.quantize_weight_mx(w, lam, 32)
    layer = dict(qweight=qw, wscales=sw, proj_down=np.zeros((K, 0), np.float32), proj_up=np.zeros((N, 0), np.float32),
                 smooth_factor=lam, wcscales=np.ones(N, np.float32), wtscale=np.float32([1.0]))
    _, y, _ = mx.svdq_linear_mx(x, layer, 32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.25
