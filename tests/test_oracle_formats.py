"""Pins of the oracle's number formats (E2M1, float8_e4m3fn, bf16).

E2M1 and e4m3 are the formats the "SVDQuant W4A4" page names for the
checkpoint (section "Checkpoint contract", precision nvfp4).  The e4m3 codec is
checked against torch's CPU float8_e4m3fn conversion (a library routine); the
E2M1 encoder, for which no library conversion exists here, against a
brute-force nearest-value search in float64 with the tie rule written out.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_e2m1(v):
    """Nearest E2M1 magnitude by exhaustive search; ties to the code with mantissa bit 0."""
    out = []
    for x in np.asarray(v, dtype=np.float32).tolist():
        a = abs(x)
        sign = 8 if np.signbit(np.float32(x)) else 0
        if a == float("inf"):
            out.append(sign | 7)
            continue
        dists = [abs(Fraction(a) - Fraction(g)) for g in GRID]
        best = min(dists)
        cands = [c for c, d in enumerate(dists) if d == best]
        if len(cands) == 2:
            c = cands[0] if cands[0] % 2 == 0 else cands[1]
        else:
            c = cands[0]
        out.append(sign | c)
    return np.array(out, dtype=np.uint8)


def _near(values, n_ulps):
    """float32 values within +-n_ulps of each given float32 value."""
    base = np.asarray(values, dtype=np.float32).view(np.int32).astype(np.int64)
    offs = np.arange(-n_ulps, n_ulps + 1, dtype=np.int64)
    u = (base[:, None] + offs[None, :]).reshape(-1)
    u = u[(u >= 0) & (u < 0x7F800000)]
    return u.astype(np.int32).view(np.float32)


def test_e2m1_decode_table():
    vals = formats.e2m1_decode(np.arange(16))
    assert vals[:8].tolist() == GRID
    assert vals[8:].tolist() == [-g for g in GRID]
    assert np.signbit(vals[8])


def test_e2m1_encode_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(formats.e2m1_encode(formats.e2m1_decode(codes)), codes)


def test_e2m1_encode_matches_brute_force_near_decision_points():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + GRID[1:] + [6.5, 7.0, 8.0]
    v = _near(mids, 3)
    v = np.concatenate([v, -v, np.float32([0.0, -0.0, 1e-45, -1e-45, np.inf, -np.inf, 1e30, -1e30])])
    assert np.array_equal(formats.e2m1_encode(v), _brute_e2m1(v))


def test_e2m1_encode_matches_brute_force_random():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 0x41400000, 20000, dtype=np.int64).astype(np.int32)  # |v| < 12
    v = u.view(np.float32)
    v = np.where(rng.random(v.shape) < 0.5, -v, v).astype(np.float32)
    assert np.array_equal(formats.e2m1_encode(v), _brute_e2m1(v))


def test_e2m1_ties_and_saturation():
    enc = formats.e2m1_encode
    assert enc(np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert enc(np.float32([6.0, 7.0, 1e6, np.inf])).tolist() == [7, 7, 7, 7]
    assert enc(np.float32([-0.0, -1e-30, -0.25])).tolist() == [8, 8, 8]


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = formats.e4m3_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert formats.e4m3_decode(np.uint8([0x7E, 0x01, 0x38, 0x08])).tolist() == [448.0, 2.0 ** -9, 1.0, 2.0 ** -6]


def test_e4m3_encode_roundtrip_all_finite_codes():
    b = np.array([c for c in range(0x7F)], dtype=np.uint8)  # non-negative finite codes
    assert np.array_equal(formats.e4m3_encode(formats.e4m3_decode(b)), b)


def test_e4m3_encode_matches_torch_below_464():
    vals = formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0  # every rounding boundary (exact in float32)
    probes = [_near(vals.astype(np.float32), 3), _near(mids.astype(np.float32), 3)]
    rng = np.random.default_rng(2)
    probes.append(rng.integers(0, 0x43E80001, 300000, dtype=np.int64).astype(np.int32).view(np.float32))
    bf = (np.arange(0, 0x43E9, dtype=np.uint32) << 16).view(np.float32)  # every bf16 value <= 464
    probes.append(bf)
    x = np.concatenate(probes)
    x = x[(x >= 0) & (x <= 464.0)]
    assert np.array_equal(formats.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_saturates():
    assert formats.e4m3_encode(np.float32([448.0, 465.0, 1e10, np.inf])).tolist() == [0x7E] * 4


def test_bf16_from_f64_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 0x7F800000, 200000, dtype=np.int64).astype(np.int32)
    x = u.view(np.float32)
    x = np.where(rng.random(x.shape) < 0.5, -x, x).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.bf16_from_f64(x.astype(np.float64)), ref)


def test_bf16_from_f64_single_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-7: the exact
    # rounding goes up; rounding through float32 first would tie and go down.
    y = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert formats.bf16_from_f64(np.float64([y])).tolist() == [0x3F81]
    rng = np.random.default_rng(4)
    ys = rng.standard_normal(300) * np.exp2(rng.integers(-20, 20, 300))
    for yv, bits in zip(ys, formats.bf16_from_f64(ys)):
        got = Fraction(float(formats.bf16_to_f32(np.uint16(bits))))
        # the exact nearest bf16: check no representable neighbour is closer
        f = np.float32(float(formats.bf16_to_f32(np.uint16(bits))))
        up = formats.bf16_to_f32(np.uint16(bits + 1))
        dn = formats.bf16_to_f32(np.uint16(bits - 1))
        d = abs(Fraction(float(yv)) - got)
        assert d <= abs(Fraction(float(yv)) - Fraction(float(up)))
        assert d <= abs(Fraction(float(yv)) - Fraction(float(dn)))
        assert np.isfinite(f)


@pytest.mark.parametrize("y,bits", [(0.0, 0x0000), (-0.0, 0x8000), (np.inf, 0x7F80), (-np.inf, 0xFF80),
                                    (3.5e38, 0x7F80), (1.0, 0x3F80), (-2.0, 0xC000)])
def test_bf16_from_f64_specials(y, bits):
    assert int(formats.bf16_from_f64(np.float64([y]))[0]) == bits
