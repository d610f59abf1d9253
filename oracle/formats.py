"""Number formats of the W4A4 checkpoint contract (oracle, test infrastructure only).

Source: "SVDQuant W4A4" page, section "Checkpoint contract" -- weights are FP4
values packed two per byte with float8_e4m3fn scales, and the configuration's
``precision`` is ``nvfp4`` (E2M1 elements, one e4m3 scale per 16 elements).
The pages name the formats only; the encodings below are the OCP definitions:

* E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no inf/NaN.
* float8_e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormal step
  2^-9; largest finite 448 (0x7E); 0x7F/0xFF are NaN; no inf.

Readings taken where the pages are silent:

* encoders round to nearest, ties to the even mantissa bit;
* the e4m3 scale encoder saturates every value >= 448 to 0x7E (never NaN);
* the E2M1 encoder saturates to +-6 and keeps the sign of zero (-0 -> 0x8).

Pins: ``e4m3_encode``/``e4m3_decode`` against torch's CPU float8_e4m3fn
conversion; ``e2m1_encode`` against a brute-force nearest-of-grid search in
float64 with an explicit tie rule; ``bf16_from_f64`` against exact rational
rounding and torch's float32->bfloat16 conversion.
"""

import numpy as np

# E2M1 magnitudes, indexed by the low 3 bits of a code (exponent:mantissa).
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (0..15) as float32 (exact)."""
    c = np.asarray(codes).astype(np.uint8) & np.uint8(0xF)
    mag = _E2M1_MAG[c & np.uint8(7)]
    return np.where(c & np.uint8(8), -mag, mag).astype(np.float32)


def e2m1_encode(v):
    """Round float32 values to E2M1 codes (uint8 in 0..15).

    Round to nearest on the E2M1 grid.  A value exactly half way between two
    neighbours goes to the one with mantissa bit 0, which puts the ties 0.25,
    1.25, 2.5 and 5 on the lower neighbour and 0.75, 1.75 and 3.5 on the upper
    one.  Magnitudes above 5 (including inf) saturate to 6.  The sign bit of the
    input is kept, so -0.0 and tiny negatives encode as 0x8.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    code = np.full(a.shape, 7, dtype=np.uint8)
    # Walk the decision points from the top down; each test overwrites the
    # code for every magnitude at or below (or strictly below) the point.
    code = np.where(a <= np.float32(5.0), np.uint8(6), code)
    code = np.where(a < np.float32(3.5), np.uint8(5), code)
    code = np.where(a <= np.float32(2.5), np.uint8(4), code)
    code = np.where(a < np.float32(1.75), np.uint8(3), code)
    code = np.where(a <= np.float32(1.25), np.uint8(2), code)
    code = np.where(a < np.float32(0.75), np.uint8(1), code)
    code = np.where(a <= np.float32(0.25), np.uint8(0), code)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    return (code | sign).astype(np.uint8)


def e4m3_decode(b):
    """Value of each float8_e4m3fn byte as float32 (exact; 0x7F/0xFF -> NaN)."""
    b = np.asarray(b).astype(np.uint8)
    s = (b >> 7) & 1
    e = ((b >> 3) & 0xF).astype(np.int32)
    m = (b & 7).astype(np.float64)
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where(s == 1, -val, val)
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float32)


def e4m3_encode(s):
    """Encode non-negative float32 scales as float8_e4m3fn bytes.

    Round to nearest, ties to even mantissa; values below the smallest normal
    2^-6 use the subnormal step 2^-9; every value >= 448 (and +inf) saturates
    to 0x7E.  Only non-negative inputs occur (scales are amax / 6).
    """
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    out = np.zeros(s.shape, dtype=np.int64)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        small = s < 2.0 ** -6
        # subnormal range: integer multiple of 2^-9, RNE (np.rint is ties-to-even)
        m_sub = np.rint(np.where(small, s, 0.0) * 2.0 ** 9).astype(np.int64)
        # normal range: s = f * 2^x with f in [0.5, 1)  ->  exponent x - 1
        safe = np.where(small | ~np.isfinite(s), 1.0, s)
        _, x = np.frexp(safe)
        e = x.astype(np.int64) - 1
        mant = safe / np.exp2(e.astype(np.float64))  # in [1, 2), exact
        m = np.rint((mant - 1.0) * 8.0).astype(np.int64)  # 0..8, exact RNE
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        code_n = ((e + 7) << 3) | m
        out = np.where(small, m_sub, code_n)  # m_sub == 8 is 0x08, the smallest normal
        out = np.where(s >= 448.0, 0x7E, out)
        out = np.where(np.isnan(s), 0x7F, out)
    return out.astype(np.uint8)


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_from_f64(y):
    """Round float64 values once, to nearest-even, to bf16 bit patterns (uint16).

    Rounding is done directly from float64 (no float32 step, so there is no
    double rounding).  Overflow past the largest bf16 goes to +-inf; NaN maps
    to the canonical quiet NaN 0x7FC0.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        safe = np.where((a > 0) & np.isfinite(a), a, 1.0)
        _, x = np.frexp(safe)
        e = np.maximum(x.astype(np.int64) - 1, -126)  # subnormals share the 2^-126 ulp grid
        ulp = np.exp2((e - 7).astype(np.float64))  # bf16 keeps 8 significant bits
        r = np.rint(safe / ulp) * ulp
        r = np.where(a > 0, r, 0.0)
        r = np.where(np.isinf(a) | (r >= 2.0 ** 128), np.inf, r)
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(y), bits | np.uint16(0x8000), bits).astype(np.uint16)
    bits = np.where(np.isnan(y), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits
