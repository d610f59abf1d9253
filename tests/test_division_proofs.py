"""Exactness of the quantizer's two fast divisions (CPU, exact rational arithmetic).

The activation quantizer never issues a divide instruction per element:

* smoothing, x / lambda (rotate notes section 1 and the "SVDQuant W4A4" page's smooth_factor):
  x and lambda are bf16; lambda = m 2^E with m one of 128 significands.  A table holds, per m,
  rh = RD(1/m) and rl = RN((1 - m rh) rh) (the residual 1 - m rh is exact and >= 0); per column
  the kernel scales both by 2^-E (exact), and per element it computes

      q = RN(x * rh + RN(x * rl))       (a multiply, then a fused multiply-add)

  Claim: q == RN(x/lambda) bit for bit, signed zeros included, whenever 2^-64 <= |x| < 2^96 (or
  x = +-0) and 2^-32 <= lambda <= 2^32 (the kernel takes the IEEE division for any wave holding
  an input outside this range).
* group quantization, v / sd (rotate notes section 1: q = round(x / scale)): v is any float32,
  sd a nonzero e4m3 scale, r = RN(1/sd) comes from a 128-entry table and one Markstein
  correction follows, each step a single IEEE float32 rounding (the corrections are fused
  multiply-adds, rounded once):

      q0 = RN(v * r);   e = RN(q0 * sd - v);   q = RN(q0 - e * r)

  Claim: the E2M1 code of q equals the code of RN(v/sd) for every finite v.

Every step below is emulated with Python Fractions and an exact round-to-nearest-even to
float32 (normal and subnormal), so nothing here runs the kernel's arithmetic in float32.
The rounding emulation itself is pinned against numpy's IEEE float32 operations.
"""

import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats

F = Fraction
TWO = F(2)


def rn32(v):
    """Round an exact rational to the nearest float32 value (ties to even), as a Fraction.
    Subnormals use the fixed step 2^-149; overflow is an error here (never reached)."""
    if v == 0:
        return F(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if TWO ** e > a:
        e -= 1
    assert TWO ** e <= a < TWO ** (e + 1)
    e = max(e, -126)
    ulp = TWO ** (e - 23)
    q, r = divmod(a, ulp)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    out = q * ulp
    assert out < TWO ** 128, "float32 overflow"
    return s * out


def markstein(x, d, r):
    """The kernel's division sequence, each step rounded once (fused steps: exact product)."""
    q0 = rn32(x * r)
    e = rn32(q0 * d - x)
    return rn32(q0 - e * r)


def _fma_signed(a, b, c):
    """RN(a * b + c) on (value, negative) pairs, with IEEE signed zeros: an exact zero sum of two
    zeros is negative only if both are; an exact cancellation of nonzero terms gives +0; a nonzero
    value that rounds to zero keeps its sign."""
    (av, an), (bv, bn), (cv, cn) = a, b, c
    pv, pn = av * bv, an != bn
    ex = pv + cv
    out = rn32(ex)
    if out != 0:
        return out, out < 0
    if ex != 0:
        return out, ex < 0
    if pv == 0 and cv == 0:
        return out, pn and cn
    return out, False


def markstein_signed(x, d, r):
    """markstein() on (value, negative) pairs: the sign of a zero result is tracked."""
    p = x[0] * r  # plain multiply: the sign of a zero product is the xor of the signs (r > 0)
    q0 = (rn32(p), x[1] if rn32(p) == 0 else p < 0)
    e = _fma_signed(q0, (d, False), (-x[0], not x[1]))
    return _fma_signed((-e[0], not e[1]), (r, False), q0)


def test_rounding_emulation_matches_ieee_float32():
    """rn32 agrees with numpy's float32 multiply, divide and float64 -> float32 conversion
    (each a correctly rounded IEEE operation) on random operands, subnormal results included."""
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-70, 70, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-70, 70, 3000))).astype(np.float32)
    with np.errstate(all="ignore"):
        prod = a * b
        quot = a / b
    for i in range(3000):
        fa, fb = F(float(a[i])), F(float(b[i]))
        if np.isfinite(prod[i]) and abs(float(prod[i])) < 3e38:
            assert rn32(fa * fb) == F(float(prod[i])), (a[i], b[i])
        if np.isfinite(quot[i]) and abs(float(quot[i])) < 3e38:
            assert rn32(fa / fb) == F(float(quot[i])), (a[i], b[i])
    d = rng.standard_normal(2000) * np.exp2(rng.integers(-160, 100, 2000).astype(np.float64))
    for v in d:
        assert rn32(F(float(v))) == F(float(np.float32(v))), v


def _bf16_values(lo_exp, hi_exp):
    """Every positive bf16 value with exponent in [lo_exp, hi_exp] (8 significant bits)."""
    return [F(m, 128) * TWO ** e for e in range(lo_exp, hi_exp + 1) for m in range(128, 256)]


def _prev32(v):
    """The float32 value just below the positive normal float32 v (its bit pattern minus one)."""
    return F(float(np.nextafter(np.float32(float(v)), np.float32(0))))


def recip_parts(lam):
    """(rh, rl) of a bf16 lambda = m 2^E as the kernel forms them: the table entry of m, built
    with one IEEE division, a round-down step and the exact residual, scaled by 2^-E."""
    e_ = 0
    m = lam
    while m >= 2:
        m, e_ = m / 2, e_ + 1
    while m < 1:
        m, e_ = m * 2, e_ - 1
    rh = rn32(1 / m)
    if rn32(1 - m * rh) < 0:  # the kernel's test: fma(-m, rh, 1) < 0
        rh = _prev32(rh)
    res = 1 - m * rh
    assert res >= 0 and rn32(res) == res, "the residual of a round-down reciprocal is exact"
    rl = rn32(res * rh)
    return rh * TWO ** -e_, rl * TWO ** -e_


def smooth_div(x, lam, parts=None):
    """The kernel's smoothing quotient: RN(x rh + RN(x rl))."""
    rh, rl = parts or recip_parts(lam)
    return rn32(x * rh + rn32(x * rl))


def smooth_div_signed(x, lam):
    """smooth_div() on (value, negative) pairs: the sign of a zero result is tracked (rh > 0 and
    rl >= 0, so x * rl is a zero of x's sign when x is zero)."""
    rh, rl = recip_parts(lam)
    t = rn32(x[0] * rl)
    return _fma_signed(x, (rh, False), (t, x[1] if t == 0 else t < 0))


def test_reciprocal_table_entries():
    """For each of the 128 bf16 significands m: rh = RD(1/m) (never above 1/m, within one ulp),
    the residual 1 - m rh exact and non-negative (asserted inside recip_parts), and rh + rl
    within 2^-46 of 1/m: the two-part reciprocal the per-element sequence relies on."""
    for k in range(128, 256):
        m = F(k, 128)
        rh, rl = recip_parts(m)
        assert rh <= 1 / m < rh + TWO ** -23
        assert rl >= 0
        assert abs(rh + rl - 1 / m) <= TWO ** -46 / m


def test_smoothing_division_exact_over_every_bf16_mantissa_pair():
    """Every pair of bf16 significands (x in [1, 2), lambda in [1, 2)): q == RN(x / lambda).
    Within the stated ranges the quotient and x rh are normal float32 values and RN(x rl) errs by
    far less than the quotient's distance to a rounding midpoint (a quotient of two 8-bit
    significands is exact or at least 2^-33 of its size away from every float32 midpoint, while
    rh + rl and the rounding of x rl stay within 2^-45 of it), so the pairs cover all exponents;
    the corners of the range are checked directly below.  The sequence is odd in x, so negative
    x follow; the sign of zero is checked separately."""
    xs = _bf16_values(0, 0)
    bad = []
    for lam in xs:
        parts = recip_parts(lam)
        for x in xs:
            if smooth_div(x, lam, parts) != rn32(x / lam):
                bad.append((x, lam))
    assert not bad, f"{len(bad)} pairs differ, first {bad[:3]}"


@pytest.mark.parametrize("xe,le", [(-64, 32), (95, -32), (-64, -32), (95, 32), (40, 7), (-20, -5)])
def test_smoothing_division_exact_at_the_range_ends(xe, le):
    """The corners of the stated range (|x| = 2^-64 .. 2^96, lambda = 2^-32 .. 2^32), where x rl
    can be subnormal: every x significand against a stride of lambda significands."""
    lam_e = le if le < 32 else 31  # lambda <= 2^32: significands of the binade below, and 2^32 itself
    lams = [F(m, 128) * TWO ** lam_e for m in range(128, 256, 5)] + [TWO ** le]
    for lam in lams:
        parts = recip_parts(lam)
        for m in range(128, 256):
            x = F(m, 128) * TWO ** xe
            assert smooth_div(x, lam, parts) == rn32(x / lam), (x, lam)
            assert smooth_div(-x, lam, parts) == -rn32(x / lam), (-x, lam)


def test_smoothing_division_signed_zero():
    """x = +0 gives +0 and x = -0 gives -0, as the IEEE division does (lambda > 0)."""
    for lam in (F(1), F(3, 2), F(255, 128), TWO ** -32, TWO ** 32):
        for neg in (False, True):
            assert smooth_div_signed((F(0), neg), lam) == (F(0), neg)


def test_smoothing_sequence_is_not_exact_with_rounded_reciprocal_alone():
    """Planted-mistake check of the proof itself: with only rh (rl dropped) some pairs round
    differently, so the exhaustive test above does detect a wrong sequence."""
    xs = _bf16_values(0, 0)
    diff = 0
    for lam in xs[::7]:
        rh, _ = recip_parts(lam)
        diff += sum(rn32(x * rh) != rn32(x / lam) for x in xs)
    assert diff > 0


E2M1_POINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _code(v):
    return int(formats.e2m1_encode(np.float32(float(v))))


def _f32_neighbours(T, k):
    """T and the k float32 values on each side of it (as Fractions)."""
    t = np.float32(float(T))
    out = [t]
    up = dn = t
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return [F(float(u)) for u in out]


def test_group_division_codes_at_every_decision_point():
    """For every nonzero finite e4m3 scale sd (codes 1 .. 126) and every E2M1 decision point t,
    the float32 values v within 8 ulps of t * sd (exact in float32: at most 7 significant bits):
    the table sequence gives exactly RN(v / sd), hence the same code, for both signs.
    Away from the decision points the codes cannot differ: the sequence's result is within one
    ulp of v / sd (it is RN(v/sd + eps) with |eps| below 2^-45 |v/sd|), so only a quotient within
    one ulp of a decision point could change code, and those are the values checked here."""
    for s8 in range(1, 127):
        sd = F(float(formats.e4m3_decode(np.uint8(s8))))
        r = rn32(1 / sd)
        for t in E2M1_POINTS:
            T = F(t) * sd
            assert rn32(T) == T, "t * sd is exact in float32"
            for v in _f32_neighbours(T, 8):
                ieee = rn32(v / sd)
                q = markstein(v, sd, r)
                assert q == ieee, (s8, t, v)
                assert _code(q) == _code(ieee)
                assert markstein(-v, sd, r) == -ieee


def test_group_division_exact_on_random_operands():
    """Random float32 v across the binades a group holds (|v / sd| from 2^-6 to 14) for every
    scale: the sequence equals the IEEE quotient, so the codes agree everywhere, not only near
    ties (sd has at most 4 significant bits, so v / sd is never within 2^-45 of a float32
    midpoint unless it is exact).  Subnormal v: the same code (0, or 0x8 when negative)."""
    rnd = random.Random(1)
    for s8 in range(1, 127):
        sd = F(float(formats.e4m3_decode(np.uint8(s8))))
        r = rn32(1 / sd)
        for _ in range(60):
            mant = rnd.randrange(1 << 23, 1 << 24)
            v = F(mant, 1 << 23) * sd * F(rnd.choice([1, 3, 5, 7]), 8) * TWO ** rnd.randrange(-3, 3)
            v = rn32(v)
            assert markstein(v, sd, r) == rn32(v / sd), (s8, v)
        for k in (1, 3, 1000, (1 << 23) - 1):
            # subnormal v: the residual e can underflow, so q may miss RN(v / sd) by an ulp, but
            # both lie far below the first decision point: the same code, 0x8 when negative
            v = F(k) * TWO ** -149
            for neg in (False, True):
                q, qn = markstein_signed((-v if neg else v, neg), sd, r)
                ieee = rn32((-v if neg else v) / sd)
                assert abs(q) < F(1, 4) and abs(ieee) < F(1, 4) and qn == neg, (s8, k, neg)
                assert _code(q) | (8 if qn else 0) == _code(ieee) | (8 if neg else 0)
