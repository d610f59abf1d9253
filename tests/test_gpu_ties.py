"""E2M1 rounding at its decision points, on the GPU quantizers (needs an MI355X).

Rotate notes, section 1: q = round(x / scale).  The E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} has
its decision points at 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 (and saturates above 6); a value
exactly on one rounds to the neighbour with an even mantissa bit.  Random data almost never
lands there, so these tests build groups that do: with smooth_factor = 1 the quantized value is
the bf16 input itself, a group holding 6 sd has stored scale sd exactly (amax / 6 = sd), and
t * sd is a bf16 value for every decision point t and every e4m3 scale sd.  Each group also
holds the bf16 neighbours of t * sd (one step either side), negatives, zeros and -0.  The weight
quantizer is also fed exact bf16 x bf16 products that fall just beside the decision points.
Codes and scale bytes must equal the oracle's bit for bit, and the tie codes must be the even
neighbours that the round-to-nearest-even definition gives.
"""

import numpy as np
import pytest

import helpers as H
from oracle import formats
from oracle import mx as omx
from oracle import quant as oquant

pytestmark = pytest.mark.gpu

POINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
# round to nearest, ties to the even mantissa bit: the code each decision point itself takes
TIE_CODES = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}


@pytest.fixture(scope="module")
def w4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import w4a4_bit_quantized_amd as w
    w.load_library()
    return w


def _bf16_exact(v):
    bits = formats.bf16_from_f64(np.float64(v))
    assert float(formats.bf16_to_f32(bits)) == v, v
    return int(bits)


def _step(bits, d):
    """The bf16 value d steps away from a positive bf16 value (bit patterns are monotonic)."""
    return bits + d


def _tie_groups(sd):
    """Two 16-element groups (bf16 bit patterns) whose maximum magnitude is 6 sd."""
    top = _bf16_exact(6.0 * sd)
    ties = [_bf16_exact(t * sd) for t in POINTS]
    g1 = [top] + ties + [_step(b, d) for b in ties[:4] for d in (-1, 1)]
    g2 = [top] + [_step(b, d) for b in ties[4:] for d in (-1, 1)] + [b | 0x8000 for b in ties] + [0x0000, 0x8000]
    assert len(g1) == 16 and len(g2) == 16
    return g1, g2


def _tie_rows():
    """One row per nonzero finite e4m3 scale (codes 1 .. 126), two groups each: x (126, 32)."""
    rows = []
    for s8 in range(1, 127):
        sd = float(formats.e4m3_decode(np.uint8(s8)))
        g1, g2 = _tie_groups(sd)
        rows.append(g1 + g2)
    return np.array(rows, dtype=np.uint16)


def _expected_tie_codes(x_bits):
    """The oracle's codes for the tie rows, also checked here against the even-neighbour rule."""
    x = formats.bf16_to_f32(x_bits)
    codes, s8 = oquant.group_quantize(x)
    assert np.array_equal(s8[:, 0], np.arange(1, 127)) and np.array_equal(s8[:, 1], np.arange(1, 127))
    for i, t in enumerate(POINTS):
        assert np.all(codes[:, 1 + i] == TIE_CODES[t])          # +t sd
        assert np.all(codes[:, 16 + 7 + i] == 8 | TIE_CODES[t])  # -t sd
    assert np.all(codes[:, 30] == 0) and np.all(codes[:, 31] == 8)  # +0, -0
    assert np.all(codes[:, 0] == 7) and np.all(codes[:, 16] == 7)   # 6 sd
    return codes, s8


def test_activation_quantizer_at_decision_points(w4):
    import torch
    x_bits = _tie_rows()
    M, K = x_bits.shape
    _expected_tie_codes(x_bits)
    ones = formats.bf16_from_f64(np.ones(K))
    pd = np.zeros((K, 0), dtype=np.uint16)
    qa, sa, _ = w4.svdq_quantize_act(H.to_dev_bf16(x_bits), H.to_dev_bf16(ones), H.to_dev_bf16(pd), 0)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = oquant.quantize_act(formats.bf16_to_f32(x_bits), formats.bf16_to_f32(ones),
                                          np.zeros((K, 0), np.float32), 0)
    assert np.array_equal(sa.cpu().numpy(), s_ref)
    bad = np.argwhere(qa.cpu().numpy() != q_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"


def test_weight_quantizer_at_decision_points(w4):
    """Exact ties (smooth_factor 1), then exact bf16 x bf16 products beside every tie: for each
    group the column smoothing factors are bf16 values in [0.5, 2] and the weights the bf16
    values nearest t * sd / lambda and one step either side."""
    import torch
    x_bits = _tie_rows()
    N, K = x_bits.shape
    ones = formats.bf16_from_f64(np.ones(K))
    qw, ws = w4.svdq_quantize_weight(H.to_dev_bf16(x_bits), H.to_dev_bf16(ones), 0)
    torch.cuda.synchronize()
    q_ref, s_ref = oquant.quantize_weight(formats.bf16_to_f32(x_bits), formats.bf16_to_f32(ones), 0)
    assert np.array_equal(ws.cpu().numpy(), s_ref) and np.array_equal(qw.cpu().numpy(), q_ref)

    # near ties from products: column 0 of each group has lambda = 1 and w = 6 sd (the scale)
    rng = np.random.default_rng(7)
    G = 6
    lam = formats.bf16_from_f64(rng.uniform(0.5, 2.0, 16 * G))
    lam[::16] = formats.bf16_from_f64(np.ones(G))
    lam_f = formats.bf16_to_f32(lam).astype(np.float64)
    w = np.zeros((126, 16 * G), dtype=np.uint16)
    for s8 in range(1, 127):
        sd = float(formats.e4m3_decode(np.uint8(s8)))
        for g in range(G):
            w[s8 - 1, 16 * g] = _bf16_exact(6.0 * sd)
            for j in range(1, 16):
                t = POINTS[(j - 1 + g) % 7]
                col = 16 * g + j
                base = int(formats.bf16_from_f64(t * sd / lam_f[col]))
                w[s8 - 1, col] = _step(base, (j + g) % 3 - 1)
    qw, ws = w4.svdq_quantize_weight(H.to_dev_bf16(w), H.to_dev_bf16(lam), 0)
    torch.cuda.synchronize()
    q_ref, s_ref = oquant.quantize_weight(formats.bf16_to_f32(w), formats.bf16_to_f32(lam), 0)
    assert np.array_equal(ws.cpu().numpy(), s_ref)
    bad = np.argwhere(qw.cpu().numpy() != q_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"


def _mx_tie_rows():
    """MX blocks of 32 with amax = 6 * 2^e (scale 2^e exactly) for e = -20 .. 20: the seven
    decision points times 2^e, their bf16 neighbours, negatives and signed zeros."""
    rows = []
    for e in range(-20, 21):
        s = 2.0 ** e
        top = _bf16_exact(6.0 * s)
        ties = [_bf16_exact(t * s) for t in POINTS]
        blk = [top] + ties + [_step(b, d) for b in ties for d in (-1, 1)] + [b | 0x8000 for b in ties]
        blk += [0x0000, 0x8000, top | 0x8000]
        assert len(blk) == 32
        rows.append(blk + blk[::-1])
    return np.array(rows, dtype=np.uint16)


def test_mx_quantizers_at_decision_points(w4):
    import torch
    x_bits = _mx_tie_rows()
    M, K = x_bits.shape
    ones = formats.bf16_from_f64(np.ones(K))
    pd = np.zeros((K, 0), dtype=np.uint16)
    x_f = formats.bf16_to_f32(x_bits)
    codes, e8 = omx.group_quantize_mx(x_f)
    assert np.array_equal(e8[:, 0].astype(int) - 127, np.arange(-20, 21))
    for i, t in enumerate(POINTS):
        assert np.all(codes[:, 1 + i] == TIE_CODES[t])
    qa, sa, _ = w4.svdq_quantize_act_mx(H.to_dev_bf16(x_bits), H.to_dev_bf16(ones), H.to_dev_bf16(pd), 0)
    qw, sw = w4.svdq_quantize_weight_mx(H.to_dev_bf16(x_bits), H.to_dev_bf16(ones), 0)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = omx.quantize_act_mx(x_f, formats.bf16_to_f32(ones), np.zeros((K, 0), np.float32), 0)
    assert np.array_equal(qa.cpu().numpy(), q_ref) and np.array_equal(sa.cpu().numpy(), s_ref)
    qw_ref, sw_ref = omx.quantize_weight_mx(x_f, formats.bf16_to_f32(ones), 0)
    assert np.array_equal(qw.cpu().numpy(), qw_ref) and np.array_equal(sw.cpu().numpy(), sw_ref)
