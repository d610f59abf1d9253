"""MXFP4 variant of the W4A4 layer (oracle, test infrastructure only).

Source: rotate notes, section 3.3 (FP-Quant): activations are rotated with a
32 x 32 Hadamard per group (``hadamard_group_size = 32``) and quantized to
``forward_dtype = "mxfp4"`` with ``forward_method = "abs_max"`` in one fused
kernel (``fused_quantize_mx(x, H, method) -> (x_q, x_scales)``), then
``matmul_mxf4_bf16(x_q, qweight, x_scales, w_scales, alpha)`` multiplies.  The
pages name the format only.  MXFP4 is the OCP microscaling format: E2M1
elements in blocks of 32 along K sharing one E8M0 scale (an 8-bit power-of-two
exponent with bias 127, value 2^(b - 127); 0xFF is NaN).

Readings taken where the pages are silent (the GPU path uses the same ones):

* "abs_max" scale for a block: the smallest power of two not below
  float32(amax / 6) -- the power-of-two analogue of the nvfp4 scale amax / 6,
  so that no element is clipped by the scale (OCP's floor(log2 amax) - 2 rule
  clips blocks whose amax lies in (6, 8) x 2^k).  The exponent is clamped to
  the E8M0 range [-127, 127]; an all-zero block gets 2^-127.
* elements are multiplied by the exact power of two 2^-e (no rounding except
  underflow far below the first E2M1 step) and rounded to E2M1 exactly as in the
  nvfp4 path (nearest even, saturating at 6, sign of zero kept);
* activation scales are laid out (K/32, Mp) with Mp = M rounded up to a
  multiple of 4 (the padding columns are zero bytes), weight scales (K/32, N);
* everything else -- smoothing, the optional rotation (here normally B = 32),
  the unrotated low-rank branch, the epilogue -- is the nvfp4 layer's.

Inputs are finite, and so are their rotated values (a block that holds an
infinity or NaN, or whose rotation overflows float32, has no defined MX scale
here).

Pins (``tests/test_oracle_mx.py``): E8M0 values from the OCP table and the
doubling invariant; the scale exponent against a brute-force search over
powers of two; every grid value at every scale reproduced exactly; the
reconstruction bound; a pure-Python block-scaled triple loop for the GEMM.
"""

import numpy as np

from . import formats, quant
from .hadamard import fwht_blocks

MX_GROUP = 32
E8M0_BIAS = 127


def e8m0_decode(b):
    """Value 2^(b - 127) of each E8M0 byte as float64 (exact); 0xFF -> NaN."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - E8M0_BIAS)
    return np.where(b == 0xFF, np.nan, v)


def scale_exponent(amax):
    """Exponent e of the block scale 2^e: the least e with 2^e >= float32(amax / 6), clamped to [-127, 127].

    ``amax`` are float32 block maxima (finite, non-negative).
    """
    q = (np.asarray(amax, dtype=np.float32) / np.float32(6.0)).astype(np.float32)  # IEEE float32 division
    f, x = np.frexp(q.astype(np.float64))  # q = f * 2^x, f in [0.5, 1) (exact)
    e = np.where(f == 0.5, x - 1, x).astype(np.int64)  # exact power of two: no round-up
    e = np.where(q == 0, -E8M0_BIAS, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def group_quantize_mx(v):
    """Quantize float32 rows (..., K) into E2M1 codes (..., K) and E8M0 bytes (..., K/32)."""
    v = np.asarray(v, dtype=np.float32)
    k = v.shape[-1]
    if k % MX_GROUP:
        raise ValueError("K must be a multiple of 32")
    g = v.reshape(v.shape[:-1] + (k // MX_GROUP, MX_GROUP))
    amax = np.max(np.abs(g), axis=-1)
    e = scale_exponent(amax)
    t = (g.astype(np.float64) * np.ldexp(1.0, -e)[..., None]).astype(np.float32)  # exact, then float32
    codes = formats.e2m1_encode(t)
    return codes.reshape(v.shape), (e + E8M0_BIAS).astype(np.uint8)


def pad_rows4(n):
    return (n + 3) // 4 * 4


def quantize_act_mx(x, smooth_factor, proj_down, hadamard_block=32):
    """Online activation path of the MX variant.

    Returns ``qact (M, K/2) uint8``, ``ascales (K/32, Mp) uint8`` (E8M0, Mp = M
    rounded up to 4, padding zero) and ``lora_act (M, R) float64``.
    """
    xs = quant.smooth(x, smooth_factor)
    v = fwht_blocks(xs, hadamard_block) if hadamard_block else xs
    codes, e8 = group_quantize_mx(v)
    m = xs.shape[0]
    ascales = np.zeros((e8.shape[1], pad_rows4(m)), dtype=np.uint8)
    ascales[:, :m] = e8.T
    pd = np.asarray(proj_down, dtype=np.float64)
    lora = xs.astype(np.float64) @ pd if pd.shape[1] else np.zeros((m, 0))
    return quant.pack_nibbles(codes), ascales, lora


def quantize_weight_mx(w, smooth_factor, hadamard_block=32):
    """Offline weight path of the MX variant: fold smoothing, rotate, quantize.  Returns qweight, wscales (K/32, N)."""
    wq = (np.asarray(w, dtype=np.float32) * np.asarray(smooth_factor, dtype=np.float32)[None, :]).astype(np.float32)
    if hadamard_block:
        wq = fwht_blocks(wq, hadamard_block)
    codes, e8 = group_quantize_mx(wq)
    return quant.pack_nibbles(codes), np.ascontiguousarray(e8.T)


def dequant_mx(packed, scales_t, rows):
    """Dequantize packed codes (rows, K/2) with E8M0 scales (K/32, >= rows) -> float64 (rows, K)."""
    vals = formats.e2m1_decode(quant.unpack_nibbles(packed)).astype(np.float64)
    sd = e8m0_decode(np.asarray(scales_t)[:, :rows].T)  # (rows, K/32)
    return vals * np.repeat(sd, MX_GROUP, axis=1)


def gemm_lowrank_mx(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, bias=None):
    """MX block-scaled product plus the layer's epilogue.  Returns (y_bits bf16, y_f64)."""
    m, n = qact.shape[0], qweight.shape[0]
    a = dequant_mx(qact, ascales, m)
    wd = dequant_mx(qweight, wscales, n)
    acc = a @ wd.T
    col = np.asarray(wcscales, dtype=np.float64) * np.float64(np.asarray(wtscale, dtype=np.float64).reshape(-1)[0])
    y = acc * col[None, :]
    pu = np.asarray(proj_up, dtype=np.float64)
    if pu.shape[1]:
        y = y + np.asarray(lora_act, dtype=np.float64) @ pu.T
    if bias is not None:  # the optional per-output offset, as in the nvfp4 layer
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return formats.bf16_from_f64(y), y


def svdq_linear_mx(x, layer, hadamard_block=32):
    """Whole MX layer: ``quantize_act_mx`` then ``gemm_lowrank_mx``."""
    qact, ascales, lora = quantize_act_mx(x, layer["smooth_factor"], layer["proj_down"], hadamard_block)
    yb, y = gemm_lowrank_mx(qact, ascales, lora, layer["qweight"], layer["wscales"], layer["proj_up"],
                            layer["wcscales"], layer["wtscale"], layer.get("bias"))
    return yb, y, (qact, ascales, lora)
