"""Quantizers of the W4A4 linear (oracle, test infrastructure only).

Sources:

* "SVDQuant W4A4" page, "Checkpoint contract": FP4 pairs packed per byte,
  one float8_e4m3fn scale per 16 inputs along K (``wscales`` is (K/16, N)),
  ``smooth_factor (K,)``, ``proj_down (K, R)``; "Overview": 4-bit weights and
  activations plus a low-rank branch; the checkpoint is quantized offline.
* Rotate notes, section 1: absmax quantization, scale = max|x| / qmax,
  q = round(x / scale), x_hat = q * scale (signed INT4 uses qmax = 7, unsigned
  qmax = 15); section 2.1: weights rotated offline (R W), activations online
  (x R^T).

Readings taken where the pages are silent (the GPU path uses the same ones):

* group scale = float32(amax / 6), 6 being the largest E2M1 magnitude, stored
  as e4m3 (round to nearest even, saturating at 448);
* elements are divided by the *decoded* stored scale (IEEE float32 division)
  and rounded to E2M1; a group whose stored scale is 0 gets all-zero codes;
* two codes per byte, the even-k element in the low nibble;
* activation scales are laid out (K/16, M), mirroring ``wscales (K/16, N)``;
* smoothing divides activations by ``smooth_factor`` (IEEE float32) and folds
  the same factor into the weights by multiplication (SmoothQuant direction);
* the optional rotation follows smoothing; the low-rank down-projection uses
  the smoothed, unrotated activations (it approximates W diag(smooth) in the
  unrotated basis);
* the low-rank product x_s @ proj_down is accumulated in float64 from the
  float32 smoothed values.

Pins: INT4 worked examples of the rotate notes; reconstruction bound and
special cases of the group quantizer; byte-level layout checks; dense
brute-force composition (see ``tests/test_oracle_quant.py``).
"""

import numpy as np

from . import formats
from .hadamard import fwht_blocks

GROUP = 16
E2M1_MAX = np.float32(6.0)


def group_quantize(v):
    """Quantize float32 rows (..., K) into E2M1 codes (..., K) and e4m3 scale bytes (..., K/16).

    For each group of 16 consecutive elements along the last axis:
    amax = max |v|, s = float32(amax / 6), s8 = e4m3(s), sd = decode(s8),
    code_k = e2m1(float32(v_k / sd)) if sd != 0 else 0.
    """
    v = np.asarray(v, dtype=np.float32)
    k = v.shape[-1]
    if k % GROUP:
        raise ValueError("K must be a multiple of 16")
    g = v.reshape(v.shape[:-1] + (k // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    s = (amax / E2M1_MAX).astype(np.float32)  # IEEE float32 division
    s8 = formats.e4m3_encode(s)
    sd = formats.e4m3_decode(s8)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g / sd[..., None]).astype(np.float32)  # IEEE float32 division
    codes = formats.e2m1_encode(t)
    codes = np.where((sd == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(v.shape), s8


def pack_nibbles(codes):
    """Pack codes (..., K) two per byte: byte j = code[2j] | code[2j+1] << 4."""
    c = np.asarray(codes).astype(np.uint8)
    lo = c[..., 0::2] & np.uint8(0xF)
    hi = c[..., 1::2] & np.uint8(0xF)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of ``pack_nibbles``: bytes (..., K/2) -> codes (..., K)."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def smooth(x, smooth_factor):
    """x_s = float32(x) / float32(smooth_factor) along the last axis (IEEE division)."""
    x = np.asarray(x, dtype=np.float32)
    lam = np.asarray(smooth_factor, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (x / lam).astype(np.float32)


def quantize_act(x, smooth_factor, proj_down, hadamard_block=0):
    """Online activation path: smooth, optional rotation, group quantization, low-rank down-projection.

    ``x`` (M, K), ``smooth_factor`` (K,), ``proj_down`` (K, R) are float arrays
    holding bf16 values.  Returns ``qact (M, K/2) uint8``, ``ascales (K/16, M)
    uint8`` (e4m3 bytes) and ``lora_act (M, R) float64``.
    """
    xs = smooth(x, smooth_factor)
    v = fwht_blocks(xs, hadamard_block) if hadamard_block else xs
    codes, s8 = group_quantize(v)
    qact = pack_nibbles(codes)
    ascales = np.ascontiguousarray(s8.T)
    pd = np.asarray(proj_down, dtype=np.float64)
    lora = xs.astype(np.float64) @ pd if pd.shape[1] else np.zeros((xs.shape[0], 0))
    return qact, ascales, lora


def quantize_weight(w, smooth_factor, hadamard_block=0):
    """Offline weight path: fold smoothing (multiply), optional rotation, group quantization.

    ``w`` (N, K) holds bf16 values.  The product of two bf16 values is exact in
    float32.  Returns ``qweight (N, K/2) uint8`` and ``wscales (K/16, N) uint8``.
    """
    wq = (np.asarray(w, dtype=np.float32) * np.asarray(smooth_factor, dtype=np.float32)[None, :]).astype(np.float32)
    if hadamard_block:
        wq = fwht_blocks(wq, hadamard_block)
    codes, s8 = group_quantize(wq)
    return pack_nibbles(codes), np.ascontiguousarray(s8.T)


def int4_absmax(x, signed=True):
    """The rotate notes' INT4 absmax quantizer (float64): returns (q, scale, x_hat).

    scale = max|x| / qmax with qmax = 7 (signed) or 15 (unsigned); q is
    round-to-nearest of x / scale; x_hat = q * scale.
    """
    x = np.asarray(x, dtype=np.float64)
    qmax = 7.0 if signed else 15.0
    scale = np.max(np.abs(x)) / qmax
    q = np.rint(x / scale)
    q = np.clip(q, -8.0, 7.0) if signed else np.clip(q, 0.0, 15.0)
    return q, scale, q * scale
