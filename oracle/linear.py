"""Block-scaled W4A4 GEMM with the low-rank correction (oracle, test infrastructure only).

Source: "SVDQuant W4A4" page.  "Runtime support": BF16 input, an NVFP4 GEMM,
then the BF16 rank correction; "Checkpoint contract": ``proj_up (N, R)``,
``wcscales (N,)`` (per-output correction, ones when unused) and ``wtscale
(1,)``.  "Overview": 4-bit weights and activations plus a small low-rank branch.

What is computed (plain definition, float64, one final rounding to bf16):

    A[m, k]  = e2m1(qact[m, k])    * e4m3(ascales[k // 16, m])
    Wd[n, k] = e2m1(qweight[n, k]) * e4m3(wscales[k // 16, n])
    y[m, n]  = bf16( (A @ Wd^T)[m, n] * wcscales[n] * wtscale
                     + (lora_act @ proj_up^T)[m, n] + bias[n] )

Every A and Wd entry has at most 6 significant bits and every product at most
12, so the dequantized operands and products are exact in float64; the sum is
the float64 BLAS sum.  Readings where the pages are silent: ``wcscales`` and
``wtscale`` multiply the quantized product only, not the low-rank term; the
optional ``bias (N,)`` (bf16) that the rotate notes' linear wrapper hands to the
quantized method (section 3.2, ``apply(layer, x, bias)``) is a plain per-output
offset added before the single rounding, scaled by nothing.

Pins: a pure-Python triple loop over the block-scaled sum
sum_g sa * sw * sum_{k in g} qa * qw on tiny shapes; the identity-quantizer
reduction to x W^T * wcscales * wtscale + low-rank term (see
``tests/test_oracle_linear.py``).
"""

import numpy as np

from . import formats, quant


def dequant(packed, scales_t):
    """Dequantize packed codes (rows, K/2) with scales (K/16, rows) -> float64 (rows, K)."""
    codes = quant.unpack_nibbles(packed)
    vals = formats.e2m1_decode(codes).astype(np.float64)
    sd = formats.e4m3_decode(np.asarray(scales_t).T).astype(np.float64)  # (rows, K/16)
    return vals * np.repeat(sd, quant.GROUP, axis=1)


def gemm_lowrank(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, bias=None):
    """Quantized product plus epilogue.  Returns (y_bits (M, N) uint16 bf16, y_f64 before rounding)."""
    a = dequant(qact, ascales)
    wd = dequant(qweight, wscales)
    acc = a @ wd.T
    col = np.asarray(wcscales, dtype=np.float64) * np.float64(np.asarray(wtscale, dtype=np.float64).reshape(-1)[0])
    y = acc * col[None, :]
    pu = np.asarray(proj_up, dtype=np.float64)
    if pu.shape[1]:
        y = y + np.asarray(lora_act, dtype=np.float64) @ pu.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return formats.bf16_from_f64(y), y


def svdq_linear(x, layer, hadamard_block=0):
    """The whole online layer: activation quantization followed by ``gemm_lowrank``.

    ``layer`` holds ``qweight, wscales, proj_down, proj_up, smooth_factor,
    wcscales, wtscale`` and optionally ``bias``.  Returns (y_bits, y_f64,
    (qact, ascales, lora_act)).
    """
    qact, ascales, lora = quant.quantize_act(x, layer["smooth_factor"], layer["proj_down"], hadamard_block)
    yb, y = gemm_lowrank(qact, ascales, lora, layer["qweight"], layer["wscales"], layer["proj_up"],
                         layer["wcscales"], layer["wtscale"], layer.get("bias"))
    return yb, y, (qact, ascales, lora)


def unquantized_reference(x, w, proj_down, proj_up, smooth_factor, wcscales, wtscale, bias=None):
    """Ungated comparison: the same layer with the quantizer replaced by the identity (float64).

    x_s R^T (W diag(smooth) R^T)^T = x W^T, so this is
    x W^T * wcscales * wtscale + (x / smooth) proj_down proj_up^T.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    col = np.asarray(wcscales, dtype=np.float64) * np.float64(np.asarray(wtscale, dtype=np.float64).reshape(-1)[0])
    y = (x64 @ w64.T) * col[None, :]
    pd = np.asarray(proj_down, dtype=np.float64)
    if pd.shape[1]:
        xs = x64 / np.asarray(smooth_factor, dtype=np.float64)[None, :]
        y = y + (xs @ pd) @ np.asarray(proj_up, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
