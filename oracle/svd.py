"""Offline low-rank split of a smoothed weight (oracle, test infrastructure only).

Source: "SVDQuant W4A4" page, section "Overview": four-bit weights and
activations combined with a small low-rank branch that corrects part of the
quantization error, in an offline-quantized checkpoint whose tensors are
``proj_down (K, R)`` and ``proj_up (N, R)`` (section "Checkpoint contract").

What is computed (the plain definition, float64):

    W_s      = W * smooth_factor[None, :]             (the smoothed weight, exact)
    W_s      = U S V^T                                  (singular value decomposition)
    proj_up  = bf16( U[:, :R] * sqrt(S[:R]) )           (N, R)
    proj_down= bf16( V[:, :R] * sqrt(S[:R]) )           (K, R)
    residual = bf16( W_s - proj_up @ proj_down^T )     (N, K), from the stored bf16 factors

so that ``x_s @ proj_down @ proj_up^T`` is the best rank-R part of
``x_s @ W_s^T`` and the residual is what the 4-bit branch must carry.

Readings where the page is silent: the singular values are split evenly
between the two factors (square roots on both sides, so both stay in bf16's
range); the residual is taken against the rounded bf16 factors the checkpoint
stores, and rounded to bf16, the weight quantizer's input type (it is then
quantized with smooth_factor = 1, the smoothing being already inside it).
Singular vectors are unique only up to sign (and within repeated singular
values), so only products and singular values are compared.

Pins (``tests/test_oracle_svd.py``): an exactly rank-R weight is reproduced
with a residual at bf16 rounding level; the Eckart-Young identity
``||W_s - L||_F^2 = sum_{i > R} S_i^2``; orthonormal factors; the rank-0
case leaves the whole weight in the residual.
"""

import numpy as np

from . import formats


def smoothed(w, smooth_factor):
    """W * smooth_factor along K in float64 (exact for bf16 inputs)."""
    return np.asarray(w, dtype=np.float64) * np.asarray(smooth_factor, dtype=np.float64)[None, :]


def lowrank_split(w, smooth_factor, rank):
    """Returns (proj_down bf16 bits (K, R), proj_up bf16 bits (N, R), residual bf16 bits (N, K),
    singular values (min(N, K),) float64, the exact rank-R product (N, K) float64)."""
    ws = smoothed(w, smooth_factor)
    u, s, vt = np.linalg.svd(ws, full_matrices=False)
    r = int(rank)
    root = np.sqrt(s[:r])
    pu = formats.bf16_from_f64(u[:, :r] * root[None, :])
    pd = formats.bf16_from_f64(vt[:r].T * root[None, :])
    low = (u[:, :r] * s[None, :r]) @ vt[:r]
    stored = formats.bf16_to_f32(pu).astype(np.float64) @ formats.bf16_to_f32(pd).astype(np.float64).T
    resid = formats.bf16_from_f64(ws - stored)
    return pd, pu, resid, s, low
