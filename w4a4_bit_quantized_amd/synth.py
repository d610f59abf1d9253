"""Seeded synthetic inputs for the W4A4 linear layer.

This module only draws random tensors of the workloads' shapes and
distributions and rounds them to bf16; it holds none of the method's
arithmetic (no smoothing, rotation, quantization or matmul).  The same arrays
feed the GPU path and the CPU oracle, so parity never depends on the
generator.

Workloads (DiT-shaped linears; the pages publish no dataset or benchmark for
this layer, so these synthetic tensors are the workload):

  tiny              M=64,   K=256,   N=256,   R=32  x~N(0,1), 4 outlier channels x20,
                                                    wcscales = 1, no rotation
  dit_attn_proj     M=4096, K=3072,  N=3072,  R=32  x~N(0,1), 1% outlier channels x20
  dit_mlp_up        M=4096, K=3072,  N=12288, R=32  as dit_attn_proj (compute-bound headline)
  dit_mlp_down_rot  M=4096, K=12288, N=3072,  R=32  x=GELU(N(0,1)), 0.5% outliers x30,
                                                    Hadamard block 128 folded into W
  skinny            M=16,   K=5120,  N=13824, R=32  as dit_attn_proj (weight streaming)

Common draws: W ~ N(0, 1/K) (variance 1/K), proj_down ~ N(0, 1/K),
proj_up ~ N(0, 1/R), smooth_factor ~ U[0.5, 2], wcscales ~ U[0.9, 1.1] (ones
for "tiny"), wtscale = 1.  Outlier channel count is round(fraction * K).
Draw order from numpy.random.default_rng(seed): x, outlier channels, W,
proj_down, proj_up, smooth_factor, wcscales.  float32 draws are rounded to
bf16 by round-to-nearest-even.  GELU uses the exact erf form in float64.
"""

import math

import numpy as np

WORKLOADS = {
    "tiny": dict(M=64, K=256, N=256, R=32, x="normal", n_out=4, out_scale=20.0, wcs="ones", B=0),
    "dit_attn_proj": dict(M=4096, K=3072, N=3072, R=32, x="normal", out_frac=0.01, out_scale=20.0, wcs="uniform", B=0),
    "dit_mlp_up": dict(M=4096, K=3072, N=12288, R=32, x="normal", out_frac=0.01, out_scale=20.0, wcs="uniform", B=0),
    "dit_mlp_down_rot": dict(M=4096, K=12288, N=3072, R=32, x="gelu", out_frac=0.005, out_scale=30.0, wcs="uniform", B=128),
    "skinny": dict(M=16, K=5120, N=13824, R=32, x="normal", out_frac=0.01, out_scale=20.0, wcs="uniform", B=0),
}
ORDER = ["tiny", "dit_attn_proj", "dit_mlp_up", "dit_mlp_down_rot", "skinny"]


def to_bf16_bits(a):
    """Round float32 values to bf16 (nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = r.astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r).astype(np.uint16)


def bits_to_f32(bits):
    """Widen bf16 bit patterns to float32."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gelu_erf(z):
    z = np.asarray(z, dtype=np.float64)
    try:
        from scipy.special import erf
        e = erf(z / math.sqrt(2.0))
    except ImportError:  # pragma: no cover - scipy is present in this image
        e = np.vectorize(math.erf)(z / math.sqrt(2.0))
    return 0.5 * z * (1.0 + e)


def n_outliers(spec):
    if "n_out" in spec:
        return int(spec["n_out"])
    return int(round(spec["out_frac"] * spec["K"]))


def make_layer(name=None, seed=0, M=None, K=None, N=None, R=None, B=None, **overrides):
    """Draw one workload's tensors.

    ``name`` selects a workload from WORKLOADS; keyword sizes override it (used
    for small and ragged test shapes with the same distributions).  Returns a
    dict of bf16 bit arrays (uint16): x (M,K), w (N,K), proj_down (K,R),
    proj_up (N,R), smooth_factor (K,), wcscales (N,), wtscale (1,), plus the
    sizes and the rotation block ``B`` and the outlier channel indices.
    """
    spec = dict(WORKLOADS[name or "tiny"])
    for key, val in (("M", M), ("K", K), ("N", N), ("R", R), ("B", B)):
        if val is not None:
            spec[key] = val
    spec.update(overrides)
    M_, K_, N_, R_ = spec["M"], spec["K"], spec["N"], spec["R"]
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M_, K_), dtype=np.float32)
    if spec["x"] == "gelu":
        x = _gelu_erf(z).astype(np.float32)
    else:
        x = z
    n_out = min(n_outliers(spec), K_)
    idx = np.sort(rng.choice(K_, n_out, replace=False)) if n_out else np.zeros(0, dtype=np.int64)
    if n_out:
        x[:, idx] *= np.float32(spec["out_scale"])
    w = rng.standard_normal((N_, K_), dtype=np.float32) * np.float32(1.0 / math.sqrt(K_))
    pd = rng.standard_normal((K_, R_), dtype=np.float32) * np.float32(1.0 / math.sqrt(K_))
    pu = rng.standard_normal((N_, R_), dtype=np.float32) * np.float32(1.0 / math.sqrt(max(R_, 1)))
    lam = rng.uniform(0.5, 2.0, K_).astype(np.float32)
    if spec.get("wcs", "uniform") == "ones":
        wcs = np.ones(N_, dtype=np.float32)
    else:
        wcs = rng.uniform(0.9, 1.1, N_).astype(np.float32)
    wts = np.ones(1, dtype=np.float32)
    return dict(
        name=name, seed=seed, M=M_, K=K_, N=N_, R=R_, B=int(spec["B"]), outlier_channels=idx,
        x=to_bf16_bits(x), w=to_bf16_bits(w), proj_down=to_bf16_bits(pd), proj_up=to_bf16_bits(pu),
        smooth_factor=to_bf16_bits(lam), wcscales=to_bf16_bits(wcs), wtscale=to_bf16_bits(wts),
    )


def as_f32(layer):
    """float32 views of a layer's bf16 tensors (for the CPU oracle)."""
    keys = ("x", "w", "proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale")
    return {k: bits_to_f32(layer[k]) for k in keys}
