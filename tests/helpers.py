"""Helpers shared by the GPU tests: device transfer of synthetic layers and tolerance checks."""

import numpy as np

from oracle import linear as olinear
from oracle import quant as oquant
from w4a4_bit_quantized_amd import synth

# Output gates (relative Frobenius and per-element max, relative to max |y_ref|).
REL_FRO_GATE = 5e-3
MAX_ABS_GATE = 2e-2


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_u8(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def from_dev_bf16_f64(t):
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def oracle_weights(lay):
    """The checkpoint's offline-quantized weights, made by the oracle from the synthetic W."""
    f = synth.as_f32(lay)
    qw, ws = oquant.quantize_weight(f["w"], f["smooth_factor"], lay["B"])
    return qw, ws


def device_layer(lay, qweight, wscales, device="cuda"):
    return dict(
        qweight=to_dev_u8(qweight, device), wscales=to_dev_u8(wscales, device),
        proj_down=to_dev_bf16(lay["proj_down"], device), proj_up=to_dev_bf16(lay["proj_up"], device),
        smooth_factor=to_dev_bf16(lay["smooth_factor"], device), wcscales=to_dev_bf16(lay["wcscales"], device),
        wtscale=to_dev_bf16(lay["wtscale"], device),
    )


def oracle_linear_rows(lay, qweight, wscales, rows=None):
    """Oracle output for selected rows (every row is independent)."""
    f = synth.as_f32(lay)
    x = f["x"] if rows is None else f["x"][rows]
    layer = dict(qweight=qweight, wscales=wscales, proj_down=f["proj_down"], proj_up=f["proj_up"],
                 smooth_factor=f["smooth_factor"], wcscales=f["wcscales"], wtscale=f["wtscale"])
    yb, y, parts = olinear.svdq_linear(x, layer, lay["B"])
    return yb, y, parts


def gate_errors(y_gpu, y_ref):
    """(relative Frobenius error, max |diff| / max |y_ref|) in float64."""
    d = y_gpu - y_ref
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mref = np.abs(y_ref).max()
    mx = np.abs(d).max() / mref if mref > 0 else np.abs(d).max()
    return float(rel), float(mx)


def assert_gates(y_gpu, y_ref, what=""):
    rel, mx = gate_errors(y_gpu, y_ref)
    assert rel <= REL_FRO_GATE, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO_GATE}"
    assert mx <= MAX_ABS_GATE, f"{what}: max abs error {mx:.3e} * max|y| > {MAX_ABS_GATE}"
    return rel, mx


def accumulation_bound(qact, ascales, lora, qweight, wscales, proj_up, wcscales, wtscale, n_adds):
    """Per-element bound on the float32 accumulation error of the GPU GEMM:
    n_adds * 2^-24 * (|A| |W|^T |c| + |L| |P|^T)."""
    a = np.abs(olinear.dequant(qact, ascales))
    w = np.abs(olinear.dequant(qweight, wscales))
    c = np.abs(np.asarray(wcscales, np.float64) * float(np.asarray(wtscale, np.float64).reshape(-1)[0]))
    b = (a @ w.T) * c[None, :]
    if np.asarray(proj_up).shape[1]:
        b = b + np.abs(np.asarray(lora, np.float64)) @ np.abs(np.asarray(proj_up, np.float64)).T
    return n_adds * 2.0 ** -24 * b


def seeded_bias(N, seed):
    """A bf16 bias (N,) in U[-4, 4] (bit patterns), seeded."""
    from oracle import formats
    return formats.bf16_from_f64(np.random.default_rng(1000 + seed).uniform(-4.0, 4.0, N))


def bf16_values(bits):
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
