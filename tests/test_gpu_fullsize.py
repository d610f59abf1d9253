"""Whole-tensor parity at the workloads' full sizes (needs an MI355X).

For each of the five synthetic DiT-shaped workloads, in the launch configuration the benchmark
times, every byte of the GPU's qweight, wscales, qact and ascales is compared with the oracle's,
and every element of y from svdq_linear is checked against the oracle's float64 result: the
output gates ("SVDQuant W4A4" page, Checkpoint contract; relative Frobenius <= 5e-3, max |diff|
<= 2e-2 max |y|) and a per-element bound from the float32 accumulation of the GEMM, the
low-rank activations and the final bf16 rounding.  The same for the MXFP4 variant (rotate
notes, section 3.3) with its group-32 rotation.
"""

import numpy as np
import pytest

import helpers as H
from oracle import linear as olinear
from oracle import mx as omx
from oracle import quant as oquant
from w4a4_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import w4a4_bit_quantized_amd as w
    w.load_library()
    return w


def _equal_bytes(gpu, ref, what):
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    bad = np.argwhere(gpu != ref)
    assert bad.size == 0, f"{what}: {len(bad)} of {ref.size} bytes differ, first at {bad[:4].tolist()}"


def _lora_err_bound(xs, pd, K):
    """Per-element bound on the GPU's lora_act (bf16 hi + lo split of x_s, float32 accumulation)."""
    b = np.abs(xs.astype(np.float64)) @ np.abs(pd.astype(np.float64))
    return (2.0 ** -18 + (2 * K // 32 + 64) * 2.0 ** -24) * b


def _check_y(y_gpu, y_ref, a_abs, w_abs, col, lora, lora_err, pu, K, R, what):
    """Gates, then |y_gpu - y_ref| <= bf16 rounding + float32 accumulation + low-rank error."""
    rel, mx = H.assert_gates(y_gpu, y_ref, what)
    pu_abs = np.abs(pu.astype(np.float64))
    acc = (a_abs @ w_abs.T) * np.abs(col)[None, :]
    if R:
        acc += np.abs(lora) @ pu_abs.T
    lim = 2.0 ** -8 * np.abs(y_ref) + (K // 4 + 4 * R + 64) * 2.0 ** -24 * acc + 1e-30
    if R:
        lim += lora_err @ pu_abs.T
    err = np.abs(y_gpu - y_ref)
    worst = np.unravel_index(np.argmax(err - lim), err.shape)
    assert np.all(err <= lim), f"{what}: per-element bound broken at {worst}: {err[worst]:.3e} > {lim[worst]:.3e}"
    return rel, mx


@pytest.mark.parametrize("name", synth.ORDER)
def test_full_size_whole_tensors(w4, name):
    import torch
    lay = synth.make_layer(name, seed=0)
    M, N, K, R, B = lay["M"], lay["N"], lay["K"], lay["R"], lay["B"]
    f = synth.as_f32(lay)
    print(f"\n{name}: M={M} K={K} N={N} R={R} B={B}", flush=True)
    # offline weights on the GPU at full size: every byte
    qw_d, ws_d = w4.svdq_quantize_weight(H.to_dev_bf16(lay["w"]), H.to_dev_bf16(lay["smooth_factor"]), B)
    qw_ref, ws_ref = oquant.quantize_weight(f["w"], f["smooth_factor"], B)
    torch.cuda.synchronize()
    _equal_bytes(qw_d.cpu().numpy(), qw_ref, "qweight")
    _equal_bytes(ws_d.cpu().numpy(), ws_ref, "wscales")
    # the activation quantizer at full size: every byte, lora_act within its bound everywhere
    x = H.to_dev_bf16(lay["x"])
    lam, pd = H.to_dev_bf16(lay["smooth_factor"]), H.to_dev_bf16(lay["proj_down"])
    qa, sa, lo = w4.svdq_quantize_act(x, lam, pd, B)
    qa_ref, sa_ref, lo_ref = oquant.quantize_act(f["x"], f["smooth_factor"], f["proj_down"], B)
    torch.cuda.synchronize()
    _equal_bytes(qa.cpu().numpy(), qa_ref, "qact")
    _equal_bytes(sa.cpu().numpy(), sa_ref, "ascales")
    xs = oquant.smooth(f["x"], f["smooth_factor"])
    lora_err = _lora_err_bound(xs, f["proj_down"], K)
    assert np.all(np.abs(lo.cpu().numpy().astype(np.float64) - lo_ref) <= lora_err + 1e-30), "lora_act"
    del qa, sa, lo
    # the whole layer at full size (the benchmark's call): every element of y
    layer = H.device_layer(lay, np.zeros((1, 1), np.uint8), np.zeros((1, 1), np.uint8))
    layer["qweight"], layer["wscales"] = qw_d, ws_d
    y = w4.svdq_linear(x, layer, hadamard_block=B)
    torch.cuda.synchronize()
    y_gpu = H.from_dev_bf16_f64(y)
    del y
    a = olinear.dequant(qa_ref, sa_ref)
    wd = olinear.dequant(qw_ref, ws_ref)
    col = f["wcscales"].astype(np.float64) * float(f["wtscale"][0])
    y_ref = (a @ wd.T) * col[None, :]
    if R:
        y_ref += lo_ref @ f["proj_up"].astype(np.float64).T
    rel, mx = _check_y(y_gpu, y_ref, np.abs(a), np.abs(wd), col, lo_ref, lora_err, f["proj_up"], K, R, name)
    del a, wd
    ref_unq = olinear.unquantized_reference(f["x"], f["w"], f["proj_down"], f["proj_up"], f["smooth_factor"],
                                            f["wcscales"], f["wtscale"])
    rel_unq = np.linalg.norm(y_gpu - ref_unq) / np.linalg.norm(ref_unq)
    print(f"{name}: all {M * N} outputs within the gates (rel_fro={rel:.2e}, max={mx:.2e}) and the "
          f"per-element bound; {qa_ref.size + sa_ref.size} activation and {qw_ref.size + ws_ref.size} weight "
          f"bytes bit-exact; vs the unquantized linear (reported, not gated) rel_fro={rel_unq:.3f}")


@pytest.mark.parametrize("name", synth.ORDER)
def test_full_size_whole_tensors_mx(w4, name):
    import torch
    lay = synth.make_layer(name, seed=0)
    M, N, K, R = lay["M"], lay["N"], lay["K"], lay["R"]
    B = 32
    f = synth.as_f32(lay)
    print(f"\n{name} (MXFP4, rotation 32): M={M} K={K} N={N} R={R}", flush=True)
    qw_d, sw_d = w4.svdq_quantize_weight_mx(H.to_dev_bf16(lay["w"]), H.to_dev_bf16(lay["smooth_factor"]), B)
    qw_ref, sw_ref = omx.quantize_weight_mx(f["w"], f["smooth_factor"], B)
    torch.cuda.synchronize()
    _equal_bytes(qw_d.cpu().numpy(), qw_ref, "qweight (mx)")
    _equal_bytes(sw_d.cpu().numpy(), sw_ref, "wscales (mx)")
    x = H.to_dev_bf16(lay["x"])
    lam, pd = H.to_dev_bf16(lay["smooth_factor"]), H.to_dev_bf16(lay["proj_down"])
    qa, sa, lo = w4.svdq_quantize_act_mx(x, lam, pd, B)
    qa_ref, sa_ref, lo_ref = omx.quantize_act_mx(f["x"], f["smooth_factor"], f["proj_down"], B)
    torch.cuda.synchronize()
    _equal_bytes(qa.cpu().numpy(), qa_ref, "qact (mx)")
    _equal_bytes(sa.cpu().numpy(), sa_ref, "ascales (mx)")
    xs = oquant.smooth(f["x"], f["smooth_factor"])
    lora_err = _lora_err_bound(xs, f["proj_down"], K)
    assert np.all(np.abs(lo.cpu().numpy().astype(np.float64) - lo_ref) <= lora_err + 1e-30), "lora_act (mx)"
    del qa, sa, lo
    layer = H.device_layer(lay, np.zeros((1, 1), np.uint8), np.zeros((1, 1), np.uint8))
    layer["qweight"], layer["wscales"] = qw_d, sw_d
    y = w4.svdq_linear_mx(x, layer, hadamard_block=B)
    torch.cuda.synchronize()
    y_gpu = H.from_dev_bf16_f64(y)
    del y
    a = omx.dequant_mx(qa_ref, sa_ref, M)
    wd = omx.dequant_mx(qw_ref, sw_ref, N)
    col = f["wcscales"].astype(np.float64) * float(f["wtscale"][0])
    y_ref = (a @ wd.T) * col[None, :]
    if R:
        y_ref += lo_ref @ f["proj_up"].astype(np.float64).T
    rel, mx = _check_y(y_gpu, y_ref, np.abs(a), np.abs(wd), col, lo_ref, lora_err, f["proj_up"], K, R, name + " mx")
    print(f"{name} mx: all {M * N} outputs within the gates (rel_fro={rel:.2e}, max={mx:.2e}) and the per-element "
          f"bound; codes and E8M0 bytes bit-exact")
