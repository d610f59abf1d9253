"""Seeded sweep of layer shapes through ``svdq_linear`` and ``svdq_linear_mx`` (needs an MI355X).

The shapes are drawn, not picked: batch sizes on both sides of the weight-streaming limits (16 and
32 rows), ragged N and K, every rotation block the format allows, ranks 0..64, with and without a
bias.  Each call gets its workspace from the test, so besides y (within the output gates against
the oracle) the activation codes and scale bytes that the layer's own quantizer left in the
workspace are compared bit for bit with the oracle's (for small batches this is the K-split form of
the quantizer, which the standalone entry point does not run).
"""

import numpy as np
import pytest

import helpers as H
from oracle import linear as olinear
from oracle import mx as omx
from w4a4_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import w4a4_bit_quantized_amd as w
    w.load_library()
    return w


def _a256(v):
    return (v + 255) // 256 * 256


def _draw(i, mx):
    """Shape i of the sweep: (M, N, K, R, B, bias)."""
    rng = np.random.default_rng(9000 + 100 * int(mx) + i)
    band = rng.integers(0, 4)
    M = int([rng.integers(1, 17), rng.integers(17, 33), rng.integers(33, 300), rng.integers(300, 700)][band])
    if mx:
        B = int(rng.choice([0, 32]))
        K = 512 * int(rng.integers(1, 11)) if rng.random() < 0.5 else 128 * int(rng.integers(1, 24))
        N = 4 * int(rng.integers(1, 300))
    else:
        B = int(rng.choice([0, 16, 32, 64, 128]))
        step = max(B, 16)
        K = 512 * int(rng.integers(1, 11)) if rng.random() < 0.4 else step * int(rng.integers(1, 4096 // step + 1))
        N = int(rng.integers(1, 1200))
    if M <= 16 and rng.random() < 0.3:
        N = int(rng.integers(8193, 9000)) // 4 * 4  # the wide weight-streaming kernels
        K = min(K, 2048)
    R = int(rng.integers(0, 65))
    return M, N, K, R, B, bool(rng.random() < 0.5)


CASES = 16


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("i", range(CASES))
def test_linear_sweep(w4, i, mx):
    import torch
    M, N, K, R, B, bias = _draw(i, mx)
    print(f"sweep case {i} mx={mx}: M={M} N={N} K={K} R={R} B={B} bias={bias}", flush=True)
    lay = synth.make_layer("tiny", seed=31 * i + int(mx), M=M, K=K, N=N, R=R, B=B, wcs="uniform")
    f = synth.as_f32(lay)
    if mx:
        qw, ws = omx.quantize_weight_mx(f["w"], f["smooth_factor"], B)
        need = w4.svdq_linear_mx_workspace_bytes(M, K, R)
    else:
        qw, ws = H.oracle_weights(lay)
        need = w4.svdq_linear_workspace_bytes(M, K, R)
    layer = H.device_layer(lay, qw, ws)
    b_bits = H.seeded_bias(N, i) if bias else None
    if bias:
        layer["bias"] = H.to_dev_bf16(b_bits)
    work = torch.zeros(need, dtype=torch.uint8, device="cuda")
    x = H.to_dev_bf16(lay["x"])
    if mx:
        y = w4.svdq_linear_mx(x, layer, hadamard_block=B, workspace=work)
    else:
        y = w4.svdq_linear(x, layer, hadamard_block=B, workspace=work)
    torch.cuda.synchronize()

    ref_layer = dict(qweight=qw, wscales=ws, proj_down=f["proj_down"], proj_up=f["proj_up"],
                     smooth_factor=f["smooth_factor"], wcscales=f["wcscales"], wtscale=f["wtscale"],
                     bias=H.bf16_values(b_bits) if bias else None)
    if mx:
        _, y_ref, (q_ref, s_ref, _) = omx.svdq_linear_mx(f["x"], ref_layer, B)
    else:
        _, y_ref, (q_ref, s_ref, _) = olinear.svdq_linear(f["x"], ref_layer, B)

    # the workspace begins with the codes (M, K/2), then, 256-byte aligned, the scales (K/g, rows)
    ws_host = work.cpu().numpy()
    q_gpu = ws_host[: M * K // 2].reshape(M, K // 2)
    off = _a256(M * K // 2)
    s_gpu = ws_host[off: off + s_ref.size].reshape(s_ref.shape)
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(s_gpu != s_ref)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"
    H.assert_gates(H.from_dev_bf16_f64(y), y_ref, f"sweep case {i}")
