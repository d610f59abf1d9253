"""GPU parity of the MXFP4 variant (rotate notes, section 3.3: FP-Quant mxfp4 with a group-32
rotation) against the CPU oracle ``oracle/mx.py`` (needs an MI355X).

Bars as for the nvfp4 path: codes and E8M0 scale bytes bit-exact (including the zero padding
of the activation scale rows), lora_act within the float32 accumulation bound of the hi/lo
bf16 split, bf16 outputs within relative Frobenius 5e-3 and max |diff| 2e-2 max|y_ref| plus
a per-element float32 accumulation bound.  Every call goes through the C ABI.
"""

import numpy as np
import pytest

import helpers as H
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


def _lay(M, K, N, R, B, seed):
    return synth.make_layer("tiny", seed=seed, M=M, K=K, N=N, R=R, B=B, wcs="uniform")


def _mx_weights(lay):
    f = synth.as_f32(lay)
    return omx.quantize_weight_mx(f["w"], f["smooth_factor"], lay["B"])


def _lora_bound(xs, pd, K):
    b = np.abs(xs.astype(np.float64)) @ np.abs(pd.astype(np.float64))
    return (2.0 ** -18 + (2 * K // 32 + 64) * 2.0 ** -24) * b + 1e-30


@pytest.mark.parametrize("M,K,R,B", [(16, 128, 32, 32), (37, 256, 8, 0), (3, 64, 0, 32), (130, 512, 64, 32),
                                     (64, 1024, 16, 0), (5, 96, 32, 32)])
def test_quantize_act_mx_parity(w4, M, K, R, B):
    import torch
    lay = _lay(M, K, 64, R, B, seed=M + K)
    f = synth.as_f32(lay)
    qa, sa, lo = w4.svdq_quantize_act_mx(H.to_dev_bf16(lay["x"]), H.to_dev_bf16(lay["smooth_factor"]),
                                         H.to_dev_bf16(lay["proj_down"]), B)
    torch.cuda.synchronize()
    q_ref, s_ref, l_ref = omx.quantize_act_mx(f["x"], f["smooth_factor"], f["proj_down"], B)
    assert sa.shape == s_ref.shape
    bad = np.argwhere(qa.cpu().numpy() != q_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(sa.cpu().numpy() != s_ref)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"
    if R:
        xs = oquant.smooth(f["x"], f["smooth_factor"])
        err = np.abs(lo.cpu().numpy().astype(np.float64) - l_ref)
        assert np.all(err <= _lora_bound(xs, f["proj_down"], K))


@pytest.mark.parametrize("N,K,B", [(8, 64, 0), (33, 96, 32), (256, 1024, 32), (130, 512, 0)])
def test_quantize_weight_mx_parity(w4, N, K, B):
    import torch
    lay = _lay(4, K, N, 8, B, seed=N + K)
    qw, sw = w4.svdq_quantize_weight_mx(H.to_dev_bf16(lay["w"]), H.to_dev_bf16(lay["smooth_factor"]), B)
    torch.cuda.synchronize()
    q_ref, s_ref = _mx_weights(lay)
    assert np.array_equal(qw.cpu().numpy(), q_ref)
    assert np.array_equal(sw.cpu().numpy(), s_ref)


def _accumulation_bound(qa, sa, lo, qw, sw, pu, wcs, wts, M, N, n_adds):
    a = np.abs(omx.dequant_mx(qa, sa, M))
    w = np.abs(omx.dequant_mx(qw, sw, N))
    c = np.abs(np.asarray(wcs, np.float64) * float(np.asarray(wts, np.float64).reshape(-1)[0]))
    b = (a @ w.T) * c[None, :]
    if np.asarray(pu).shape[1]:
        b = b + np.abs(np.asarray(lo, np.float64)) @ np.abs(np.asarray(pu, np.float64)).T
    return n_adds * 2.0 ** -24 * b


def _check_gemm_mx(w4, lay, bias=False):
    import torch
    f = synth.as_f32(lay)
    M, N, K = lay["M"], lay["N"], lay["K"]
    qw, sw = _mx_weights(lay)
    qa, sa, lo = omx.quantize_act_mx(f["x"], f["smooth_factor"], f["proj_down"], lay["B"])
    lo32 = lo.astype(np.float32)
    b_bits = H.seeded_bias(N, M) if bias else None
    y = w4.svdq_gemm_lowrank_mx(H.to_dev_u8(qa), H.to_dev_u8(sa), torch.from_numpy(lo32).cuda(), H.to_dev_u8(qw),
                                H.to_dev_u8(sw), H.to_dev_bf16(lay["proj_up"]), H.to_dev_bf16(lay["wcscales"]),
                                H.to_dev_bf16(lay["wtscale"]), bias=H.to_dev_bf16(b_bits) if bias else None)
    torch.cuda.synchronize()
    b_f = H.bf16_values(b_bits) if bias else None
    _, y_ref = omx.gemm_lowrank_mx(qa, sa, lo32, qw, sw, f["proj_up"], f["wcscales"], f["wtscale"], b_f)
    y_gpu = H.from_dev_bf16_f64(y)
    H.assert_gates(y_gpu, y_ref, "gemm_mx")
    bound = _accumulation_bound(qa, sa, lo32, qw, sw, f["proj_up"], f["wcscales"], f["wtscale"], M, N,
                                n_adds=K // 32 + 4 * lay["R"] + 64)
    err = np.abs(y_gpu - y_ref)
    lim = 2.0 ** -8 * np.abs(y_ref) + bound + 1e-30
    if bias:  # one more float32 addition
        lim = lim + 2.0 ** -23 * (np.abs(b_f)[None, :] + np.abs(y_ref))
    assert np.all(err <= lim), f"per-element bound broken: worst excess {np.max(err - lim):.3e}"
    return y_gpu


@pytest.mark.parametrize("M,N,K,R", [(64, 256, 256, 32), (130, 200, 384, 8), (37, 68, 128, 0), (3, 40, 256, 64),
                                     (300, 520, 640, 32), (512, 512, 1024, 16)])
def test_gemm_lowrank_mx_parity(w4, M, N, K, R):
    _check_gemm_mx(w4, _lay(M, K, N, R, 32, seed=M * 7 + N))


@pytest.mark.parametrize("tile", ["4x4x2x2", "2x4x4x2", "2x2x2x2", "2x2x4x4"])
@pytest.mark.parametrize("N", [520, 516])
def test_gemm_mx_each_tile(w4, tile, N, hooks):
    """Each MX tile layout (2x2x4x4: one wave per SIMD with register prefetch)
    on a ragged shape with an odd number of K-steps, with y rows that are whole 16-byte runs
    (N = 520) and that are not (N = 516)."""
    hooks.setenv("W4A4_GEMM_TILE", tile)
    _check_gemm_mx(w4, _lay(300, 640, N, 32, 0, seed=41))


@pytest.mark.parametrize("M,N,K,R", [(16, 13824, 5120, 32), (1, 64, 512, 32), (5, 300, 1024, 8), (16, 1000, 3072, 64),
                                     (7, 132, 2560, 0), (16, 8196, 5120, 16), (13, 68, 4608, 33), (3, 4, 512, 1)])
def test_gemm_mx_weight_streaming(w4, M, N, K, R, hooks):
    """Batches of at most 16 rows with K a multiple of 512 up to 5120 stream the weights through the
    scaled 16x16x128 FP4 instruction (K = 5120 specialised, ragged N, every rank form): against
    the oracle, and against the tiled kernel (W4A4_SKINNY_PATH=tiled) within the same gates."""
    lay = _lay(M, K, N, R, 0, seed=M * 11 + N)
    y_stream = _check_gemm_mx(w4, lay)
    hooks.setenv("W4A4_SKINNY_PATH", "tiled")
    y_tiled = _check_gemm_mx(w4, lay)
    H.assert_gates(y_stream, y_tiled, "streaming vs tiled MX GEMM")


@pytest.mark.parametrize("M,N,K,R", [(16, 1028, 5120, 32), (2, 260, 1536, 0)])
def test_gemm_mx_weight_streaming_bias(w4, M, N, K, R, hooks):
    """The bias through the weight-streaming MX GEMM (added after the low-rank term, before the
    single rounding), against the oracle and the tiled kernel."""
    lay = _lay(M, K, N, R, 0, seed=N + R)
    y_stream = _check_gemm_mx(w4, lay, bias=True)
    hooks.setenv("W4A4_SKINNY_PATH", "tiled")
    y_tiled = _check_gemm_mx(w4, lay, bias=True)
    H.assert_gates(y_stream, y_tiled, "streaming vs tiled MX GEMM with bias")


@pytest.mark.parametrize("M,N,K,R,B", [(16, 2048, 5120, 32, 32), (4, 640, 1024, 16, 0)])
def test_linear_mx_small_batch(w4, M, N, K, R, B):
    """The MX layer at small batches: the K-split quantizer's partial low-rank sums meet in the
    weight-streaming GEMM's epilogue."""
    import torch
    lay = _lay(M, K, N, R, B, seed=M + K)
    qw, sw = _mx_weights(lay)
    y = w4.svdq_linear_mx(H.to_dev_bf16(lay["x"]), H.device_layer(lay, qw, sw), hadamard_block=B)
    torch.cuda.synchronize()
    f = synth.as_f32(lay)
    layer = dict(qweight=qw, wscales=sw, proj_down=f["proj_down"], proj_up=f["proj_up"],
                 smooth_factor=f["smooth_factor"], wcscales=f["wcscales"], wtscale=f["wtscale"])
    _, y_ref, _ = omx.svdq_linear_mx(f["x"], layer, B)
    H.assert_gates(H.from_dev_bf16_f64(y), y_ref, "svdq_linear_mx small batch")


@pytest.mark.parametrize("tile", ["4x4x2x2", "2x2x4x4"])
@pytest.mark.parametrize("K", [128, 256, 384])
def test_gemm_mx_few_k_steps(w4, tile, K, hooks):
    """Fewer K-steps than pipeline stages."""
    hooks.setenv("W4A4_GEMM_TILE", tile)
    _check_gemm_mx(w4, _lay(260, K, 264, 16, 0, seed=K))


@pytest.mark.parametrize("M,N,K,R,B", [(64, 256, 256, 32, 32), (37, 68, 384, 16, 0), (16, 200, 2048, 32, 32),
                                       (5, 132, 512, 8, 32)])
def test_linear_mx_parity(w4, M, N, K, R, B):
    import torch
    lay = _lay(M, K, N, R, B, seed=3 + M)
    qw, sw = _mx_weights(lay)
    y = w4.svdq_linear_mx(H.to_dev_bf16(lay["x"]), H.device_layer(lay, qw, sw), hadamard_block=B)
    torch.cuda.synchronize()
    f = synth.as_f32(lay)
    layer = dict(qweight=qw, wscales=sw, proj_down=f["proj_down"], proj_up=f["proj_up"],
                 smooth_factor=f["smooth_factor"], wcscales=f["wcscales"], wtscale=f["wtscale"])
    _, y_ref, _ = omx.svdq_linear_mx(f["x"], layer, B)
    H.assert_gates(H.from_dev_bf16_f64(y), y_ref, "svdq_linear_mx")


@pytest.mark.parametrize("tile", ["4x4x2x2", "2x2x4x4", "2x2x2x2"])
def test_gemm_mx_bias(w4, tile, hooks):
    """The optional bias (rotate notes, section 3.2) through the MX GEMM's bias entry point."""
    hooks.setenv("W4A4_GEMM_TILE", tile)
    _check_gemm_mx(w4, _lay(300, 640, 520, 32, 0, seed=43), bias=True)


def test_linear_mx_bias(w4):
    import torch
    lay = _lay(64, 512, 264, 32, 32, seed=5)
    qw, sw = _mx_weights(lay)
    layer = H.device_layer(lay, qw, sw)
    b_bits = H.seeded_bias(264, 64)
    layer["bias"] = H.to_dev_bf16(b_bits)
    y = w4.svdq_linear_mx(H.to_dev_bf16(lay["x"]).reshape(4, 16, 512), layer, hadamard_block=32)
    torch.cuda.synchronize()
    f = synth.as_f32(lay)
    ref_layer = dict(qweight=qw, wscales=sw, bias=H.bf16_values(b_bits), proj_down=f["proj_down"],
                     proj_up=f["proj_up"], smooth_factor=f["smooth_factor"], wcscales=f["wcscales"],
                     wtscale=f["wtscale"])
    _, y_ref, _ = omx.svdq_linear_mx(f["x"], ref_layer, 32)
    assert tuple(y.shape) == (4, 16, 264)
    H.assert_gates(H.from_dev_bf16_f64(y.reshape(64, 264)), y_ref, "svdq_linear_mx with bias")


@pytest.mark.parametrize("B", [0, 32])
def test_quantize_act_mx_special_values(w4, B):
    """E8M0 edge cases, bit-exact: all-zero and negative-zero blocks (exponent clamped to -127),
    block maxima exactly at 6 * 2^k (no round-up) and one bf16 step above it, subnormal-range
    maxima, and maxima near the largest bf16 (exponent near +127)."""
    import torch
    M, K = 12, 256
    lay = _lay(M, K, 64, 8, B, seed=77)
    x = synth.bits_to_f32(lay["x"]).copy()
    x[0, :] = 0.0
    x[1, :32] = -0.0
    x[1, 32:64] = 0.0
    x[2, :32] = np.float32(6.0 * 2.0 ** 3)          # amax / 6 is exactly 2^3
    x[3, :32] = np.float32(6.0 * 2.0 ** -20)
    x[4, :32] = synth.bits_to_f32(synth.to_bf16_bits(np.float32([6.0 * 2.0 ** 3 * (1 + 2.0 ** -7)])))[0]  # next bf16
    x[5, :32] = np.float32(2.0 ** -133)              # subnormal: amax / 6 far below 2^-127
    x[6, :32] = np.float32(1e-38)
    # exponent near the top of the E8M0 range (with the rotation, small enough that the 32-point
    # sums stay finite: blocks whose rotated values overflow have no defined scale)
    x[7, :32] = np.float32(3.0e38 if B == 0 else 5.0e36)
    x[8, ::2] = -x[8, ::2]
    x[9, 64:96] = np.float32(-5.0e37 if B == 0 else -5.0e36)
    lay["x"] = synth.to_bf16_bits(x)
    lay["smooth_factor"] = synth.to_bf16_bits(np.ones(K, np.float32))
    lay["proj_down"] = synth.to_bf16_bits(np.zeros((K, 8), np.float32))
    f = synth.as_f32(lay)
    qa, sa, lo = w4.svdq_quantize_act_mx(H.to_dev_bf16(lay["x"]), H.to_dev_bf16(lay["smooth_factor"]),
                                         H.to_dev_bf16(lay["proj_down"]), B)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = omx.quantize_act_mx(f["x"], f["smooth_factor"], f["proj_down"], B)
    assert np.array_equal(sa.cpu().numpy(), s_ref)
    assert np.array_equal(qa.cpu().numpy(), q_ref)
    assert s_ref[0, 0] == 0 and s_ref[0, 2] == 127 + 3 and s_ref[0, 4] == 127 + 4 if B == 0 else True


def test_linear_mx_in_hip_graph(w4):
    """svdq_linear_mx captured once in a HIP graph and replayed four times, with eager launches on
    another input between the replays: every replay is bit-identical to the eager call."""
    import torch
    lay = _lay(600, 1024, 1040, 32, 32, seed=77)
    qw, sw = _mx_weights(lay)
    layer = H.device_layer(lay, qw, sw)
    x = H.to_dev_bf16(lay["x"])
    x_other = H.to_dev_bf16(_lay(600, 1024, 1040, 32, 32, seed=78)["x"])
    ref = w4.svdq_linear_mx(x, layer, hadamard_block=32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w4.svdq_linear_mx(x, layer, hadamard_block=32)
        with torch.cuda.graph(g, stream=s):
            y_g = w4.svdq_linear_mx(x, layer, hadamard_block=32)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        y_g.zero_()
        other = w4.svdq_linear_mx(x_other, layer, hadamard_block=32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, ref), f"replay {rep} differs from the eager result"
        assert not torch.equal(other, ref)
