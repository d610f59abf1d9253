"""GPU parity of the standalone block Hadamard transform (rotate notes, section 3.1: the Hadacore
kernel, in place or not, per head_dim block and on output partitions) against the CPU oracle
``oracle/hadamard.py: hadamard_transform`` (needs an MI355X).

The kernel performs the oracle's float32 operations in the oracle's order and rounds once to the
storage type, so every comparison is bit-exact.  Every call goes through the C ABI.
"""

import numpy as np
import pytest

from oracle import hadamard as oh

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": "bfloat16", "f16": "float16", "f32": "float32"}


@pytest.fixture(scope="module")
def w4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import w4a4_bit_quantized_amd as w
    w.load_library()
    return w


def _stored(rng, shape, dtype, scale=3.0):
    return oh.from_f32((rng.standard_normal(shape) * scale).astype(np.float32), dtype)


def _to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _to_host(t, dtype):
    import torch
    t = t.cpu()
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def _same(got, ref, dtype):
    g = np.asarray(got).view(np.uint16 if dtype != "f32" else np.uint32)
    r = np.asarray(ref).view(np.uint16 if dtype != "f32" else np.uint32)
    bad = np.argwhere(g != r)
    assert bad.size == 0, f"{len(bad)} of {g.size} values differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("block", [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_transform_parity(w4, dtype, block):
    """Every block size and storage type, bit-exact; rows that are not a multiple of the wave
    count and rows shorter than one 512-column unit."""
    import torch
    rng = np.random.default_rng(block)
    cols = max(block, 3 * block if block <= 512 else block * 2)
    x = _stored(rng, (37, cols), dtype)
    y = w4.hadamard_transform(_to_dev(x, dtype), block)
    torch.cuda.synchronize()
    _same(_to_host(y, dtype), oh.hadamard_transform(x, block, dtype), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block,cols", [(64, 192), (128, 640), (16, 48), (2, 6), (4, 12), (8, 8)])
def test_ragged_units(w4, dtype, block, cols):
    """Column counts that end inside a 512-column unit (idle lanes) and that are not multiples
    of 8 (element-wise path)."""
    import torch
    rng = np.random.default_rng(cols)
    x = _stored(rng, (5, cols), dtype)
    y = w4.hadamard_transform(_to_dev(x, dtype), block)
    torch.cuda.synchronize()
    _same(_to_host(y, dtype), oh.hadamard_transform(x, block, dtype), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_in_place_and_involution(w4, dtype):
    """inplace=True writes into x; applying the transform twice returns x (exactly, for powers
    of four and small integers)."""
    import torch
    rng = np.random.default_rng(2)
    xi = rng.integers(-1, 2, size=(9, 4 * 64)).astype(np.float32)
    x = oh.from_f32(xi, dtype)
    t = _to_dev(x, dtype)
    ptr = t.data_ptr()
    out = w4.hadamard_transform(t, 64, inplace=True)
    assert out.data_ptr() == ptr
    torch.cuda.synchronize()
    _same(_to_host(t, dtype), oh.hadamard_transform(x, 64, dtype), dtype)
    w4.hadamard_transform(t, 64, inplace=True)
    torch.cuda.synchronize()
    assert np.array_equal(oh.to_f32(_to_host(t, dtype), dtype), xi)


def test_output_partition(w4):
    """A column partition [start, start + length) of a row-major matrix, addressed with the full
    row stride, is transformed in place; the other columns keep their bytes."""
    import torch
    rng = np.random.default_rng(4)
    x = _stored(rng, (33, 1024), "bf16")
    t = _to_dev(x, "bf16")
    w4.hadamard_transform(t[:, 256:256 + 384], 128, inplace=True)
    torch.cuda.synchronize()
    _same(_to_host(t, "bf16"), oh.hadamard_transform(x, 128, "bf16", start=256, length=384), "bf16")


def test_misaligned_start_takes_element_path(w4):
    """A partition starting one element past a 16-byte boundary (element-wise loads and stores)."""
    import torch
    rng = np.random.default_rng(6)
    x = _stored(rng, (7, 136), "f16")
    t = _to_dev(x, "f16")
    out = torch.zeros_like(t)
    w4.hadamard_transform(t[:, 1:129], 64, out=out[:, 1:129])
    torch.cuda.synchronize()
    ref = oh.hadamard_transform(x[:, 1:129], 64, "f16")
    _same(_to_host(out, "f16")[:, 1:129], ref, "f16")
    assert not _to_host(out, "f16")[:, 129:].any() and not _to_host(out, "f16")[:, :1].any()


def test_head_dim_blocks_of_3d_tensor(w4):
    """(tokens, heads, head_dim) tensors: blocking by head_dim is the transform of each head."""
    import torch
    rng = np.random.default_rng(8)
    x = _stored(rng, (6, 12, 64), "bf16")
    y = w4.hadamard_transform(_to_dev(x, "bf16"), 64)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (6, 12, 64)
    _same(_to_host(y, "bf16").reshape(72, 64), oh.hadamard_transform(x.reshape(72, 64), 64, "bf16"), "bf16")


def test_empty_and_errors(w4):
    import torch
    t = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    assert w4.hadamard_transform(t, 128).shape == (0, 128)
    with pytest.raises(w4.W4A4Error):
        w4.hadamard_transform(torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda"), 64)  # 96 % 64
    with pytest.raises(w4.W4A4Error):
        w4.hadamard_transform(torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda"), 48)  # not a power of two


def test_full_size_dit_activation(w4):
    """The rotated down-projection's activation (4096 x 12288 bf16, blocks of 128), as the bench
    times it, checked on sampled rows."""
    import torch
    rng = np.random.default_rng(10)
    x = _stored(rng, (4096, 12288), "bf16", scale=1.0)
    t = _to_dev(x, "bf16")
    y = w4.hadamard_transform(t, 128)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(4096, 48, replace=False))
    _same(_to_host(y, "bf16")[rows], oh.hadamard_transform(x[rows], 128, "bf16"), "bf16")
