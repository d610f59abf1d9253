"""Block Sylvester Hadamard rotation (oracle, test infrastructure only).

Source: "Rotate techniques in quantization and their vLLM implementation"
(llx-08 notes).  Section 2.1: an orthogonal R is inserted into y = x W as
(x R^T)(R W), so activations are rotated online and weights offline.  Section
2.2: the Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]], H H^T = n I, and
H = H^T; it can be applied like an FFT in O(n log n).  Section 1 (the 4-element
example) normalises by 1/sqrt(n) (every entry of H_4 is +-0.5).  Section 3.1:
the transform is its own inverse and equals a product with the dense matrix.

Reading where the pages leave the order open: each contiguous block of B
elements along the last axis is transformed with butterfly stages of span
h = 1, 2, 4, ..., B/2 in that order; a stage replaces each pair (a, b) at
positions (j, j + h), j mod 2h < h, by (a + b, a - b) in float32; after the
last stage every element is multiplied once by float32(1/sqrt(B)).  This is
x_block @ H_B^T with H_B the normalised Sylvester matrix.

Standalone transform (section 3.1: the Hadacore kernel, in place or not, also
applied per head_dim block and to column partitions of a linear layer's output):
``hadamard_transform`` widens the stored values to float32, applies
``fwht_blocks`` to the chosen columns of every row, and rounds the result once
to the storage type (bf16 or f16 to nearest even; float32 unchanged).  Columns
outside the chosen range are left as they are.

Pins: the pages' worked example [1.2, 0.8, 1.5, 12.0] -> [7.75, -5.05, -5.75,
5.45]; equality with a dense Sylvester matrix built by the recursion;
orthogonality H H^T = I and symmetry; involution (applying it twice returns the
input up to float32 rounding); for the standalone transform, the dense product
rounded once to the storage type, exact involution for powers of four on small
integers, and untouched columns outside the partition.
"""

import numpy as np

from . import formats


def norm_const(block):
    """float32(1/sqrt(B)): the normalisation applied after the butterflies."""
    return np.float32(1.0 / np.sqrt(np.float64(block)))


def fwht_blocks(v, block):
    """Apply the normalised Sylvester Hadamard transform to every B-block of the last axis.

    ``v`` is converted to float32; the last axis length must be a multiple of
    ``block``, which must be a power of two.  Returns a new float32 array.
    """
    v = np.array(v, dtype=np.float32, copy=True)
    if block <= 1:
        return v
    if block & (block - 1):
        raise ValueError("block must be a power of two")
    k = v.shape[-1]
    if k % block:
        raise ValueError("last axis must be a multiple of the block")
    lead = v.shape[:-1]
    h = 1
    while h < block:
        # view each block as (pairs of spans of length h): [..., nblk, block/(2h), 2, h]
        w = v.reshape(lead + (k // block, block // (2 * h), 2, h))
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b  # float32 + float32 -> float32 (IEEE)
        w[..., 1, :] = a - b
        v = w.reshape(lead + (k,))
        h *= 2
    return (v * norm_const(block)).astype(np.float32)


DTYPES = ("bf16", "f16", "f32")


def to_f32(stored, dtype):
    """Stored values (bf16 bit patterns as uint16, float16 or float32 arrays) -> float32 (exact)."""
    if dtype == "bf16":
        return formats.bf16_to_f32(np.asarray(stored, dtype=np.uint16))
    if dtype == "f16":
        return np.asarray(stored, dtype=np.float16).astype(np.float32)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32)
    raise ValueError(dtype)


def from_f32(v, dtype):
    """float32 values -> the storage type, rounded once to nearest even."""
    v = np.asarray(v, dtype=np.float32)
    if dtype == "bf16":
        return formats.bf16_from_f64(v.astype(np.float64))  # float32 -> float64 is exact: one rounding
    if dtype == "f16":
        return v.astype(np.float16)  # IEEE round to nearest even
    if dtype == "f32":
        return v.copy()
    raise ValueError(dtype)


def hadamard_transform(stored, block, dtype="bf16", start=0, length=None):
    """Normalised block Sylvester transform of columns [start, start + length) of every row.

    ``stored`` is a 2-D array in the storage type of ``dtype``; returns a new
    array of the same type where the chosen columns hold the transformed
    values (rounded once) and every other column is copied unchanged.
    """
    stored = np.asarray(stored)
    out = stored.copy()
    n = stored.shape[-1] - start if length is None else length
    v = to_f32(stored[..., start:start + n], dtype)
    out[..., start:start + n] = from_f32(fwht_blocks(v, block), dtype)
    return out
