"""w4a4_bit_quantized_amd -- SVDQuant W4A4 linear layer on AMD MI355X (gfx950).

The compute path is the C-ABI library ``libw4a4.so`` (hand-written HIP kernels,
declared in ``include/w4a4.h``); ``binding`` marshals torch device tensors to
it.  ``synth`` draws the seeded synthetic workloads.

Importing this package never loads the library; the first call into
``binding`` does, and raises if the library has not been built.
"""

__version__ = "0.1.0"

from .binding import (  # noqa: F401
    W4A4Error,
    hadamard_transform,
    library_path,
    load_library,
    svdq_gemm_lowrank,
    svdq_linear,
    svdq_linear_workspace_bytes,
    svdq_quantize_act,
    svdq_quantize_weight,
    svdq_gemm_lowrank_mx,
    svdq_linear_mx,
    svdq_linear_mx_workspace_bytes,
    svdq_linear_noalloc,
    svdq_lowrank_split,
    svdq_quantize_act_mx,
    svdq_quantize_weight_mx,
)
