"""ctypes binding of libw4a4 (include/w4a4.h).

Argument marshalling only: dtype/device/contiguity checks on torch tensors,
output allocation with torch, the current torch stream as the HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  The library is loaded on first use and a missing build raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS_NAMES = {0: "W4A4_OK", 1: "W4A4_ERR_NULL", 2: "W4A4_ERR_SHAPE", 3: "W4A4_ERR_ALIGN",
                4: "W4A4_ERR_UNSUPPORTED", 5: "W4A4_ERR_HIP", 6: "W4A4_ERR_SCRATCH"}

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_p = ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/w4a4.h
SIGNATURES = {
    "w4a4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a4_version": (ctypes.c_int, []),
    "svdq_quantize_act": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p, _c_p]),
    "svdq_quantize_weight": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "svdq_gemm_lowrank": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                         _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "svdq_linear_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "svdq_linear": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                   _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "svdq_quantize_act_mx": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p,
                                            _c_p]),
    "svdq_quantize_weight_mx": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "svdq_gemm_lowrank_mx": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                            _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "svdq_linear_mx_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "svdq_linear_mx": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                      _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "w4a4_hadamard_transform": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_p]),
    "svdq_gemm_lowrank_bias": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                              _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "svdq_linear_bias": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                        _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "svdq_gemm_lowrank_mx_bias": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                 _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "svdq_lowrank_split": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, ctypes.c_uint64,
                                          _c_i32, _c_p, _c_p, _c_p, _c_p]),
    "svdq_linear_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p]),
    "svdq_linear_mx_bias": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_p, _c_p, ctypes.c_size_t,
                                           _c_p]),
}

# storage type codes of w4a4_hadamard_transform
DTYPE_BF16, DTYPE_F16, DTYPE_F32 = 0, 1, 2
HADAMARD_MAX_BLOCK = 4096


class W4A4Error(RuntimeError):
    """A libw4a4 call returned a non-OK status (or the library is missing)."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def library_path():
    return os.environ.get("W4A4_LIBRARY", os.path.join(_HERE, "libw4a4.so"))


def test_library_path():
    """The test build (path-forcing hooks read from the environment); only tests load it."""
    return os.path.join(_HERE, "libw4a4_test.so")


def open_library(path):
    """Open one build of the library and declare its C signatures (no caching)."""
    if not os.path.exists(path):
        raise W4A4Error(f"{os.path.basename(path)} is not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_library():
    """Load libw4a4.so (once) and declare its C signatures."""
    global _LIB
    if _LIB is None:
        _LIB = open_library(library_path())
    return _LIB


def _check(status, what):
    if status != 0:
        name = STATUS_NAMES.get(status, str(status))
        msg = load_library().w4a4_status_string(status).decode()
        raise W4A4Error(f"{what} failed: {name} ({msg})", status)


def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name, dtypes, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, name, shape):
    """Raise ValueError unless tensor ``t`` has exactly ``shape`` (the C ABI sees raw pointers, so
    a mis-sized tensor would be read or written past its end)."""
    got = tuple(int(d) for d in t.shape)
    want = tuple(int(d) for d in shape)
    if got != want:
        raise ValueError(f"{name} has shape {got}, expected {want}")


def check_quantize_act_shapes(x, smooth_factor, proj_down):
    """Sizes (M, K, R) of an activation quantizer call, after checking that every tensor agrees."""
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D (M, K), got shape {tuple(x.shape)}")
    M, K = (int(d) for d in x.shape)
    if proj_down.dim() != 2:
        raise ValueError(f"proj_down must be 2-D (K, R), got shape {tuple(proj_down.shape)}")
    R = int(proj_down.shape[1])
    _shape(smooth_factor, "smooth_factor", (K,))
    _shape(proj_down, "proj_down", (K, R))
    return M, K, R


def check_gemm_shapes(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, y=None, bias=None,
                      group=16, scale_rows=None):
    """Sizes (M, N, K, R) of a GEMM call, after checking every tensor against them.  ``group`` is
    16 (e4m3 scales) or 32 (E8M0); ``scale_rows`` the activation scale row count (default M)."""
    for t, n in ((qact, "qact"), (qweight, "qweight"), (proj_up, "proj_up")):
        if t.dim() != 2:
            raise ValueError(f"{n} must be 2-D, got shape {tuple(t.shape)}")
    M, K = int(qact.shape[0]), 2 * int(qact.shape[1])
    N, R = int(qweight.shape[0]), int(proj_up.shape[1])
    _shape(ascales, "ascales", (K // group, M if scale_rows is None else scale_rows))
    _shape(lora_act, "lora_act", (M, R))
    _shape(qweight, "qweight", (N, K // 2))
    _shape(wscales, "wscales", (K // group, N))
    _shape(proj_up, "proj_up", (N, R))
    _shape(wcscales, "wcscales", (N,))
    if wtscale.numel() != 1:
        raise ValueError(f"wtscale must hold one value, got shape {tuple(wtscale.shape)}")
    if y is not None:
        _shape(y, "out", (M, N))
    if bias is not None:
        _shape(bias, "bias", (N,))
    return M, N, K, R


def check_layer_shapes(M, K, layer, group=16, y=None):
    """Sizes (N, R) of a whole-layer call on an (M, K) input, after checking every checkpoint
    tensor of ``layer`` (and ``out``, ``bias``) against them."""
    qw, pu = layer["qweight"], layer["proj_up"]
    if qw.dim() != 2 or pu.dim() != 2:
        raise ValueError("qweight and proj_up must be 2-D")
    N, R = int(qw.shape[0]), int(pu.shape[1])
    _shape(qw, "qweight", (N, K // 2))
    _shape(layer["wscales"], "wscales", (K // group, N))
    _shape(layer["proj_down"], "proj_down", (K, R))
    _shape(pu, "proj_up", (N, R))
    _shape(layer["smooth_factor"], "smooth_factor", (K,))
    _shape(layer["wcscales"], "wcscales", (N,))
    if layer["wtscale"].numel() != 1:
        raise ValueError(f"wtscale must hold one value, got shape {tuple(layer['wtscale'].shape)}")
    if layer.get("bias") is not None:
        _shape(layer["bias"], "bias", (N,))
    if y is not None:
        _shape(y, "out", (M, N))
    return N, R


def _bytes_dtypes():
    torch = _torch()
    return (torch.uint8, torch.int8)


def _scale_dtypes():
    torch = _torch()
    return (torch.uint8, torch.float8_e4m3fn)


def svdq_linear_workspace_bytes(M, K, R):
    return int(load_library().svdq_linear_workspace_bytes(int(M), int(K), int(R)))


def svdq_quantize_act(x, smooth_factor, proj_down, hadamard_block=0):
    """x (M, K) bf16 -> (qact (M, K/2) u8, ascales (K/16, M) u8, lora_act (M, R) f32)."""
    torch = _torch()
    lib = load_library()
    x = _dev(x, "x", (torch.bfloat16,))
    dev = x.device
    M, K = x.shape
    _dev(smooth_factor, "smooth_factor", (torch.bfloat16,), dev)
    _dev(proj_down, "proj_down", (torch.bfloat16,), dev)
    M, K, R = check_quantize_act_shapes(x, smooth_factor, proj_down)
    qact = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    ascales = torch.empty((K // 16, M), dtype=torch.uint8, device=dev)
    lora = torch.empty((M, R), dtype=torch.float32, device=dev)
    st = lib.svdq_quantize_act(_ptr(x), _ptr(smooth_factor), _ptr(proj_down), M, K, R, int(hadamard_block),
                               _ptr(qact), _ptr(ascales), _ptr(lora), _stream(dev))
    _check(st, "svdq_quantize_act")
    return qact, ascales, lora


def svdq_quantize_weight(w, smooth_factor, hadamard_block=0):
    """w (N, K) bf16 -> (qweight (N, K/2) u8, wscales (K/16, N) u8)."""
    torch = _torch()
    lib = load_library()
    w = _dev(w, "w", (torch.bfloat16,))
    dev = w.device
    N, K = w.shape
    _dev(smooth_factor, "smooth_factor", (torch.bfloat16,), dev)
    _shape(smooth_factor, "smooth_factor", (K,))
    qweight = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wscales = torch.empty((K // 16, N), dtype=torch.uint8, device=dev)
    st = lib.svdq_quantize_weight(_ptr(w), _ptr(smooth_factor), N, K, int(hadamard_block),
                                  _ptr(qweight), _ptr(wscales), _stream(dev))
    _check(st, "svdq_quantize_weight")
    return qweight, wscales


def svdq_gemm_lowrank(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, out=None, bias=None):
    """Block-scaled FP4 GEMM + epilogue -> y (M, N) bf16; ``bias`` (N,) bf16 is optional."""
    torch = _torch()
    lib = load_library()
    qact = _dev(qact, "qact", _bytes_dtypes())
    dev = qact.device
    _dev(ascales, "ascales", _scale_dtypes(), dev)
    _dev(lora_act, "lora_act", (torch.float32,), dev)
    _dev(qweight, "qweight", _bytes_dtypes(), dev)
    _dev(wscales, "wscales", _scale_dtypes(), dev)
    _dev(proj_up, "proj_up", (torch.bfloat16,), dev)
    _dev(wcscales, "wcscales", (torch.bfloat16,), dev)
    _dev(wtscale, "wtscale", (torch.bfloat16,), dev)
    if bias is not None:
        _dev(bias, "bias", (torch.bfloat16,), dev)
    M, N, K, R = check_gemm_shapes(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, out, bias)
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", (torch.bfloat16,), dev)
    if bias is None:
        st = lib.svdq_gemm_lowrank(_ptr(qact), _ptr(ascales), _ptr(lora_act), _ptr(qweight), _ptr(wscales),
                                   _ptr(proj_up), _ptr(wcscales), _ptr(wtscale), M, N, K, R, _ptr(y), _stream(dev))
    else:
        _dev(bias, "bias", (torch.bfloat16,), dev)
        st = lib.svdq_gemm_lowrank_bias(_ptr(qact), _ptr(ascales), _ptr(lora_act), _ptr(qweight), _ptr(wscales),
                                        _ptr(proj_up), _ptr(wcscales), _ptr(wtscale), _ptr(bias), M, N, K, R,
                                        _ptr(y), _stream(dev))
    _check(st, "svdq_gemm_lowrank")
    return y


LAYER_KEYS = ("qweight", "wscales", "proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale")


def svdq_linear(x, layer, hadamard_block=0, workspace=None, out=None):
    """The whole W4A4 layer.  ``x`` (..., K) bf16; leading dims are flattened into M.

    ``layer`` maps the checkpoint names (qweight, wscales, proj_down, proj_up,
    smooth_factor, wcscales, wtscale) to device tensors, and optionally ``bias``
    (N,) bf16.  ``workspace`` (u8, at least svdq_linear_workspace_bytes bytes)
    and ``out`` may be passed to avoid allocation.
    """
    torch = _torch()
    lib = load_library()
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    _dev(x2, "x", (torch.bfloat16,))
    dev = x2.device
    M, K = x2.shape
    t = {k: layer[k] for k in LAYER_KEYS}
    _dev(t["qweight"], "qweight", _bytes_dtypes(), dev)
    _dev(t["wscales"], "wscales", _scale_dtypes(), dev)
    for k in ("proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale"):
        _dev(t[k], k, (torch.bfloat16,), dev)
    if layer.get("bias") is not None:
        _dev(layer["bias"], "bias", (torch.bfloat16,), dev)
    N, R = check_layer_shapes(M, K, layer, group=16, y=out)
    need = int(lib.svdq_linear_workspace_bytes(M, K, R))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", (torch.uint8,), dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", (torch.bfloat16,), dev)
    common = (_ptr(x2), _ptr(t["qweight"]), _ptr(t["wscales"]), _ptr(t["proj_down"]), _ptr(t["proj_up"]),
              _ptr(t["smooth_factor"]), _ptr(t["wcscales"]), _ptr(t["wtscale"]))
    tail = (M, N, K, R, int(hadamard_block), _ptr(y), _ptr(workspace), workspace.numel(), _stream(dev))
    bias = layer.get("bias")
    if bias is None:
        st = lib.svdq_linear(*common, *tail)
    else:
        _dev(bias, "bias", (torch.bfloat16,), dev)
        st = lib.svdq_linear_bias(*common, _ptr(bias), *tail)
    _check(st, "svdq_linear")
    return y.reshape(*lead, N)


NOALLOC_SCRATCH_BYTES = 64 << 20  # W4A4_NOALLOC_SCRATCH_BYTES


def svdq_linear_noalloc(x, layer, hadamard_block=0, out=None):
    """``svdq_linear`` through the entry point without allocation: the library's static device
    workspace instead of a caller-provided one (the binding still allocates ``out`` unless given)."""
    torch = _torch()
    lib = load_library()
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    _dev(x2, "x", (torch.bfloat16,))
    dev = x2.device
    M, K = x2.shape
    t = {k: layer[k] for k in LAYER_KEYS}
    _dev(t["qweight"], "qweight", _bytes_dtypes(), dev)
    _dev(t["wscales"], "wscales", _scale_dtypes(), dev)
    for k in ("proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale"):
        _dev(t[k], k, (torch.bfloat16,), dev)
    bias = layer.get("bias")
    if bias is not None:
        _dev(bias, "bias", (torch.bfloat16,), dev)
    N, R = check_layer_shapes(M, K, layer, group=16, y=out)
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", (torch.bfloat16,), dev)
    st = lib.svdq_linear_noalloc(_ptr(x2), _ptr(t["qweight"]), _ptr(t["wscales"]), _ptr(t["proj_down"]),
                                 _ptr(t["proj_up"]), _ptr(t["smooth_factor"]), _ptr(t["wcscales"]), _ptr(t["wtscale"]),
                                 _ptr(bias), M, N, K, R, int(hadamard_block), _ptr(y), _stream(dev))
    _check(st, "svdq_linear_noalloc")
    return y.reshape(*lead, N)


# ---- MXFP4 variant (E2M1 in blocks of 32 with one E8M0 scale per block) ---------------------

def mx_scale_rows(M):
    """Row stride of the MX activation scale tensor: M rounded up to a multiple of 4."""
    return (int(M) + 3) // 4 * 4


def svdq_linear_mx_workspace_bytes(M, K, R):
    return int(load_library().svdq_linear_mx_workspace_bytes(int(M), int(K), int(R)))


def svdq_quantize_act_mx(x, smooth_factor, proj_down, hadamard_block=32):
    """x (M, K) bf16 -> (qact (M, K/2) u8, ascales (K/32, Mp) u8 E8M0, lora_act (M, R) f32)."""
    torch = _torch()
    lib = load_library()
    x = _dev(x, "x", (torch.bfloat16,))
    dev = x.device
    M, K = x.shape
    _dev(smooth_factor, "smooth_factor", (torch.bfloat16,), dev)
    _dev(proj_down, "proj_down", (torch.bfloat16,), dev)
    M, K, R = check_quantize_act_shapes(x, smooth_factor, proj_down)
    qact = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    ascales = torch.empty((K // 32, mx_scale_rows(M)), dtype=torch.uint8, device=dev)
    lora = torch.empty((M, R), dtype=torch.float32, device=dev)
    st = lib.svdq_quantize_act_mx(_ptr(x), _ptr(smooth_factor), _ptr(proj_down), M, K, R, int(hadamard_block),
                                  _ptr(qact), _ptr(ascales), _ptr(lora), _stream(dev))
    _check(st, "svdq_quantize_act_mx")
    return qact, ascales, lora


def svdq_quantize_weight_mx(w, smooth_factor, hadamard_block=32):
    """w (N, K) bf16 -> (qweight (N, K/2) u8, wscales (K/32, N) u8 E8M0)."""
    torch = _torch()
    lib = load_library()
    w = _dev(w, "w", (torch.bfloat16,))
    dev = w.device
    N, K = w.shape
    _dev(smooth_factor, "smooth_factor", (torch.bfloat16,), dev)
    _shape(smooth_factor, "smooth_factor", (K,))
    qweight = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wscales = torch.empty((K // 32, N), dtype=torch.uint8, device=dev)
    st = lib.svdq_quantize_weight_mx(_ptr(w), _ptr(smooth_factor), N, K, int(hadamard_block),
                                     _ptr(qweight), _ptr(wscales), _stream(dev))
    _check(st, "svdq_quantize_weight_mx")
    return qweight, wscales


def svdq_gemm_lowrank_mx(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, out=None,
                         bias=None):
    """MXFP4 GEMM + epilogue -> y (M, N) bf16; ``bias`` (N,) bf16 is optional."""
    torch = _torch()
    lib = load_library()
    qact = _dev(qact, "qact", _bytes_dtypes())
    dev = qact.device
    _dev(ascales, "ascales", (torch.uint8,), dev)
    _dev(lora_act, "lora_act", (torch.float32,), dev)
    _dev(qweight, "qweight", _bytes_dtypes(), dev)
    _dev(wscales, "wscales", (torch.uint8,), dev)
    _dev(proj_up, "proj_up", (torch.bfloat16,), dev)
    _dev(wcscales, "wcscales", (torch.bfloat16,), dev)
    _dev(wtscale, "wtscale", (torch.bfloat16,), dev)
    if bias is not None:
        _dev(bias, "bias", (torch.bfloat16,), dev)
    M, N, K, R = check_gemm_shapes(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, out, bias,
                                   group=32, scale_rows=mx_scale_rows(qact.shape[0]))
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", (torch.bfloat16,), dev)
    if bias is None:
        st = lib.svdq_gemm_lowrank_mx(_ptr(qact), _ptr(ascales), _ptr(lora_act), _ptr(qweight), _ptr(wscales),
                                      _ptr(proj_up), _ptr(wcscales), _ptr(wtscale), M, N, K, R, _ptr(y), _stream(dev))
    else:
        _dev(bias, "bias", (torch.bfloat16,), dev)
        st = lib.svdq_gemm_lowrank_mx_bias(_ptr(qact), _ptr(ascales), _ptr(lora_act), _ptr(qweight), _ptr(wscales),
                                           _ptr(proj_up), _ptr(wcscales), _ptr(wtscale), _ptr(bias), M, N, K, R,
                                           _ptr(y), _stream(dev))
    _check(st, "svdq_gemm_lowrank_mx")
    return y


def svdq_linear_mx(x, layer, hadamard_block=32, workspace=None, out=None):
    """The whole MXFP4 layer (``layer`` as for ``svdq_linear``, with MX qweight / wscales; optional ``bias``)."""
    torch = _torch()
    lib = load_library()
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    _dev(x2, "x", (torch.bfloat16,))
    dev = x2.device
    M, K = x2.shape
    t = {k: layer[k] for k in LAYER_KEYS}
    _dev(t["qweight"], "qweight", _bytes_dtypes(), dev)
    _dev(t["wscales"], "wscales", (torch.uint8,), dev)
    for k in ("proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale"):
        _dev(t[k], k, (torch.bfloat16,), dev)
    if layer.get("bias") is not None:
        _dev(layer["bias"], "bias", (torch.bfloat16,), dev)
    N, R = check_layer_shapes(M, K, layer, group=32, y=out)
    need = int(lib.svdq_linear_mx_workspace_bytes(M, K, R))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", (torch.uint8,), dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", (torch.bfloat16,), dev)
    common = (_ptr(x2), _ptr(t["qweight"]), _ptr(t["wscales"]), _ptr(t["proj_down"]), _ptr(t["proj_up"]),
              _ptr(t["smooth_factor"]), _ptr(t["wcscales"]), _ptr(t["wtscale"]))
    tail = (M, N, K, R, int(hadamard_block), _ptr(y), _ptr(workspace), workspace.numel(), _stream(dev))
    bias = layer.get("bias")
    if bias is None:
        st = lib.svdq_linear_mx(*common, *tail)
    else:
        _dev(bias, "bias", (torch.bfloat16,), dev)
        st = lib.svdq_linear_mx_bias(*common, _ptr(bias), *tail)
    _check(st, "svdq_linear_mx")
    return y.reshape(*lead, N)


def _rows_view(t, name):
    """(rows, cols, row stride) of a tensor whose last dimension is dense: 2-D with any row stride
    (a column partition of a larger matrix), or any shape that flattens to rows without copying."""
    if t.dim() == 0 or t.stride(-1) != 1:
        raise ValueError(f"{name} must have a dense last dimension")
    cols = t.shape[-1]
    if t.dim() == 1:
        return 1, cols, cols
    if t.dim() == 2:
        if t.shape[0] > 1 and t.stride(0) < cols:
            raise ValueError(f"{name} rows overlap (row stride {t.stride(0)} < {cols})")
        return t.shape[0], cols, t.stride(0) if t.shape[0] > 1 else cols
    if not t.is_contiguous():
        raise ValueError(f"{name} with more than two dimensions must be contiguous")
    return t.numel() // max(cols, 1), cols, cols


def hadamard_transform(x, block=None, inplace=False, out=None):
    """Normalised block Sylvester Hadamard transform of the last dimension, per `block` columns
    (default: the whole last dimension, a power of two up to HADAMARD_MAX_BLOCK); its own inverse.

    x: bf16, f16 or f32 device tensor with a dense last dimension (a 2-D column slice such as
    y[:, start:start + length] is fine).  inplace=True writes into x and returns it; otherwise
    the result goes to `out` (same shape and dtype) or a new tensor."""
    torch = _torch()
    lib = load_library()
    codes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a device tensor")
    if x.dtype not in codes:
        raise TypeError(f"x must be bf16, f16 or f32, got {x.dtype}")
    rows, cols, ldx = _rows_view(x, "x")
    block = int(cols if block is None else block)
    if inplace:
        y = x
    else:
        y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
        if y.shape != x.shape or y.dtype != x.dtype or y.device != x.device:
            raise ValueError("out must match x in shape, dtype and device")
    _, _, ldy = _rows_view(y, "out")
    st = lib.w4a4_hadamard_transform(_ptr(x), ldx, _ptr(y), ldy, rows, cols, block, codes[x.dtype],
                                     _stream(x.device))
    _check(st, "w4a4_hadamard_transform")
    return y


def svdq_lowrank_split(w, smooth_factor, rank, oversample=16, power_iters=4, seed=0, threads=0):
    """Offline low-rank split of W * smooth_factor on the host (numpy bf16 bit patterns in, out).

    ``w`` (N, K) and ``smooth_factor`` (K,) are uint16 arrays of bf16 bits.  Returns
    (proj_down (K, R), proj_up (N, R), residual (N, K)) as uint16 bf16 bits and the R singular
    values (float32).  The residual already carries the smoothing: quantize it with a
    smooth_factor of ones."""
    import numpy as np
    lib = load_library()
    w = np.ascontiguousarray(w, dtype=np.uint16)
    lam = np.ascontiguousarray(smooth_factor, dtype=np.uint16)
    N, K = w.shape
    R = int(rank)
    pd = np.zeros((K, R), dtype=np.uint16)
    pu = np.zeros((N, R), dtype=np.uint16)
    resid = np.zeros((N, K), dtype=np.uint16)
    sv = np.zeros(max(R, 1), dtype=np.float32)
    st = lib.svdq_lowrank_split(w.ctypes.data, lam.ctypes.data, N, K, R, int(oversample), int(power_iters),
                                int(seed), int(threads), pd.ctypes.data if R else None,
                                pu.ctypes.data if R else None, resid.ctypes.data, sv.ctypes.data)
    _check(st, "svdq_lowrank_split")
    return pd, pu, resid, sv[:R]
