"""Checkpoint contract of the SVDQuant W4A4 linear layer ("SVDQuant W4A4" page, "Checkpoint
contract"): the ``quantization_config`` entry, the per-layer tensor table, and which modules
stay unconverted.

* ``parse_config`` checks the ``quantization_config`` dict (``quant_method`` "svdquant",
  ``rank``, ``precision`` "nvfp4", ``act_unsigned``, ``modules_to_not_convert``).
* ``is_converted`` says whether a module runs through this layer: modules listed in
  ``modules_to_not_convert`` keep their checkpoint precision and never reach the library
  (reading: an entry matches a module whose dotted name contains it).
* ``check_layer`` checks one layer's tensors against the table: ``qweight (N, K/2)`` int8/uint8,
  ``wscales (K/16, N)`` float8_e4m3fn/uint8, ``proj_down (K, R)``, ``proj_up (N, R)``,
  ``smooth_factor (K,)``, ``wcscales (N,)``, ``wtscale (1,)`` bf16, K % 16 == 0, and an optional
  ``bias (N,)`` bf16.
* ``W4A4Linear`` holds one converted layer on the GPU and calls ``svdq_linear``.

Nothing here computes: the layer itself is the C-ABI library.
"""

SUFFIXES = ("qweight", "wscales", "proj_down", "proj_up", "smooth_factor", "wcscales", "wtscale")


class ContractError(ValueError):
    """A configuration or tensor that does not follow the checkpoint contract."""


def parse_config(cfg):
    """Validate a ``quantization_config`` dict; returns a normalised copy."""
    if not isinstance(cfg, dict):
        raise ContractError("quantization_config must be a dict")
    if cfg.get("quant_method") != "svdquant":
        raise ContractError(f"quant_method must be 'svdquant', got {cfg.get('quant_method')!r}")
    rank = cfg.get("rank")
    if not isinstance(rank, int) or rank < 0:
        raise ContractError(f"rank must be a non-negative integer, got {rank!r}")
    if cfg.get("precision", "nvfp4") != "nvfp4":
        raise ContractError(f"precision must be 'nvfp4', got {cfg.get('precision')!r}")
    if cfg.get("act_unsigned", False):
        raise ContractError("act_unsigned = true is not supported: activations are quantized as signed E2M1")
    skip = cfg.get("modules_to_not_convert", []) or []
    if not isinstance(skip, (list, tuple)) or not all(isinstance(m, str) for m in skip):
        raise ContractError("modules_to_not_convert must be a list of module names")
    return {"quant_method": "svdquant", "rank": rank, "precision": "nvfp4", "act_unsigned": False,
            "modules_to_not_convert": list(skip)}


def is_converted(module_name, cfg):
    """False for modules that keep their checkpoint precision (listed in modules_to_not_convert)."""
    return not any(m and m in module_name for m in cfg["modules_to_not_convert"])


def _shape(t):
    return tuple(int(d) for d in t.shape)


def check_layer(tensors, rank=None):
    """Check one layer's tensors (a dict of the contract's suffixes, torch tensors on any device).
    Returns (N, K, R)."""
    import torch
    missing = [s for s in SUFFIXES if s not in tensors]
    if missing:
        raise ContractError(f"missing tensors: {missing}")
    qw = tensors["qweight"]
    if qw.dim() != 2:
        raise ContractError("qweight must be (N, K/2)")
    N, K = _shape(qw)[0], _shape(qw)[1] * 2
    if K % 16:
        raise ContractError(f"K = {K} must be divisible by 16")
    R = _shape(tensors["proj_up"])[1] if tensors["proj_up"].dim() == 2 else -1
    if rank is not None and R != rank:
        raise ContractError(f"proj_up rank {R} != config rank {rank}")
    want = {
        "qweight": ((N, K // 2), (torch.int8, torch.uint8)),
        "wscales": ((K // 16, N), (torch.float8_e4m3fn, torch.uint8)),
        "proj_down": ((K, R), (torch.bfloat16,)),
        "proj_up": ((N, R), (torch.bfloat16,)),
        "smooth_factor": ((K,), (torch.bfloat16,)),
        "wcscales": ((N,), (torch.bfloat16,)),
        "wtscale": ((1,), (torch.bfloat16,)),
    }
    if tensors.get("bias") is not None:
        want["bias"] = ((N,), (torch.bfloat16,))
    for name, (shape, dtypes) in want.items():
        t = tensors[name]
        if _shape(t) != shape:
            raise ContractError(f"{name} has shape {_shape(t)}, expected {shape}")
        if t.dtype not in dtypes:
            raise ContractError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return N, K, R


class W4A4Linear:
    """One converted linear layer on the GPU: y = svdq_linear(x, tensors) (+ bias)."""

    def __init__(self, tensors, hadamard_block=0, rank=None):
        from . import binding
        self.N, self.K, self.R = check_layer(tensors, rank)
        self.tensors = {k: v for k, v in tensors.items() if k in SUFFIXES or (k == "bias" and v is not None)}
        self.hadamard_block = int(hadamard_block)
        self._binding = binding

    @classmethod
    def from_state_dict(cls, prefix, state, cfg, device="cuda", hadamard_block=0):
        """The layer `prefix` of a checkpoint (`state` maps '<prefix>.<suffix>' to tensors), or None
        when the configuration leaves it unconverted."""
        cfg = parse_config(cfg)
        if not is_converted(prefix, cfg):
            return None
        t = {s: state[f"{prefix}.{s}"].to(device) for s in SUFFIXES}
        if f"{prefix}.bias" in state:
            t["bias"] = state[f"{prefix}.bias"].to(device)
        return cls(t, hadamard_block, cfg["rank"])

    def __call__(self, x, out=None):
        return self._binding.svdq_linear(x, self.tensors, self.hadamard_block, out=out)
