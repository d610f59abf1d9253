"""The checkpoint contract helpers ("SVDQuant W4A4" page, "Checkpoint contract"): the
quantization_config entry, modules kept in checkpoint precision, and the per-layer tensor table.
CPU only."""

import pytest
import torch

from w4a4_bit_quantized_amd import checkpoint as ck

CFG = {"quant_method": "svdquant", "rank": 32, "precision": "nvfp4", "act_unsigned": False,
       "modules_to_not_convert": ["proj_out", "norm_out"]}


def _layer(N=64, K=128, R=32, bias=False):
    t = {
        "qweight": torch.zeros((N, K // 2), dtype=torch.int8),
        "wscales": torch.zeros((K // 16, N), dtype=torch.float8_e4m3fn),
        "proj_down": torch.zeros((K, R), dtype=torch.bfloat16),
        "proj_up": torch.zeros((N, R), dtype=torch.bfloat16),
        "smooth_factor": torch.ones(K, dtype=torch.bfloat16),
        "wcscales": torch.ones(N, dtype=torch.bfloat16),
        "wtscale": torch.ones(1, dtype=torch.bfloat16),
    }
    if bias:
        t["bias"] = torch.zeros(N, dtype=torch.bfloat16)
    return t


def test_parse_config_accepts_the_page_entry():
    cfg = ck.parse_config(CFG)
    assert cfg["rank"] == 32 and cfg["modules_to_not_convert"] == ["proj_out", "norm_out"]
    assert ck.parse_config({"quant_method": "svdquant", "rank": 16})["precision"] == "nvfp4"


@pytest.mark.parametrize("bad", [{"quant_method": "awq", "rank": 32}, {"quant_method": "svdquant", "rank": -1},
                                 {"quant_method": "svdquant", "rank": 32, "precision": "int4"},
                                 {"quant_method": "svdquant", "rank": 32, "act_unsigned": True},
                                 {"quant_method": "svdquant", "rank": 32, "modules_to_not_convert": "x"}])
def test_parse_config_rejects(bad):
    with pytest.raises(ck.ContractError):
        ck.parse_config(bad)


def test_modules_to_not_convert_keep_their_precision():
    cfg = ck.parse_config(CFG)
    assert not ck.is_converted("transformer.proj_out", cfg)
    assert not ck.is_converted("transformer.norm_out.linear", cfg)
    assert ck.is_converted("transformer.blocks.0.attn.to_q", cfg)
    assert ck.W4A4Linear.from_state_dict("transformer.proj_out", {}, CFG) is None  # nothing loaded


def test_check_layer_table():
    assert ck.check_layer(_layer()) == (64, 128, 32)
    assert ck.check_layer(_layer(bias=True), rank=32) == (64, 128, 32)
    t = _layer()
    t["wscales"] = torch.zeros((64, 8), dtype=torch.uint8)  # transposed layout
    with pytest.raises(ck.ContractError):
        ck.check_layer(t)
    t = _layer()
    t["proj_up"] = t["proj_up"].float()
    with pytest.raises(ck.ContractError):
        ck.check_layer(t)
    with pytest.raises(ck.ContractError):
        ck.check_layer(_layer(K=120))  # K % 16
    with pytest.raises(ck.ContractError):
        ck.check_layer(_layer(), rank=16)
    t = _layer()
    del t["wtscale"]
    with pytest.raises(ck.ContractError):
        ck.check_layer(t)
