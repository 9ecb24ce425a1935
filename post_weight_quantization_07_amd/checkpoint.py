"""Checkpoint export and load of quantized layers.

AutoGPTQ examples walkthrough (save_quantized / from_quantized, and the
BaseQuantizeConfig section): the quantized weights go to one file named
gptq_model-{bits}bit-{group_size}g (.safetensors when asked for it), next to
quantize_config.json, which records the quantization parameters; loading
reads quantize_config.json first and takes bits and group_size from it to
find the weight file.  The chapter on group quantization describes each
group's scale and zero point as one float16 each.

The pages name neither the tensors nor their layout; this module stores, per
layer `name`:
  name.qweight  int32   [d_in * bits / 32, d_out]  the ABI's pack layout
  name.scales   float16 [n_groups, d_out]          (the solve's fp32 scales, rounded)
  name.zeros    float16 [n_groups, d_out]          integer zero points (exact in float16)
  name.g_idx    int32   [d_in]                     original column -> group
and quantize_config.json with BaseQuantizeConfig's fields plus
model_name_or_path and model_file_base_name.
"""
from __future__ import annotations

import json
import os
from typing import Dict, Mapping, Tuple

import torch

from ._lib import QuantizeConfig

CONFIG_NAME = "quantize_config.json"


def model_file_base_name(bits: int, group_size: int) -> str:
    return f"gptq_model-{bits}bit-{group_size}g"


def save_quantized(out_dir: str, layers: Mapping[str, Mapping[str, torch.Tensor]], cfg: QuantizeConfig,
                   model_name_or_path: str = "", true_sequential: bool = True) -> str:
    """Write the layers' qweight / scales / zeros / g_idx (as returned by
    solve_layer or solve_layers_shared) and quantize_config.json into out_dir;
    returns the weight file's path."""
    from safetensors.torch import save_file
    os.makedirs(out_dir, exist_ok=True)
    tensors: Dict[str, torch.Tensor] = {}
    for name, r in layers.items():
        qweight, scales, zeros, g_idx = r["qweight"], r["scales"], r["zeros"], r["g_idx"]
        if qweight.dtype != torch.int32 or g_idx.dtype != torch.int32 or zeros.dtype != torch.int32:
            raise ValueError(f"save_quantized: {name}: qweight, zeros and g_idx must be int32")
        if scales.shape != zeros.shape or qweight.shape[1] != scales.shape[1]:
            raise ValueError(f"save_quantized: {name}: inconsistent shapes")
        if int(zeros.max()) > 2048 or int(zeros.min()) < 0:
            raise ValueError(f"save_quantized: {name}: zero points outside [0, 2048] are not exact in float16")
        tensors[f"{name}.qweight"] = qweight.detach().contiguous().cpu()
        tensors[f"{name}.scales"] = scales.detach().to(torch.float16).contiguous().cpu()
        tensors[f"{name}.zeros"] = zeros.detach().to(torch.float16).contiguous().cpu()
        tensors[f"{name}.g_idx"] = g_idx.detach().contiguous().cpu()
    base = model_file_base_name(cfg.bits, cfg.group_size)
    path = os.path.join(out_dir, base + ".safetensors")
    save_file(tensors, path, metadata={"format": "pt"})
    conf = {"bits": cfg.bits, "group_size": cfg.group_size, "damp_percent": cfg.damp_percent,
            "desc_act": cfg.desc_act, "static_groups": cfg.static_groups, "sym": cfg.sym,
            "true_sequential": true_sequential, "model_name_or_path": model_name_or_path,
            "model_file_base_name": base}
    with open(os.path.join(out_dir, CONFIG_NAME), "w") as f:
        json.dump(conf, f, indent=2)
    return path


def load_quantized(in_dir: str, device="cpu") -> Tuple[QuantizeConfig, Dict[str, Dict[str, torch.Tensor]]]:
    """Read quantize_config.json, then the weight file it names; returns the
    config and, per layer, qweight, scales, zeros (float16 as stored) and g_idx."""
    from safetensors.torch import load_file
    with open(os.path.join(in_dir, CONFIG_NAME)) as f:
        conf = json.load(f)
    cfg = QuantizeConfig(bits=conf["bits"], group_size=conf["group_size"], damp_percent=conf["damp_percent"],
                         desc_act=conf["desc_act"], static_groups=conf["static_groups"], sym=conf["sym"])
    base = conf.get("model_file_base_name") or model_file_base_name(cfg.bits, cfg.group_size)
    flat = load_file(os.path.join(in_dir, base + ".safetensors"), device=str(device))
    layers: Dict[str, Dict[str, torch.Tensor]] = {}
    for key, t in flat.items():
        name, field = key.rsplit(".", 1)
        layers.setdefault(name, {})[field] = t
    for name, r in layers.items():
        missing = {"qweight", "scales", "zeros", "g_idx"} - set(r)
        if missing:
            raise ValueError(f"load_quantized: {name}: missing {sorted(missing)}")
    return cfg, layers


def dequant_layer(r: Mapping[str, torch.Tensor], bits: int, device="cuda:0") -> Dict[str, torch.Tensor]:
    """A loaded layer in the form the dequantizing product reads, on `device`:
    int32 qweight, zeros and g_idx, fp32 scales (the stored float16 values).
    When some 32-channel chunk spans several groups (act-order with dynamic
    groups) the layer is put in group order once by gptq_dequant_order, which
    replaces qweight and g_idx and adds `order`; apply it with dequant_apply."""
    from ._lib import gptq_dequant_order
    g_host = r["g_idx"].detach().to("cpu", torch.int32)
    out = {"qweight": r["qweight"].to(device, torch.int32).contiguous(),
           "scales": r["scales"].to(device, torch.float32).contiguous(),
           "zeros": r["zeros"].to(device).round().to(torch.int32).contiguous(),
           "g_idx": g_host.to(device).contiguous()}
    if g_host.numel() % 32 != 0:
        raise ValueError("dequant_layer: d_in must be a multiple of 32")
    chunks = g_host.view(-1, 32)
    if bool((chunks != chunks[:, :1]).any()):
        out["qweight"], out["g_idx"], out["order"] = gptq_dequant_order(out["qweight"], out["g_idx"], bits)
    return out


def dequant_apply(x: torch.Tensor, layer: Mapping[str, torch.Tensor], bits: int, **kw) -> torch.Tensor:
    """y = x W^T for a layer prepared by dequant_layer (x in the original
    channel order)."""
    from ._lib import gptq_dequant_matmul, gptq_dequant_matmul_ordered
    if "order" in layer:
        return gptq_dequant_matmul_ordered(x, layer["qweight"], layer["scales"], layer["zeros"], layer["g_idx"],
                                           layer["order"], bits, **kw)
    return gptq_dequant_matmul(x, layer["qweight"], layer["scales"], layer["zeros"], layer["g_idx"], bits, **kw)
