"""MI355X (gfx950) GPTQ per-layer quantization solve.

The four calls of the C ABI (include/gptq.h) with the same names, plus
QuantizeConfig (BaseQuantizeConfig's fields), gptq_dequant_matmul (the
quantized layer applied to activations; gptq_dequant_order and
gptq_dequant_matmul_ordered for act-order layers put in group order once),
solve_layer, which chains them
for one linear layer, and solve_layers_shared, which quantizes several layers
that read the same input (q/k/v, gate/up) against one Hessian and one factor.
All arithmetic runs in libgptq.so's HIP kernels.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import torch

from ._lib import (EXPORTS, GptqError, NonFiniteHessian, NotPositiveDefinite, QuantizeConfig,  # noqa: F401
                   gptq_dequant_matmul, gptq_dequant_matmul_noalloc, gptq_dequant_matmul_ordered,
                   gptq_dequant_noalloc_need, gptq_dequant_order, gptq_dequant_ordered_workspace_size,
                   gptq_dequant_scratch_bytes, gptq_dequant_workspace_size, gptq_hessian_accumulate,
                   gptq_hessian_workspace_size, gptq_pack, gptq_prepare_hinv, gptq_prepare_workspace_size,
                   gptq_quantize_layer, gptq_workspace_size, library_path)

__all__ = ["QuantizeConfig", "GptqError", "NotPositiveDefinite", "NonFiniteHessian", "gptq_hessian_accumulate",
           "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_pack", "gptq_hessian_workspace_size",
           "gptq_prepare_workspace_size", "gptq_workspace_size", "gptq_dequant_matmul", "gptq_dequant_workspace_size",
           "gptq_dequant_order", "gptq_dequant_matmul_ordered", "gptq_dequant_ordered_workspace_size",
           "gptq_dequant_matmul_noalloc", "gptq_dequant_noalloc_need", "gptq_dequant_scratch_bytes", "solve_layer",
           "solve_layers_shared", "library_path"]


def _accumulate(d_in: int, X_chunks: Iterable[torch.Tensor], device, stream):
    S = torch.zeros((d_in, d_in), dtype=torch.float32, device=device)
    n = 0
    ws = None
    for X in X_chunks:
        need = gptq_hessian_workspace_size(d_in, X.shape[0], X.dtype)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        gptq_hessian_accumulate(S, X, ws=ws, stream=stream)
        n += X.shape[0]
    return S, n


def solve_layer(W: torch.Tensor, X_chunks: Iterable[torch.Tensor], cfg: QuantizeConfig, want_q: bool = True,
                stream=None) -> dict:
    """Quantize one linear layer W [d_out, d_in] from calibration activations
    given as token-major chunks [tokens, d_in]: accumulate S, prepare U, sweep,
    pack.  Returns the outputs of gptq_quantize_layer plus qweight, H, U, perm
    and the token count."""
    d_out, d_in = W.shape
    S, n = _accumulate(d_in, X_chunks, W.device, stream)
    U, perm, _ = gptq_prepare_hinv(S, n, cfg, stream=stream)
    out = gptq_quantize_layer(W, U, perm, cfg, want_q=want_q, stream=stream)
    out["qweight"] = gptq_pack(out["codes"], cfg.bits, stream=stream)
    out.update(H=S, U=U, perm=perm, n_tokens=n)
    return out


def solve_layers_shared(Ws: Sequence[torch.Tensor], X_chunks: Iterable[torch.Tensor], cfg: QuantizeConfig,
                        want_q: bool = True, stream=None) -> List[dict]:
    """Quantize layers that read the same input (q/k/v, gate/up; the layers
    AutoGPTQ groups in one step) against one Hessian and one factor: the
    activations are accumulated once, U is prepared once, and the stacked rows
    [W_0; W_1; ...] go through one sweep and one pack.  Output rows are
    independent given U and every product sums in a fixed order, so each
    layer's result equals its own solve_layer with the same U, bit for bit.
    Returns one dict per layer with the keys of solve_layer (codes, Q and
    row_loss rows, scales / zeros / qweight columns as views into the stacked
    outputs; g_idx, H, U and perm shared)."""
    if len(Ws) == 0:
        return []
    d_in = Ws[0].shape[1]
    for W in Ws:
        if W.dim() != 2 or W.shape[1] != d_in or W.dtype != Ws[0].dtype or W.device != Ws[0].device:
            raise ValueError("solve_layers_shared: the layers must share d_in, dtype and device")
    S, n = _accumulate(d_in, X_chunks, Ws[0].device, stream)
    U, perm, _ = gptq_prepare_hinv(S, n, cfg, stream=stream)
    W_all = torch.cat(list(Ws), dim=0)
    out = gptq_quantize_layer(W_all, U, perm, cfg, want_q=want_q, stream=stream)
    qweight = gptq_pack(out["codes"], cfg.bits, stream=stream)
    res = []
    r0 = 0
    for W in Ws:
        r1 = r0 + W.shape[0]
        o = {"codes": out["codes"][r0:r1], "scales": out["scales"][:, r0:r1], "zeros": out["zeros"][:, r0:r1],
             "g_idx": out["g_idx"], "qweight": qweight[:, r0:r1], "H": S, "U": U, "perm": perm, "n_tokens": n}
        if "Q" in out:
            o["Q"] = out["Q"][r0:r1]
        if "row_loss" in out:
            o["row_loss"] = out["row_loss"][r0:r1]
        res.append(o)
        r0 = r1
    return res
