"""MI355X (gfx950) GPTQ per-layer quantization solve.

The four calls of the C ABI (include/gptq.h) with the same names, plus
QuantizeConfig (BaseQuantizeConfig's fields) and solve_layer, which chains
them for one linear layer.  All arithmetic runs in libgptq.so's HIP kernels.
"""
from __future__ import annotations

from typing import Iterable, Optional

import torch

from ._lib import (EXPORTS, GptqError, NotPositiveDefinite, QuantizeConfig, gptq_hessian_accumulate,  # noqa: F401
                   gptq_hessian_workspace_size, gptq_pack, gptq_prepare_hinv, gptq_prepare_workspace_size,
                   gptq_quantize_layer, gptq_workspace_size, library_path)

__all__ = ["QuantizeConfig", "GptqError", "NotPositiveDefinite", "gptq_hessian_accumulate", "gptq_prepare_hinv",
           "gptq_quantize_layer", "gptq_pack", "gptq_hessian_workspace_size", "gptq_prepare_workspace_size",
           "gptq_workspace_size", "solve_layer", "library_path"]


def solve_layer(W: torch.Tensor, X_chunks: Iterable[torch.Tensor], cfg: QuantizeConfig, want_q: bool = True,
                stream=None) -> dict:
    """Quantize one linear layer W [d_out, d_in] from calibration activations
    given as token-major chunks [tokens, d_in]: accumulate S, prepare U, sweep,
    pack.  Returns the outputs of gptq_quantize_layer plus qweight, H, U, perm
    and the token count."""
    d_out, d_in = W.shape
    S = torch.zeros((d_in, d_in), dtype=torch.float32, device=W.device)
    n = 0
    ws = None
    for X in X_chunks:
        need = gptq_hessian_workspace_size(d_in, X.shape[0], X.dtype)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=W.device)
        gptq_hessian_accumulate(S, X, ws=ws, stream=stream)
        n += X.shape[0]
    U, perm, _ = gptq_prepare_hinv(S, n, cfg, stream=stream)
    out = gptq_quantize_layer(W, U, perm, cfg, want_q=want_q, stream=stream)
    out["qweight"] = gptq_pack(out["codes"], cfg.bits, stream=stream)
    out.update(H=S, U=U, perm=perm, n_tokens=n)
    return out
