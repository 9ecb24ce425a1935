"""Layer-sequential quantization of one transformer block.

AutoGPTQ examples walkthrough (true_sequential; the layer groups of a
decoder block, inside_layer_modules) and the GPTQ 实战 chapter's layer loop:
calibration activations run through the block, the inputs of the layers about
to be quantized are collected, H is accumulated from them, the layers are
solved, and the following layers see the outputs of the already-quantized
ones.  The groups, in order:

    k_proj, v_proj, q_proj    (one input: the normalized hidden states)
    o_proj                    (the attention output)
    up_proj, gate_proj        (the normalized hidden states after attention)
    down_proj                 (silu(gate) * up)

Each group shares one input, so it is solved against one H and one U
(solve_layers_shared).  The block is Llama-shaped: RMSNorm with unit weights,
causal multi-head attention without position encoding, a SiLU-gated MLP.
The block's own arithmetic (norms, attention, activation) is the driver's
plumbing and runs in torch (fp32); the layer solves run in libgptq.so.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch
import torch.nn.functional as F

from . import solve_layers_shared
from ._lib import QuantizeConfig

QUANT_ORDER: List[List[str]] = [["k_proj", "v_proj", "q_proj"], ["o_proj"], ["up_proj", "gate_proj"],
                                ["down_proj"]]


@dataclass
class Block:
    d_model: int
    n_heads: int
    d_ff: int
    weights: Dict[str, torch.Tensor]  # name -> [d_out, d_in] fp32 on the device
    eps: float = 1e-6


def rms_norm(x: torch.Tensor, eps: float) -> torch.Tensor:
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + eps)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_seq: int, seq_len: int, n_heads: int,
              seqs_per_call: int = 8) -> torch.Tensor:
    """Causal multi-head attention over n_seq sequences of seq_len tokens
    (rows of q, k, v are tokens, sequence-major), fp32, a few sequences per call."""
    d = q.shape[1]
    hd = d // n_heads
    out = torch.empty_like(q)
    for s0 in range(0, n_seq, seqs_per_call):
        s1 = min(n_seq, s0 + seqs_per_call)
        r0, r1 = s0 * seq_len, s1 * seq_len

        def heads(t):
            return t[r0:r1].reshape(s1 - s0, seq_len, n_heads, hd).transpose(1, 2).contiguous()
        o = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
        out[r0:r1] = o.transpose(1, 2).reshape((s1 - s0) * seq_len, d)
    return out


@dataclass
class BlockResult:
    layers: Dict[str, dict] = field(default_factory=dict)   # per layer: solve outputs
    inputs: Dict[str, torch.Tensor] = field(default_factory=dict)  # per group (first member): bf16 input
    output: Optional[torch.Tensor] = None                   # block output with the quantized weights
    ms: Dict[str, float] = field(default_factory=dict)      # forward / solve time per group


def quantize_block(block: Block, x0: torch.Tensor, n_seq: int, seq_len: int, cfg: QuantizeConfig,
                   keep_inputs: bool = False, timed: bool = False) -> BlockResult:
    """Quantize the block's seven layers group by group (true-sequential).
    x0: hidden states entering the block, [n_seq * seq_len, d_model] fp32.
    Each quantized layer's weights are replaced by its dequantized Q before the
    next group's input is computed.  Returns the solve outputs per layer, the
    block output computed with the quantized weights, optionally each group's
    input (bf16, as accumulated into H) and, with `timed`, per-stage times."""
    res = BlockResult()
    W = block.weights
    ev = {}

    def mark(tag):
        if timed:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev[tag] = e

    def solve(group: List[str], inp: torch.Tensor):
        xb = inp.to(torch.bfloat16)
        if keep_inputs:
            res.inputs[group[0]] = xb
        mark(f"solve {'+'.join(group)} start")
        outs = solve_layers_shared([W[n].to(torch.bfloat16) for n in group], [xb], cfg)
        mark(f"solve {'+'.join(group)} end")
        for n, o in zip(group, outs):
            res.layers[n] = o
            W[n] = o["Q"].contiguous()

    mark("forward 1 start")
    xn1 = rms_norm(x0, block.eps)
    mark("forward 1 end")
    solve(QUANT_ORDER[0], xn1)
    mark("forward 2 start")
    att = attention(F.linear(xn1, W["q_proj"]), F.linear(xn1, W["k_proj"]), F.linear(xn1, W["v_proj"]), n_seq,
                    seq_len, block.n_heads)
    mark("forward 2 end")
    solve(QUANT_ORDER[1], att)
    mark("forward 3 start")
    h = x0 + F.linear(att, W["o_proj"])
    xn2 = rms_norm(h, block.eps)
    mark("forward 3 end")
    solve(QUANT_ORDER[2], xn2)
    mark("forward 4 start")
    m = F.silu(F.linear(xn2, W["gate_proj"])) * F.linear(xn2, W["up_proj"])
    mark("forward 4 end")
    solve(QUANT_ORDER[3], m)
    mark("forward 5 start")
    res.output = h + F.linear(m, W["down_proj"])
    mark("forward 5 end")
    if timed:
        torch.cuda.synchronize()
        tags = sorted({t.rsplit(" ", 1)[0] for t in ev})
        res.ms = {t: ev[t + " start"].elapsed_time(ev[t + " end"]) for t in tags}
    return res
