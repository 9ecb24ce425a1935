"""gptq_dequant_matmul_noalloc (the dequantizing product on the library's fixed
scratch buffer) against gptq_dequant_matmul with a caller workspace: the same
kernels on the same inputs, so y must agree bit for bit.  Calls run back to
back, each later one on a smaller input than the one before, so a call that
read a partial sum it had not written (stale contents of the shared buffer)
would show.  A call that needs more than the buffer is rejected on the host."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import banner, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import post_weight_quantization_07_amd as G
    assert torch.cuda.is_available()
    return G


def _layer(d_out, d_in, bits, group, act, seed):
    t = synth.quantized_layer(d_out, d_in, bits, group, act, seed=seed)
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev()) for k, v in t.items()}


def _x(m, d_in, dtype, seed):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal((m, d_in)).astype(np.float32))
    return (x.to(torch.bfloat16) if dtype == "bf16" else x).to(dev())


# (d_out, d_in, bits, group, act-order, m, x dtype): largest first, then smaller
SEQUENCES = [
    [(8192, 28672, 4, 128, False, 8, "bf16"), (4096, 4096, 4, 128, False, 1, "bf16")],
    [(28672, 8192, 4, 128, False, 16, "bf16"), (11008, 4096, 3, 32, True, 5, "bf16"),
     (1000, 2048, 2, 64, False, 2, "f32")],
    [(4096, 11008, 8, -1, False, 40, "bf16"), (4096, 11008, 8, -1, False, 19, "bf16")],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_call(G, seq):
    cap = G.gptq_dequant_scratch_bytes()
    assert cap == 16 << 20
    for i, (d_out, d_in, bits, group, act, m, xdt) in enumerate(SEQUENCES[seq]):
        g = group if group > 0 else d_in
        banner(f"noalloc call {i}: {d_out}x{d_in} b{bits} g{group} act={act} m={m} x={xdt}")
        t = _layer(d_out, d_in, bits, g, act, seed=17 + 3 * seq + i)
        x = _x(m, d_in, xdt, seed=100 * seq + i)
        need = G.gptq_dequant_noalloc_need(m, x.dtype, d_in, bits, d_out)
        assert 0 < need <= cap
        y_ref = G.gptq_dequant_matmul(x, t["qweight"], t["scales"], t["zeros"], t["g_idx"], bits)
        y = torch.full((m, d_out), float("nan"), dtype=torch.float32, device=dev())
        G.gptq_dequant_matmul_noalloc(x, t["qweight"], t["scales"], t["zeros"], t["g_idx"], bits, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i}: max |dy| {float((y - y_ref).abs().max())}"


def test_noalloc_rejects_oversize(G):
    # fp32 x with 16 tokens on a 28672 x 8192 layer needs 29.4 MB of partial sums
    banner("noalloc oversize call")
    d_out, d_in, bits = 28672, 8192, 4
    need = G.gptq_dequant_noalloc_need(16, torch.float32, d_in, bits, d_out)
    assert need > G.gptq_dequant_scratch_bytes()
    t = _layer(d_out, d_in, bits, 128, False, seed=5)
    x = _x(16, d_in, "f32", seed=5)
    y = torch.zeros((16, d_out), dtype=torch.float32, device=dev())
    with pytest.raises(G.GptqError, match="fixed buffer"):
        G.gptq_dequant_matmul_noalloc(x, t["qweight"], t["scales"], t["zeros"], t["g_idx"], bits, y)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0           # nothing was enqueued
