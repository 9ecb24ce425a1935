"""The dequantizing product y = x W_hat^T against the oracle (fp64).

W_hat is rebuilt from a quantized layer's stored tensors (qweight, scales,
zeros, g_idx): those of an oracle solve for the small cases, seeded stand-ins
(synth.quantized_layer) for the long and full-size ones.  The GPU sums in
fp32.  A chunk of 32 codes that lies in one group is
summed as s (sum_k x_k q_k - z sum_k x_k), at 4 bits with bf16 x (dot and
MFMA forms) as s (sum_k x_k (16 + q_k) - (16 + z) sum_k x_k): every term and partial sum is
then bounded by |x_k| s (q_k + z + c), c = 32 at 4 bits and 0 otherwise (codes
and zero points are non-negative), so the rigorous bound for a sum of d_in
such terms, (d_in + 64) 2^-24 sum_k |x_k| s (q_k + z + c), is used; it also
holds for the paths that form s (q_k - z) per code, since q_k + z >= |q_k - z|.  Cases cover every bit
width, ragged d_out, token counts across the 16-row passes, bf16 and fp32
activations, groups that share a 32-code chunk (one scale per chunk) and
act-order dynamic groups (a scale per code), K ranges of several 16-chunk
stages with a short last one, and the full-size layer shapes of the 7B and 70B
configurations (sampled output columns).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import banner, dev, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import post_weight_quantization_07_amd as G
    assert torch.cuda.is_available()
    return G


def _params(bits, group, desc, static, d_out, d_in, seed):
    L = synth.scaled(synth.config_layers(2)[0], d_out=d_out, d_in=d_in, n_tokens=2048, correlated=True, bits=bits,
                     group_size=group, desc_act=desc, static_groups=static, layer_id=seed)
    res = O.solve_layer(synth.weight(L), [synth.activations(L)], **L.quant_kwargs())
    return res


def _check_tensors(G, qweight, scales, zeros, g_idx, bits, x_host, x_dtype, cols=None, ordered=False):
    """GPU product against the oracle's; with `cols`, only those output
    columns are compared (the oracle dequantizes just them).  With `ordered`,
    the layer is first put in group order on the GPU (gptq_dequant_order) and
    the product runs on it (gptq_dequant_matmul_ordered); the reference is
    still the oracle's product of the original tensors."""
    x = to_dev(x_host, x_dtype)
    xe = host(x).astype(np.float64)  # the exact values the GPU reads
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    if ordered:
        qs, gs, order = G.gptq_dequant_order(d(qweight), d(g_idx), bits)
        y = G.gptq_dequant_matmul_ordered(x, qs, d(scales), d(zeros), gs, order, bits)
    else:
        y = G.gptq_dequant_matmul(x, d(qweight), d(scales), d(zeros), d(g_idx), bits)
    y = y.cpu().numpy().astype(np.float64)
    if cols is not None:
        qweight, scales, zeros, y = qweight[:, cols], scales[:, cols], zeros[:, cols], y[:, cols]
    ref = O.dequant_matmul(xe, qweight, scales, zeros, g_idx, bits)
    # |s| (q + z + c): the dequantized weights with the zero points negated and offset
    c = 32 if bits == 4 else 0
    Wb = O.dequantize(qweight, np.abs(scales), -(zeros.astype(np.int64) + c), g_idx, bits, xe.shape[1])
    bound = (xe.shape[1] + 64) * 2.0 ** -24 * (np.abs(xe) @ Wb.T)
    err = np.abs(y - ref)
    assert np.all(err <= bound + 1e-30), float(np.max(err / (bound + 1e-30)))
    return float(np.max(err / (bound + 1e-30)))


def _check(G, res, bits, x_host, x_dtype):
    sw = res.sweep
    return _check_tensors(G, res.qweight.astype(np.int32), sw.scales.astype(np.float32), sw.zeros.astype(np.int32),
                          sw.g_idx.astype(np.int32), bits, x_host, x_dtype)


CASES = [  # bits, group, desc_act, static, d_out, d_in
    (4, 128, False, False, 200, 512),
    (3, 32, True, False, 96, 256),     # act-order dynamic groups: a scale per code
    (2, 64, True, True, 130, 256),     # act-order static groups: chunks inside one group
    (8, -1, False, False, 64, 128),    # one group per row
    (4, 32, True, False, 70, 384),
]


@pytest.mark.parametrize("bits,group,desc,static,d_out,d_in", CASES)
@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 40])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_dequant_matmul_small(G, bits, group, desc, static, d_out, d_in, m, x_dtype):
    banner(f"dequant b{bits} g{group} desc={desc} static={static} {d_out}x{d_in} m={m} x={x_dtype}")
    res = _params(bits, group, desc, static, d_out, d_in, 7 * bits + d_out)
    x = np.random.default_rng(m).standard_normal((m, d_in)).astype(np.float32)
    _check(G, res, bits, x, x_dtype)


# K ranges of several 16-chunk stages with a short last stage (515 chunks in
# slices of 17 on the 16-token path), ragged columns and a ragged last group;
# 1 and 2 tokens take the VALU kernel over 58 K slices of 9 chunks (the reduction
# runs three loads-of-16 passes and a tail)
@pytest.mark.parametrize("bits,group,act", [(4, 128, False), (2, 64, False), (3, 128, False), (8, 128, False),
                                            (4, 128, True)])
@pytest.mark.parametrize("m", [1, 2, 16, 40])
def test_dequant_matmul_long_k(G, bits, group, act, m):
    d_out, d_in = 1000, 16480
    banner(f"dequant long K b{bits} g{group} act={act} {d_out}x{d_in} m={m}")
    t = synth.quantized_layer(d_out, d_in, bits, group, act, seed=bits)
    x = synth.round_to_bf16(np.random.default_rng(m).standard_normal((m, d_in)).astype(np.float32))
    _check_tensors(G, t["qweight"], t["scales"], t["zeros"], t["g_idx"], bits, x, "bf16")


# the layer shapes of the 7B and 70B configurations at full size, 192 sampled
# output columns (both ends and random ones) checked against the oracle
@pytest.mark.parametrize("d_out,d_in", [(4096, 4096), (28672, 8192), (8192, 28672)])
@pytest.mark.parametrize("m", [1, 16])
def test_dequant_matmul_full_layer(G, d_out, d_in, m):
    banner(f"dequant full layer {d_out}x{d_in} m={m}")
    t = synth.quantized_layer(d_out, d_in, 4, 128, False, seed=3)
    x = synth.round_to_bf16(np.random.default_rng(100 + m).standard_normal((m, d_in)).astype(np.float32))
    r = np.random.default_rng(d_out)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(d_out - 64, d_out), r.integers(0, d_out, 64)]))
    worst = _check_tensors(G, t["qweight"], t["scales"], t["zeros"], t["g_idx"], 4, x, "bf16", cols=cols)
    print(f"  worst error / bound {worst:.3e}", flush=True)


# act-order layers put in group order once: the order is the stable sort of
# the channels by group, g_idx follows it, and every reordered code is the
# original code of its channel (bit-exact)
@pytest.mark.parametrize("bits,group,d_out,d_in", [(3, 32, 96, 256), (4, 32, 70, 384), (2, 64, 130, 512),
                                                   (8, 128, 33, 1024), (4, 128, 1000, 16480)])
def test_dequant_order(G, bits, group, d_out, d_in):
    banner(f"dequant order b{bits} g{group} {d_out}x{d_in}")
    t = synth.quantized_layer(d_out, d_in, bits, group, True, seed=11 * bits)
    dq = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    qs, gs, order = G.gptq_dequant_order(dq(t["qweight"]), dq(t["g_idx"]), bits)
    order, gs, qs = order.cpu().numpy(), gs.cpu().numpy(), qs.cpu().numpy()
    g = t["g_idx"]
    assert np.array_equal(np.sort(order), np.arange(d_in))
    assert np.array_equal(gs, g[order])
    # sorted by group, channels of one group in increasing k: the stable order
    assert np.all((gs[1:] > gs[:-1]) | ((gs[1:] == gs[:-1]) & (order[1:] > order[:-1])))
    codes = O.unpack(t["qweight"], bits, d_in)
    assert np.array_equal(O.unpack(qs, bits, d_in), codes[:, order])


# the product on the reordered layer equals the oracle's product of the
# original one, within the same bound (a permutation of the sum's terms)
@pytest.mark.parametrize("bits,group,desc,static,d_out,d_in", [c for c in CASES if c[2]])
@pytest.mark.parametrize("m", [1, 2, 16, 40])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_dequant_matmul_ordered_small(G, bits, group, desc, static, d_out, d_in, m, x_dtype):
    banner(f"dequant ordered b{bits} g{group} static={static} {d_out}x{d_in} m={m} x={x_dtype}")
    res = _params(bits, group, desc, static, d_out, d_in, 7 * bits + d_out)
    x = np.random.default_rng(m).standard_normal((m, d_in)).astype(np.float32)
    sw = res.sweep
    _check_tensors(G, res.qweight.astype(np.int32), sw.scales.astype(np.float32), sw.zeros.astype(np.int32),
                   sw.g_idx.astype(np.int32), bits, x, x_dtype, ordered=True)


@pytest.mark.parametrize("d_out,d_in,bits,group,m", [(1000, 16480, 4, 128, 1), (1000, 16480, 4, 128, 16),
                                                     (1000, 16480, 3, 32, 2), (28672, 8192, 4, 128, 16)])
def test_dequant_matmul_ordered_long(G, d_out, d_in, bits, group, m):
    banner(f"dequant ordered long b{bits} g{group} {d_out}x{d_in} m={m}")
    t = synth.quantized_layer(d_out, d_in, bits, group, True, seed=5)
    x = synth.round_to_bf16(np.random.default_rng(200 + m).standard_normal((m, d_in)).astype(np.float32))
    cols = None
    if d_out > 4096:
        r = np.random.default_rng(d_out)
        cols = np.unique(np.concatenate([np.arange(64), np.arange(d_out - 64, d_out), r.integers(0, d_out, 64)]))
    _check_tensors(G, t["qweight"], t["scales"], t["zeros"], t["g_idx"], bits, x, "bf16", cols=cols, ordered=True)
