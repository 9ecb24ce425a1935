"""Seeded synthetic inputs for the GPTQ layer solve.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic, so both the oracle's tests and the
HIP path can consume it.  Every array is a deterministic function of
(seed, cfg, layer, role, chunk) through numpy's PCG64 fed by a SeedSequence.

Distributions follow the layer workloads the GPTQ guides describe (weights of
an nn.Linear of shape [d_out, d_in], calibration activations of N tokens):

* weights       W = 0.02 * N(0, 1), optional Bernoulli(0.005) outliers x40
* activations   X[n, c] = sigma_c * z,  z ~ N(0, 1), sigma_c = exp(N(0, 1))
                optional round(0.01 * d_in) outlier channels with sigma x50
* activations are produced in 8192-token chunks, each from its own seed, so
  a consumer can stream them without materialising N x d_in at once.

bf16 storage is produced by integer round-to-nearest-even on the fp32 bits,
so every consumer sees identical bf16 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, List, Optional, Tuple

import numpy as np

CHUNK_TOKENS = 8192

ROLE_W = 0
ROLE_X = 1
ROLE_SIGMA = 2
ROLE_OUTLIER_CH = 3
ROLE_W_OUTLIER = 4
ROLE_MIX = 5
ROLE_QPARAMS = 6


def rng(seed: int, cfg: int, layer: int, role: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, layer, role, chunk])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even on the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 array holding exactly the bf16-representable values nearest to a."""
    return bf16_to_f32(bf16_bits(a))


@dataclass(frozen=True)
class Layer:
    """One synthetic linear layer: W [d_out, d_in] and N calibration tokens."""
    name: str
    d_out: int
    d_in: int
    n_tokens: int
    w_dtype: str            # "f32" | "bf16"
    x_dtype: str            # "f32" | "bf16"
    w_outliers: bool
    x_outlier_channels: bool
    bits: int = 4
    group_size: int = 128
    sym: bool = True
    desc_act: bool = False
    static_groups: bool = False
    damp_percent: float = 0.01
    cfg: int = 1
    layer_id: int = 0
    seed: int = 0
    correlated: bool = False  # mix channels through a random matrix (small tests only)
    w_key: int = -1           # >= 0: W drawn under this key instead of layer_id (layers sharing one X)

    def quant_kwargs(self) -> dict:
        return dict(bits=self.bits, group_size=self.group_size, sym=self.sym,
                    desc_act=self.desc_act, static_groups=self.static_groups,
                    damp_percent=self.damp_percent)

    def n_chunks(self) -> int:
        return (self.n_tokens + CHUNK_TOKENS - 1) // CHUNK_TOKENS


def weight(layer: Layer) -> np.ndarray:
    """W as fp32 (bf16-exact values when the layer stores bf16)."""
    wk = layer.layer_id if layer.w_key < 0 else layer.w_key
    g = rng(layer.seed, layer.cfg, wk, ROLE_W)
    w = g.standard_normal((layer.d_out, layer.d_in), dtype=np.float32) * np.float32(0.02)
    if layer.w_outliers:
        go = rng(layer.seed, layer.cfg, wk, ROLE_W_OUTLIER)
        mask = go.random((layer.d_out, layer.d_in), dtype=np.float32) < np.float32(0.005)
        w = np.where(mask, w * np.float32(40.0), w).astype(np.float32)
    if layer.w_dtype == "bf16":
        w = round_to_bf16(w)
    return np.ascontiguousarray(w, dtype=np.float32)


def channel_sigma(layer: Layer) -> np.ndarray:
    g = rng(layer.seed, layer.cfg, layer.layer_id, ROLE_SIGMA)
    sigma = np.exp(g.standard_normal(layer.d_in)).astype(np.float32)
    if layer.x_outlier_channels:
        k = int(round(0.01 * layer.d_in))
        go = rng(layer.seed, layer.cfg, layer.layer_id, ROLE_OUTLIER_CH)
        idx = go.choice(layer.d_in, size=k, replace=False)
        sigma[idx] *= np.float32(50.0)
    return sigma


def _mixing(layer: Layer) -> Optional[np.ndarray]:
    if not layer.correlated:
        return None
    g = rng(layer.seed, layer.cfg, layer.layer_id, ROLE_MIX)
    return (g.standard_normal((layer.d_in, layer.d_in)) / np.sqrt(layer.d_in)).astype(np.float32)


def activation_chunk(layer: Layer, chunk: int, sigma: Optional[np.ndarray] = None,
                     mix: Optional[np.ndarray] = None) -> np.ndarray:
    """Tokens [chunk*8192, min(N, (chunk+1)*8192)) of X, fp32 (bf16-exact if bf16)."""
    if sigma is None:
        sigma = channel_sigma(layer)
    if mix is None:
        mix = _mixing(layer)
    t0 = chunk * CHUNK_TOKENS
    n = min(layer.n_tokens, t0 + CHUNK_TOKENS) - t0
    if n <= 0:
        return np.zeros((0, layer.d_in), dtype=np.float32)
    g = rng(layer.seed, layer.cfg, layer.layer_id, ROLE_X, chunk)
    z = g.standard_normal((n, layer.d_in), dtype=np.float32)
    if mix is not None:
        z = z @ mix
    x = z * sigma[None, :]
    if layer.x_dtype == "bf16":
        x = round_to_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def activation_chunks(layer: Layer) -> Iterator[np.ndarray]:
    sigma = channel_sigma(layer)
    mix = _mixing(layer)
    for c in range(layer.n_chunks()):
        yield activation_chunk(layer, c, sigma, mix)


def activation_chunks_threaded(layer: Layer, workers: int = 8, as_bf16_bits: bool = False):
    """Same chunks as activation_chunks, produced by a thread pool, in order.
    With as_bf16_bits the chunks come as uint16 bf16 bit patterns."""
    import concurrent.futures as cf
    sigma = channel_sigma(layer)
    mix = _mixing(layer)

    def make(c):
        x = activation_chunk(layer, c, sigma, mix)
        return bf16_bits(x) if as_bf16_bits else x

    with cf.ThreadPoolExecutor(max(1, workers)) as ex:
        futs = [ex.submit(make, c) for c in range(min(layer.n_chunks(), 2 * workers))]
        nxt = len(futs)
        for c in range(layer.n_chunks()):
            x = futs[c].result()
            futs[c] = None
            if nxt < layer.n_chunks():
                futs.append(ex.submit(make, nxt))
                nxt += 1
            yield x


def activations(layer: Layer) -> np.ndarray:
    """All of X [N, d_in] (fp32 values); small layers only."""
    return np.concatenate(list(activation_chunks(layer)), axis=0)


# --------------------------------------------------------------------------
# Workload table: the five layer-solve configurations.
# --------------------------------------------------------------------------

def _cfg1() -> List[Layer]:
    return [Layer("single_768", 768, 768, 2048, "f32", "f32", True, False,
                  bits=4, group_size=128, sym=True, desc_act=False, damp_percent=0.01, cfg=1)]


def _cfg2() -> List[Layer]:
    shapes = [("q_proj", 768, 768), ("k_proj", 768, 768), ("v_proj", 768, 768),
              ("out_proj", 768, 768), ("fc1", 3072, 768), ("fc2", 768, 3072)]
    return [Layer(n, o, i, 16384, "bf16", "f32", False, False, bits=4, group_size=128,
                  sym=False, desc_act=False, damp_percent=0.01, cfg=2, layer_id=k)
            for k, (n, o, i) in enumerate(shapes)]


def _cfg3() -> List[Layer]:
    shapes = [("q_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
              ("down_proj", 4096, 11008)]
    return [Layer(n, o, i, 262144, "bf16", "bf16", True, True, bits=4, group_size=128,
                  sym=True, desc_act=False, damp_percent=0.01, cfg=3, layer_id=k)
            for k, (n, o, i) in enumerate(shapes)]


def _cfg4() -> List[Layer]:
    out = []
    k = 0
    for name, o, i in [("q_proj", 4096, 4096), ("gate_proj", 11008, 4096)]:
        for static in (True, False):
            for bits, g in ((3, 32), (2, 64)):
                out.append(Layer(f"{name}_b{bits}g{g}_{'static' if static else 'dynamic'}", o, i,
                                 131072, "bf16", "bf16", True, True, bits=bits, group_size=g,
                                 sym=True, desc_act=True, static_groups=static,
                                 damp_percent=0.005, cfg=4, layer_id=k))
                k += 1
    return out


def _cfg5() -> List[Layer]:
    shapes = [("q_proj", 8192, 8192), ("gate_proj", 28672, 8192), ("up_proj", 28672, 8192),
              ("down_proj", 8192, 28672)]
    out = [Layer(n, o, i, 262144, "bf16", "bf16", True, True, bits=4, group_size=128, sym=True,
                 desc_act=False, damp_percent=0.01, cfg=5, layer_id=k)
           for k, (n, o, i) in enumerate(shapes)]
    out.append(Layer("q_proj_b8", 8192, 8192, 262144, "bf16", "bf16", True, True, bits=8,
                     group_size=-1, sym=True, desc_act=False, damp_percent=0.01, cfg=5, layer_id=4))
    return out


CONFIGS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


def config_layers(cfg: int) -> List[Layer]:
    return CONFIGS[cfg]()


def shared_groups(cfg: int) -> List[Tuple[str, List[Layer]]]:
    """Layers that read one input and so share one H and one U (q/k/v, gate/up):
    every member has the first member's X (same layer_id) and its own W
    (w_key).  k_proj and v_proj of configurations 3 and 4 are drawn under keys
    past the configuration's layers."""
    out = []
    if cfg == 2:
        q = config_layers(2)[0]
        out.append(("qkv", [replace_layer(q, w_key=0), replace_layer(q, name="k_proj", w_key=1),
                            replace_layer(q, name="v_proj", w_key=2)]))
    elif cfg == 3:
        q, gate = config_layers(3)[0], config_layers(3)[1]
        out.append(("qkv", [replace_layer(q, w_key=0), replace_layer(q, name="k_proj", w_key=10),
                            replace_layer(q, name="v_proj", w_key=11)]))
        out.append(("gate_up", [replace_layer(gate, w_key=1), replace_layer(gate, name="up_proj", w_key=2)]))
    elif cfg == 4:
        q = [L for L in config_layers(4) if L.name == "q_proj_b3g32_dynamic"][0]
        out.append(("qkv", [replace_layer(q, w_key=q.layer_id), replace_layer(q, name="k_proj_b3g32_dynamic", w_key=20),
                            replace_layer(q, name="v_proj_b3g32_dynamic", w_key=21)]))
    return out


def replace_layer(layer: Layer, **kw) -> Layer:
    from dataclasses import replace
    return replace(layer, **kw)


def scaled(layer: Layer, d_out: Optional[int] = None, d_in: Optional[int] = None,
           n_tokens: Optional[int] = None, **over) -> Layer:
    """Same distributions and quant params at a reduced shape (parity tests)."""
    from dataclasses import replace
    kw = dict(over)
    if d_out is not None:
        kw["d_out"] = d_out
    if d_in is not None:
        kw["d_in"] = d_in
    if n_tokens is not None:
        kw["n_tokens"] = n_tokens
    return replace(layer, **kw)


# --------------------------------------------------------------------------
# A synthetic transformer block (random-init weights, synthetic hidden states)
# for the layer-sequential driver.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class BlockShape:
    name: str
    d_model: int
    n_heads: int
    d_ff: int
    seq_len: int
    n_seq: int
    bits: int = 4
    group_size: int = 128
    sym: bool = True
    desc_act: bool = False
    static_groups: bool = False
    damp_percent: float = 0.01
    cfg: int = 6
    seed: int = 0

    def quant_kwargs(self) -> dict:
        return dict(bits=self.bits, group_size=self.group_size, sym=self.sym, desc_act=self.desc_act,
                    static_groups=self.static_groups, damp_percent=self.damp_percent)

    @property
    def n_tokens(self) -> int:
        return self.seq_len * self.n_seq


# the block's linear layers: name -> (d_out, d_in) as functions of the shape
BLOCK_LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")

BLOCKS = {
    "tiny": BlockShape("tiny", d_model=64, n_heads=4, d_ff=160, seq_len=32, n_seq=8, group_size=32),
    "tiny_actorder": BlockShape("tiny_actorder", d_model=64, n_heads=4, d_ff=160, seq_len=32, n_seq=8, bits=3,
                                group_size=32, desc_act=True, seed=1),
    "llama7b": BlockShape("llama7b", d_model=4096, n_heads=32, d_ff=11008, seq_len=2048, n_seq=32),
}


def block_linear_layer(shape: BlockShape, name: str) -> Layer:
    """The Layer whose W is the block's `name` weight (W recipe of the
    configurations, key = position in BLOCK_LINEARS)."""
    d, f = shape.d_model, shape.d_ff
    dims = {"q_proj": (d, d), "k_proj": (d, d), "v_proj": (d, d), "o_proj": (d, d),
            "gate_proj": (f, d), "up_proj": (f, d), "down_proj": (d, f)}
    d_out, d_in = dims[name]
    return Layer(name, d_out, d_in, shape.n_tokens, "bf16", "bf16", False, False, cfg=shape.cfg,
                 layer_id=BLOCK_LINEARS.index(name), seed=shape.seed)


def block_input(shape: BlockShape) -> np.ndarray:
    """Hidden states entering the block, [n_seq * seq_len, d_model] fp32
    (bf16-exact): the activation recipe (log-normal channel scales, 1% outlier
    channels) under the block's own key."""
    L = Layer("block_input", shape.d_model, shape.d_model, shape.n_tokens, "bf16", "bf16", False, True,
              cfg=shape.cfg, layer_id=100, seed=shape.seed)
    return activations(L)


def quantized_layer(d_out: int, d_in: int, bits: int, group_size: int, act_order: bool, seed: int) -> dict:
    """Seeded stand-ins for a quantized layer's stored tensors (the inputs of
    the dequantizing product), drawn directly rather than by a solve:

    * qweight [d_in * bits / 32, d_out] int32: uniformly random words; every
      bit pattern is a packing of codes in [0, 2^bits)
    * scales  [n_groups, d_out] float32: 0.008 exp(0.3 N(0, 1)) (the size of
      a 4-bit step for weights of scale 0.02)
    * zeros   [n_groups, d_out] int32: uniform in [0, 2^bits - 1]
    * g_idx   [d_in] int32: k // G, or with act_order the group of the
      position each column takes in a random permutation (groups formed in
      permuted order), so that groups interleave across k

    n_groups = ceil(d_in / G), with G = d_in when group_size is -1."""
    g = d_in if group_size == -1 else group_size
    n_groups = -(-d_in // g)
    r = rng(seed, 0, d_out * 100003 + d_in, ROLE_QPARAMS)
    qweight = r.integers(-2 ** 31, 2 ** 31, size=(d_in * bits // 32, d_out), dtype=np.int64).astype(np.int32)
    scales = (0.008 * np.exp(0.3 * r.standard_normal((n_groups, d_out)))).astype(np.float32)
    zeros = r.integers(0, 2 ** bits, size=(n_groups, d_out), dtype=np.int64).astype(np.int32)
    if act_order:
        pos = np.empty(d_in, dtype=np.int64)
        pos[r.permutation(d_in)] = np.arange(d_in)
        g_idx = (pos // g).astype(np.int32)
    else:
        g_idx = (np.arange(d_in) // g).astype(np.int32)
    return {"qweight": qweight, "scales": scales, "zeros": zeros, "g_idx": g_idx}
