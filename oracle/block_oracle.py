"""CPU fp64 forward of the synthetic transformer block that the
layer-sequential driver quantizes (test infrastructure only).

AutoGPTQ examples walkthrough, true_sequential and the decoder-layer groups:
the driver collects each group's input from the block forward computed with
the already-quantized earlier layers.  The block is Llama-shaped: RMSNorm
(unit weights), causal multi-head attention (no position encoding), SiLU-gated
MLP; every stage is written out plainly here.
"""
import numpy as np


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def linear(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """x [tokens, d_in] times W^T, W [d_out, d_in] (nn.Linear without bias)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_seq: int, seq_len: int,
                     n_heads: int) -> np.ndarray:
    """Rows are tokens, sequence-major; each head attends over positions <= its own."""
    d = q.shape[1]
    hd = d // n_heads
    out = np.zeros((n_seq * seq_len, d))
    for s in range(n_seq):
        rows = slice(s * seq_len, (s + 1) * seq_len)
        for h in range(n_heads):
            cols = slice(h * hd, (h + 1) * hd)
            qs, ks, vs = q[rows, cols], k[rows, cols], v[rows, cols]
            scores = qs @ ks.T / np.sqrt(hd)
            scores = np.where(np.tril(np.ones((seq_len, seq_len), dtype=bool)), scores, -np.inf)
            scores -= scores.max(axis=1, keepdims=True)
            p = np.exp(scores)
            p /= p.sum(axis=1, keepdims=True)
            out[rows, cols] = p @ vs
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def block_stages(W: dict, x0: np.ndarray, n_seq: int, seq_len: int, n_heads: int, eps: float = 1e-6) -> dict:
    """Every intermediate of the block forward: xn1 (input of k/v/q), att
    (input of o), xn2 (input of up/gate), m (input of down) and out."""
    x0 = np.asarray(x0, dtype=np.float64)
    xn1 = rms_norm(x0, eps)
    att = causal_attention(linear(xn1, W["q_proj"]), linear(xn1, W["k_proj"]), linear(xn1, W["v_proj"]),
                           n_seq, seq_len, n_heads)
    h = x0 + linear(att, W["o_proj"])
    xn2 = rms_norm(h, eps)
    m = silu(linear(xn2, W["gate_proj"])) * linear(xn2, W["up_proj"])
    out = h + linear(m, W["down_proj"])
    return dict(xn1=xn1, att=att, h=h, xn2=xn2, m=m, out=out)
