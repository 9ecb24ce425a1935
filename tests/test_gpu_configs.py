"""Parity on every layer of the five layer-solve configurations, at full size.

Configurations 1 and 2 (d_in <= 3072, N <= 16384) are small enough for the
whole fp64 oracle solve: H, the ordering, the codes of a sweep that uses the
GPU's factor, the reconstruction error against the oracle's own solve, pack.

Configurations 3-5 run the GPU path in the launch configuration bench.py
times (one accumulate call over all N tokens, prepare, quantize, pack) and
check what the oracle can compute one by one or what holds at any size:
- H: a block of sampled channels (all their pairs, diagonal included) in fp64;
- ordering and g_idx bit-exact (stable sort of the GPU's own fp32 diagonal);
- the factor: upper triangular, and the two-sided residual
  || U H_p U^T e_j - e_j || on sampled sweep positions (U H_p U^T = I exactly);
  on config 3's q_proj also the oracle's fp64 factor of the GPU's H;
- the sweep on sampled output rows (rows are independent given U): codes
  (the oracle follows the GPU's decision only at float ties, where both codes
  are correct, so one tie does not turn the rest of its row into mismatches),
  reconstruction error through H, pack words.
X is generated chunk by chunk from the seeded generators and streamed to the
device; only the sampled channels stay on the host.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import banner, dev, rel_fro, sweep_parity, to_dev

pytestmark = pytest.mark.gpu
EPS32 = 2.0 ** -24


def _params(cfgs):
    out = []
    for c in cfgs:
        for L in synth.config_layers(c):
            marks = [pytest.mark.slow] if L.n_tokens * L.d_in >= 262144 * 8192 else []
            out.append(pytest.param(c, L.name, id=f"cfg{c}-{L.name}", marks=marks))
    return out


def _layer(cfg, name):
    return [L for L in synth.config_layers(cfg) if L.name == name][0]


@pytest.fixture(scope="module")
def G():
    import post_weight_quantization_07_amd as G
    assert torch.cuda.is_available()
    return G


# ------------------------------------------------------------ configs 1, 2 --

@pytest.mark.parametrize("cfg,name", _params([1, 2]))
def test_config_whole_oracle(G, cfg, name):
    L = _layer(cfg, name)
    banner(f"cfg{cfg} {name} {L.d_out}x{L.d_in} N={L.n_tokens} x={L.x_dtype} w={L.w_dtype} {L.quant_kwargs()}")
    W = synth.weight(L)
    X = synth.activations(L)
    qk = L.quant_kwargs()
    cfg_g = G.QuantizeConfig(**qk)
    out = G.solve_layer(to_dev(W, L.w_dtype), [to_dev(X, L.x_dtype)], cfg_g)
    torch.cuda.synchronize()
    res = O.solve_layer(W, [X], **qk)
    H_g = out["H"].cpu().numpy().astype(np.float64)
    assert rel_fro(H_g, res.prep.H) <= 1e-5
    perm_g = out["perm"].cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(perm_g, O.act_order(H_g) if L.desc_act else np.arange(L.d_in))
    # the sweep with the GPU's factor: codes decided in fp32 on both sides,
    # float ties followed
    U_g = out["U"].cpu().numpy().astype(np.float64)
    codes = out["codes"].cpu().numpy().astype(np.int64)
    ref, mism, ties = sweep_parity(W, U_g, perm_g, L, codes)
    np.testing.assert_array_equal(out["g_idx"].cpu().numpy(), ref.g_idx)
    # reconstruction error against the oracle's own solve, through X
    e_g = O.recon_error(W, out["Q"].cpu().numpy(), [X])
    e_r = O.recon_error(W, res.sweep.Q, [X])
    print(f"  code mismatch {mism:.4%} (float ties followed {ties:.4%}); recon gpu/oracle {e_g / e_r:.5f}",
          flush=True)
    assert mism <= 1e-3 and ties <= 1e-3
    assert abs(e_g / e_r - 1.0) <= 0.01
    np.testing.assert_array_equal(out["qweight"].cpu().numpy(), O.pack(codes, L.bits))


# --------------------------------------------------------- configs 3, 4, 5 --

def _stream_x(layer, cols):
    """X on the device (one tensor, bf16) and the fp64 values of channels `cols`."""
    X = torch.empty((layer.n_tokens, layer.d_in), dtype=torch.bfloat16, device=dev())
    sub = np.empty((layer.n_tokens, len(cols)), dtype=np.float64)
    r = 0
    for bits in synth.activation_chunks_threaded(layer, workers=16, as_bf16_bits=True):
        n = bits.shape[0]
        X[r:r + n].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
        sub[r:r + n] = synth.bf16_to_f32(np.ascontiguousarray(bits[:, cols]))
        r += n
    assert r == layer.n_tokens
    return X, sub


def _two_sided_residual(U, hp_matvec, js):
    """|| U H_p U^T e_j - e_j || for sweep positions js (fp64)."""
    out = []
    for j in js:
        y = U[j].astype(np.float64)              # U^T e_j = row j of U
        w = _rows_matvec(U, hp_matvec(y))
        w[j] -= 1.0
        out.append(float(np.linalg.norm(w)))
    return np.array(out)


def _rows_matvec(M, v, block=2048):
    out = np.empty(M.shape[0])
    for a in range(0, M.shape[0], block):
        out[a:a + block] = M[a:a + block].astype(np.float64) @ v
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,name", _params([3, 4, 5]))
def test_config_sampled(G, cfg, name):
    L = _layer(cfg, name)
    d, N = L.d_in, L.n_tokens
    banner(f"cfg{cfg} {name} {L.d_out}x{d} N={N} {L.quant_kwargs()}")
    rng = np.random.default_rng(1000 * cfg + L.layer_id)
    cols = np.sort(rng.choice(d, size=96, replace=False))
    X, sub = _stream_x(L, cols)
    W_host = synth.weight(L)
    W = torch.from_numpy(synth.bf16_bits(W_host).view(np.int16)).to(dev()).view(torch.bfloat16)
    cfg_g = G.QuantizeConfig(**L.quant_kwargs())
    S = torch.zeros((d, d), dtype=torch.float32, device=dev())
    G.gptq_hessian_accumulate(S, X)
    S_blk = S[cols][:, cols].cpu().numpy().astype(np.float64)
    del X
    U, perm, info = G.gptq_prepare_hinv(S, N, cfg_g)
    out = G.gptq_quantize_layer(W, U, perm, cfg_g)
    qw = G.gptq_pack(out["codes"], cfg_g.bits)
    torch.cuda.synchronize()
    print("  gpu solve done", flush=True)

    # H: every pair of the sampled channels, diagonal included, against fp64 sums
    ref = sub.T @ sub
    dg = np.sqrt(np.outer(np.diag(ref), np.diag(ref)))
    assert np.max(np.abs(S_blk - ref) / dg) <= 1e-5
    assert np.array_equal(S_blk, S_blk.T)
    H_blk = S[cols][:, cols].cpu().numpy().astype(np.float64)   # S now holds H = 2 S / N
    assert rel_fro(H_blk, O.finalize_hessian(S_blk, N)) <= 1e-6

    # ordering: bit-exact against the oracle's stable sort of the GPU's own fp32 diagonal
    H_g = S.cpu().numpy()
    perm_g = perm.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(perm_g, O.act_order(H_g) if L.desc_act else np.arange(d))

    # factor: upper triangular; two-sided residual on sampled sweep positions
    assert float(torch.tril(U, -1).abs().max()) == 0.0
    lam = L.damp_percent * float(np.mean(np.diag(H_g).astype(np.float64)))
    U_g = U.cpu().numpy()

    def hp_matvec(y):
        # H_p y with H_p = (H + lam I)[perm][:, perm]
        yo = np.zeros(d)
        yo[perm_g] = y
        z = _rows_matvec(H_g, yo) + lam * yo
        return z[perm_g]

    js = np.sort(rng.choice(d, size=8, replace=False))
    res = _two_sided_residual(U_g, hp_matvec, js)
    tol = 8.0 * d * EPS32
    print(f"  two-sided residual max {res.max():.3e} (tol {tol:.3e})", flush=True)
    if cfg == 3 and name == "q_proj":
        p = O.prepare(H_g.astype(np.float64), L.damp_percent, L.desc_act)
        ev = np.linalg.eigvalsh(p.Hp)
        kappa = float(ev[-1] / ev[0])
        err = rel_fro(U_g, p.U)
        res_o = _two_sided_residual(p.U, hp_matvec, js)
        print(f"  cond(H_p) {kappa:.3e}, U rel err vs oracle factor {err:.3e}, "
              f"oracle factor residual {res_o.max():.3e}", flush=True)
        assert err <= 50 * kappa * EPS32 + 1e-6
        assert res_o.max() <= 1e-9
    assert res.max() <= tol

    # sweep on sampled output rows with the GPU's factor and order
    rows = np.sort(rng.choice(L.d_out, size=64, replace=False))
    codes = out["codes"].cpu().numpy()[rows].astype(np.int64)
    ref, mism, ties = sweep_parity(W_host[rows], U_g, perm_g, L, codes)
    np.testing.assert_array_equal(out["g_idx"].cpu().numpy(), ref.g_idx)
    Q = out["Q"].cpu().numpy()[rows].astype(np.float64)
    D_g = W_host[rows] - Q
    D_r = W_host[rows] - ref.Q
    e_g = float(np.sum(_rows_matvec_t(H_g, D_g) * D_g))
    e_r = float(np.sum(_rows_matvec_t(H_g, D_r) * D_r))
    print(f"  sampled rows: code mismatch {mism:.5%} (float ties followed {ties:.5%}), "
          f"recon ratio {e_g / e_r:.5f}", flush=True)
    assert mism <= 1e-3 and ties <= 1e-3
    assert abs(e_g / e_r - 1.0) <= 0.01
    np.testing.assert_array_equal(qw.cpu().numpy()[:, rows], O.pack(codes, L.bits))


def _rows_matvec_t(Hs, D, block=2048):
    """D @ H in fp64, H symmetric, taken in row blocks."""
    out = np.zeros((D.shape[0], Hs.shape[0]))
    for a in range(0, Hs.shape[0], block):
        out += D[:, a:a + block] @ Hs[a:a + block].astype(np.float64)
    return out
