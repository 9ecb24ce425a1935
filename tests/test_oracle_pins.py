"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, a brute-force enumeration, an independent route
(naive OBS re-inversion, reversed Cholesky), or a library routine used for a
different purpose (eigvalsh).  A plausible slip in the oracle (a dropped
term, a sign, a transposed operand, the wrong triangle of the factor, a
wrong normaliser) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_spd(d, seed, cond_mix=True):
    g = np.random.default_rng(seed)
    X = g.standard_normal((4 * d + 3, d))
    if cond_mix:
        X = X @ (np.eye(d) + 0.6 * g.standard_normal((d, d)) / np.sqrt(d))
        X *= np.exp(g.standard_normal(d))[None, :]
    H, _ = O.hessian([X])
    return H, X


# ---------------------------------------------------------------- config ----

def test_validation_rules_from_pages():
    gold = _gold("pages_numbers.json")["bits_choices"]
    for b in gold["valid"]:
        O.validate_config(b, 128, 0.01)
    for b in gold["invalid"]:
        with pytest.raises(ValueError):
            O.validate_config(b, 128, 0.01)
    O.validate_config(4, -1, 0.01)
    for g in (0, -2, -128):
        with pytest.raises(ValueError):
            O.validate_config(4, g, 0.01)
    for dp in (0.0, 1.0, -0.1, 1.5):
        with pytest.raises(ValueError):
            O.validate_config(4, 128, dp)
    O.validate_config(4, 128, 1e-6)
    O.validate_config(4, 128, 0.999)


# --------------------------------------------------------------- Hessian ----

def test_hessian_one_hot_closed_form():
    # one-hot token rows: X^T X is diagonal with the per-channel counts
    g = np.random.default_rng(1)
    d, n = 7, 50
    idx = g.integers(0, d, n)
    X = np.zeros((n, d))
    X[np.arange(n), idx] = 1.0
    H, N = O.hessian([X[:20], X[20:]])
    counts = np.bincount(idx, minlength=d)
    assert N == n
    np.testing.assert_array_equal(H, np.diag(2.0 * counts / n))


def test_hessian_constant_columns():
    # a column constant at a gives H_cc = 2 a^2, and H_cd = 2 a b for two constants
    n = 64
    X = np.zeros((n, 3))
    X[:, 0] = 3.0
    X[:, 2] = -0.5
    H, _ = O.hessian([X])
    assert H[0, 0] == 18.0 and H[2, 2] == 0.5 and H[0, 2] == -3.0 and H[1, 1] == 0.0


def test_hessian_chunking_and_objective_link():
    # the chunked sum equals one pass, and (N/2) D H D^T equals ||D X^T||^2
    H1, X = _rand_spd(9, 3)
    H2, n = O.hessian([X[:5], X[5:17], X[17:]])
    np.testing.assert_allclose(H1, H2, rtol=1e-13, atol=1e-13)
    D = np.random.default_rng(4).standard_normal((5, 9))
    direct = float(np.sum((X @ D.T) ** 2))
    via_h = O.recon_error_from_H(D, np.zeros_like(D), H1, n)
    assert abs(direct - via_h) <= 1e-10 * direct
    assert abs(O.recon_error(D, np.zeros_like(D), [X]) - direct) <= 1e-12 * direct


def test_error_scaling_example_from_pages():
    gold = _gold("pages_numbers.json")["error_scaling"]
    X = np.array([gold["inputs"]])               # one token, two input channels
    for k, want in enumerate(gold["output_errors"]):
        D = np.zeros((1, 2))
        D[0, k] = gold["weight_error"]
        got = O.recon_error(D, np.zeros_like(D), [X])
        assert abs(got - want ** 2) <= 1e-12 * max(1.0, want ** 2)


# --------------------------------------------------------------- damping ----

@pytest.mark.parametrize("dp", [0.01, 0.005, 0.3])
def test_damping_makes_spd(dp):
    # rank-deficient H (fewer tokens than channels) becomes SPD with
    # lambda_min >= dp * mean(diag H)
    g = np.random.default_rng(5)
    X = g.standard_normal((4, 12)) * np.exp(g.standard_normal(12))
    H, _ = O.hessian([X])
    assert np.linalg.eigvalsh(H).min() < 1e-9 * np.trace(H)
    Hd, lam = O.damp(H, dp)
    assert lam == pytest.approx(dp * np.trace(H) / 12, rel=1e-14)
    assert np.linalg.eigvalsh(Hd).min() >= lam * (1 - 1e-9)
    # permutation leaves mean(diag) unchanged
    p = g.permutation(12)
    assert O.damp(H[np.ix_(p, p)], dp)[1] == pytest.approx(lam, rel=1e-14)


def test_not_spd_raises():
    H = np.diag([1.0, -1.0, 2.0])
    with pytest.raises(O.NotSPD):
        O.inverse_factor(H)


# -------------------------------------------------------- inverse factor ----

def _reversed_route(H):
    # U = J chol_lower(J H J)^-1 J: a Cholesky of H read from the last index,
    # then a triangular inverse; no explicit inverse of H
    J = np.eye(H.shape[0])[::-1]
    L = np.linalg.cholesky(J @ H @ J)
    return J @ np.linalg.inv(L) @ J


@pytest.mark.parametrize("d,seed", [(5, 0), (16, 1), (40, 2)])
def test_inverse_factor_properties(d, seed):
    H, _ = _rand_spd(d, seed)
    Hd, _ = O.damp(H, 0.01)
    U = O.inverse_factor(Hd)
    assert np.allclose(np.tril(U, -1), 0.0)
    assert np.all(np.diag(U) > 0)
    cond = np.linalg.cond(Hd)
    assert np.abs(U.T @ U @ Hd - np.eye(d)).max() <= cond * 1e-13
    np.testing.assert_allclose(U, _reversed_route(Hd), rtol=1e-8, atol=1e-10 * np.abs(U).max())


def test_inverse_factor_diagonal():
    h = np.array([4.0, 0.25, 9.0])
    np.testing.assert_allclose(O.inverse_factor(np.diag(h)), np.diag(1 / np.sqrt(h)), rtol=1e-15)


# ------------------------------------------------------------- act-order ----

def test_act_order_descending_stable():
    H = np.diag([1.0, 5.0, 5.0, 0.5, 7.0, 1.0])
    np.testing.assert_array_equal(O.act_order(H), [4, 1, 2, 0, 5, 3])


# ------------------------------------------------------------- quantizer ----

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("sym", [True, False])
def test_quantizer_is_nearest_level(bits, sym):
    g = np.random.default_rng(bits * 10 + sym)
    v = g.standard_normal((40, 16)) * 0.05 + (0 if sym else 0.02)
    v[3] = 0.0                                  # degenerate all-zero group
    v[4] = np.abs(v[4])                         # all-positive (range forced to include 0)
    scale, zero = O.quant_params(v, bits, sym)
    maxq = 2 ** bits - 1
    assert np.all(scale > 0)
    assert np.all((zero >= 0) & (zero <= maxq)) and np.all(zero == np.rint(zero))
    if sym:
        assert np.all(zero == 2 ** (bits - 1))
    codes, what = O.quantize_values(v, scale[:, None] * np.ones((1, 16), np.float32),
                                    zero[:, None] * np.ones((1, 16), np.float32), bits)
    assert codes.min() >= 0 and codes.max() <= maxq
    # brute force over every level: the code is the nearest one
    levels = scale[:, None].astype(np.float64) * (np.arange(maxq + 1)[None, :] - zero[:, None])
    for r in range(v.shape[0]):
        dist = np.abs(v[r][:, None] - levels[r][None, :])
        best = dist.min(axis=1)
        got = np.abs(v[r] - what[r])
        # decisions are taken in fp32: allow the fp32 rounding of w itself
        slack = 4 * np.finfo(np.float32).eps * np.abs(v[r]) + 1e-6 * float(scale[r])
        assert np.all(got <= best + slack)
    assert np.all(what[3] == 0.0) and np.all(codes[3] == zero[3])
    # range contains 0 and the extreme weight is representable within one step
    for r in range(v.shape[0]):
        assert np.abs(v[r] - what[r]).max() <= float(scale[r]) * (1.0 if sym else 0.5) + 1e-9


def test_levels_from_pages():
    # b bits give 2^b levels: with unit scale and zero 0 the codes of a wide
    # integer ramp saturate at exactly 2^b distinct values
    gold = _gold("pages_numbers.json")["levels"]["bits_to_levels"]
    for b, n in gold.items():
        v = np.arange(-5.0, 400.0)[None, :]
        ones = np.ones((1, v.shape[1]), np.float32)
        codes, _ = O.quantize_values(v, ones, 0 * ones, int(b))
        assert len(np.unique(codes)) == n


# ----------------------------------------------------- sweep: worked 2x2 ----

def test_worked_two_column_example():
    gd = _gold("worked_2x2.json")
    H = np.array(gd["H"])
    W = np.array([gd["w"]])
    U = O.inverse_factor(H)
    perm = np.arange(2)
    for bs in (None, 1, 2, 128):
        r = O.quantize_layer(W, U, perm, gd["bits"], gd["group_size"], gd["sym"], False, blocksize=bs)
        np.testing.assert_array_equal(r.codes[0], gd["codes_gptq"])
        assert float(r.scales[0, 0]) == pytest.approx(gd["scale"], rel=1e-6)
        assert int(r.zeros[0, 0]) == gd["zero"]
        D = W - r.Q
        assert float((D @ H @ D.T)[0, 0]) == pytest.approx(gd["E_gptq"], rel=1e-5)
        # telescoped loss: sum err^2 is the same quadratic form
        assert float(r.row_loss[0]) == pytest.approx(gd["E_gptq"], rel=1e-5)
    codes_rtn, Q_rtn = O.rtn(W, gd["bits"], gd["group_size"], gd["sym"])
    np.testing.assert_array_equal(codes_rtn[0], gd["codes_rtn"])
    D = W - Q_rtn
    assert float((D @ H @ D.T)[0, 0]) == pytest.approx(gd["E_rtn"], rel=1e-5)
    # exhaustive search over the 16 grid points
    s, z = gd["scale"], gd["zero"]
    best = min(itertools.product(range(4), repeat=2),
               key=lambda c: float((W[0] - s * (np.array(c) - z)) @ H @ (W[0] - s * (np.array(c) - z))))
    assert list(best) == gd["codes_optimal"]
    # the naive OBS route lands on the same codes
    r2 = O.naive_obq(W, H, perm, gd["bits"], gd["group_size"], gd["sym"], False)
    np.testing.assert_array_equal(r2.codes[0], gd["codes_gptq"])


# ------------------------------------------------------ sweep invariants ----

def _small_layer(d_out, d_in, seed, corr=True):
    L = synth.Layer("t", d_out, d_in, 3 * d_in + 5, "f32", "f32", True, False, cfg=99,
                    layer_id=seed, correlated=corr)
    W = synth.weight(L)
    X = synth.activations(L)
    H, n = O.hessian([X])
    return W, X, H, n


CASES = [  # bits, G, sym, desc_act, static
    (4, 8, True, False, False), (4, 8, False, True, False), (3, 4, True, True, True),
    (2, 16, False, False, True), (8, -1, True, False, False), (4, -1, False, True, False),
    (3, 32, True, True, False), (2, 4, True, True, True),
]


@pytest.mark.parametrize("bits,G,sym,desc,static", CASES)
def test_naive_obs_equals_cholesky_route(bits, G, sym, desc, static):
    """The row-read upper factor reproduces the OBS closed form of the
    chapter with explicit re-inversion at every step (so the factor's
    triangle and the normaliser U[q,q] are read correctly)."""
    W, X, H, n = _small_layer(6, 32, 7 + bits)
    p = O.prepare(H, 0.01, desc)
    a = O.quantize_layer(W, p.U, p.perm, bits, G, sym, static, blocksize=None)
    b = O.naive_obq(W, p.Hp, p.perm, bits, G, sym, static)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_allclose(a.row_loss, b.row_loss, rtol=1e-8)


@pytest.mark.parametrize("bits,G,sym,desc,static", CASES)
def test_telescoping_loss(bits, G, sym, desc, static):
    """sum_i err_i^2 = (w - w_hat) Hd (w - w_hat)^T per row: the per-step
    loss increments e^2/[H^-1]_qq of the chapter add up to the objective."""
    W, X, H, n = _small_layer(5, 48, 11 + bits)
    p = O.prepare(H, 0.01, desc)
    r = O.quantize_layer(W, p.U, p.perm, bits, G, sym, static, blocksize=16 if G in (-1, 4, 8, 16, 32) else None)
    D = W - r.Q
    quad = np.einsum("ij,jk,ik->i", D, p.Hd, D)
    np.testing.assert_allclose(r.row_loss, quad, rtol=1e-9)
    # and the chapter's objective through X (undamped H)
    assert O.recon_error(W, r.Q, [X]) == pytest.approx(O.recon_error_from_H(W, r.Q, H, n), rel=1e-10)


@pytest.mark.parametrize("bits,G,sym,desc,static", CASES)
def test_blocked_equals_unblocked(bits, G, sym, desc, static):
    """Lazy batches of B columns give the plain sweep's result whenever G
    divides B or B divides G."""
    W, X, H, n = _small_layer(7, 64, 21 + bits)
    p = O.prepare(H, 0.01, desc)
    ref = O.quantize_layer(W, p.U, p.perm, bits, G, sym, static, blocksize=None)
    for B in (1, 4, 8, 16, 32, 64):
        if G != -1 and not (B % G == 0 or G % B == 0):
            continue
        r = O.quantize_layer(W, p.U, p.perm, bits, G, sym, static, blocksize=B)
        np.testing.assert_array_equal(r.codes, ref.codes)
        np.testing.assert_allclose(r.Q, ref.Q, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r.row_loss, ref.row_loss, rtol=1e-10)
        np.testing.assert_array_equal(r.g_idx, ref.g_idx)


def test_blocked_rejects_straddling_groups():
    W, X, H, n = _small_layer(2, 48, 3)
    p = O.prepare(H, 0.01, False)
    with pytest.raises(ValueError):
        O.quantize_layer(W, p.U, p.perm, 4, 12, True, False, blocksize=8)


def test_diagonal_hessian_is_rtn():
    g = np.random.default_rng(8)
    W = g.standard_normal((9, 40)) * 0.02
    H = np.diag(np.exp(g.standard_normal(40)))
    for bits, G, sym in [(4, 8, True), (3, -1, False), (2, 20, True)]:
        p = O.prepare(H, 0.01, False)
        r = O.quantize_layer(W, p.U, p.perm, bits, G, sym, False, blocksize=None)
        c, Q = O.rtn(W, bits, G, sym)
        np.testing.assert_array_equal(r.codes, c)


def test_scale_invariance_of_codes():
    W, X, H, n = _small_layer(6, 32, 31)
    for k in (-3, 4):
        a = O.prepare(H, 0.01, True)
        b = O.prepare(H * 2.0 ** k, 0.01, True)
        ra = O.quantize_layer(W, a.U, a.perm, 4, 8, True, False)
        rb = O.quantize_layer(W, b.U, b.perm, 4, 8, True, False)
        np.testing.assert_array_equal(ra.codes, rb.codes)
        np.testing.assert_array_equal(a.perm, b.perm)


def test_desc_act_equals_permuted_problem():
    """desc_act=True is the plain sweep on (W[:, p], H[p][:, p]), unpermuted."""
    W, X, H, n = _small_layer(5, 32, 41)
    p = O.prepare(H, 0.01, True)
    assert not np.array_equal(p.perm, np.arange(32))
    r = O.quantize_layer(W, p.U, p.perm, 3, 8, True, False)
    q = O.prepare(H[np.ix_(p.perm, p.perm)], 0.01, False)
    r2 = O.quantize_layer(W[:, p.perm], q.U, q.perm, 3, 8, True, False)
    np.testing.assert_array_equal(r.codes[:, p.perm], r2.codes)
    np.testing.assert_array_equal(r.g_idx[p.perm], r2.g_idx)
    # g_idx for dynamic groups under act-order follows the sweep position
    np.testing.assert_array_equal(r.g_idx[p.perm], np.arange(32) // 8)
    rs = O.quantize_layer(W, p.U, p.perm, 3, 8, True, True)
    np.testing.assert_array_equal(rs.g_idx, np.arange(32) // 8)


@pytest.mark.parametrize("bits,d,G", [(2, 6, -1), (2, 8, 4), (4, 4, -1), (3, 5, -1)])
def test_brute_force_bound(bits, d, G):
    """Over the fixed grid (static groups / one group), no code vector beats
    the true optimum, and GPTQ's result is one of them."""
    g = np.random.default_rng(100 + d + bits)
    W = g.standard_normal((3, d)) * 0.05
    X = g.standard_normal((3 * d, d)) @ (np.eye(d) + 0.8 * g.standard_normal((d, d)))
    H, _ = O.hessian([X])
    p = O.prepare(H, 0.01, False)
    r = O.quantize_layer(W, p.U, p.perm, bits, G, False, True, blocksize=None)
    maxq = 2 ** bits - 1
    gi = np.zeros(d, dtype=int) if G == -1 else np.arange(d) // G
    cands = np.array(list(itertools.product(range(maxq + 1), repeat=d)), dtype=np.float64)
    for row in range(3):
        s = r.scales[gi, row].astype(np.float64)
        z = r.zeros[gi, row].astype(np.float64)
        Qc = s[None, :] * (cands - z[None, :])
        Dc = W[row][None, :] - Qc
        E = np.einsum("ij,jk,ik->i", Dc, p.Hd, Dc)
        Dg = W[row] - r.Q[row]
        Eg = float(Dg @ p.Hd @ Dg)
        assert E.min() <= Eg * (1 + 1e-12)
        assert np.min(np.abs(E - Eg)) <= 1e-12 * max(Eg, 1e-30)    # GPTQ's point is on the grid


def test_gptq_beats_rtn_at_layer_level():
    L = synth.scaled(synth.config_layers(1)[0], d_out=64, d_in=256, n_tokens=1024, correlated=True)
    W = synth.weight(L)
    X = synth.activations(L)
    for kw in (dict(bits=4, group_size=128, sym=True), dict(bits=3, group_size=32, sym=False),
               dict(bits=2, group_size=64, sym=True)):
        res = O.solve_layer(W, [X], desc_act=False, static_groups=False, damp_percent=0.01, **kw)
        _, Qr = O.rtn(W, kw["bits"], kw["group_size"], kw["sym"])
        e_g = O.recon_error(W, res.sweep.Q, [X])
        e_r = O.recon_error(W, Qr, [X])
        assert e_g < e_r


# ------------------------------------------------------------------ pack ----

def _pack_by_strings(codes, bits):
    """Independent construction: write each code's bits LSB-first into a
    character stream, cut it into 32-bit words, read each word back."""
    d_out, d_in = codes.shape
    nw = -(-d_in * bits // 32)
    out = np.zeros((nw, d_out), dtype=np.uint32)
    for n in range(d_out):
        s = "".join(format(int(c), f"0{bits}b")[::-1] for c in codes[n])
        s = s.ljust(32 * nw, "0")
        for w in range(nw):
            out[w, n] = int(s[32 * w:32 * w + 32][::-1], 2)
    return out.view(np.int32)


def test_pack_hand_words():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8]])
    assert O.pack(codes, 4).view(np.uint32)[0, 0] == 0x87654321
    c3 = np.array([[j % 8 for j in range(32)]])
    q3 = O.pack(c3, 3).view(np.uint32)
    assert q3.shape == (3, 1)
    assert q3[0, 0] == 0x88FAC688          # hand-computed: codes 0..7,0,1 + low bits of 2
    np.testing.assert_array_equal(O.pack(c3, 3), _pack_by_strings(c3, 3))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip_and_layout(bits):
    g = np.random.default_rng(bits)
    d_in = 96
    codes = g.integers(0, 2 ** bits, size=(5, d_in))
    q = O.pack(codes, bits)
    assert q.dtype == np.int32 and q.shape == (d_in * bits // 32, 5)
    np.testing.assert_array_equal(O.unpack(q, bits, d_in), codes)
    np.testing.assert_array_equal(q, _pack_by_strings(codes, bits))


def test_pack_density_and_group_count_from_pages():
    gold = _gold("pages_numbers.json")
    dn = gold["int4_density"]
    q = O.pack(np.ones((1, dn["codes"]), dtype=np.int64), dn["bits"])
    assert q.nbytes == dn["bytes"]
    gc = gold["group_count"]
    W = np.random.default_rng(0).standard_normal((gc["d_out"], gc["d_in"])).astype(np.float32) * 0.02
    s, z = O.gptq_oracle._static_params(W, 4, gc["group_size"], True)
    assert s.size == gc["groups"]


# ------------------------------------------------ tie-following (test use) --

def test_follow_takes_only_float_ties():
    """An exact tie: 2-bit asym over a row [0, 3, 1.5] gives scale 1, zero 0,
    and 1.5 sits on the boundary between codes 1 and 2 (rint picks 2).  A
    followed code 1 there is taken; a followed code 3 is not (1.5 is a whole
    step from the 2|3 boundary); U = I keeps the columns independent."""
    W = np.array([[0.0, 3.0, 1.5]])
    U = np.eye(3)
    perm = np.arange(3)
    kw = dict(bits=2, group_size=-1, sym=False, static_groups=False)
    plain = O.quantize_layer(W, U, perm, **kw)
    np.testing.assert_array_equal(plain.codes, [[0, 3, 2]])
    tied = O.quantize_layer(W, U, perm, **kw, follow=np.array([[0, 3, 1]]), tie_tol=1e-6)
    np.testing.assert_array_equal(tied.codes, [[0, 3, 1]])
    assert tied.ties == 1
    np.testing.assert_allclose(tied.Q, [[0.0, 3.0, 1.0]])
    far = O.quantize_layer(W, U, perm, **kw, follow=np.array([[0, 3, 3]]), tie_tol=1e-6)
    np.testing.assert_array_equal(far.codes, [[0, 3, 2]])
    assert far.ties == 0


def test_follow_own_codes_changes_nothing():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((6, 64))
    X = rng.standard_normal((300, 64)) @ rng.standard_normal((64, 64))
    p = O.prepare(O.finalize_hessian(X.T @ X, 300), 0.01, True)
    kw = dict(bits=3, group_size=16, sym=True, static_groups=False)
    a = O.quantize_layer(W, p.U, p.perm, **kw)
    b = O.quantize_layer(W, p.U, p.perm, **kw, follow=a.codes, tie_tol=2.0 ** -12)
    assert b.ties == 0
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.Q, b.Q)
    # codes one level off everywhere are almost never float ties
    c = O.quantize_layer(W, p.U, p.perm, **kw, follow=np.clip(a.codes + 1, 0, 7), tie_tol=2.0 ** -12)
    assert c.ties <= 1


# ----------------------------------------------------- shared-input layers ---

def test_stacked_rows_equal_separate_layers():
    # Layers that read one input share H and U; the sweep treats every output
    # row on its own (each row's compensation only involves that row), so the
    # sweep of the stacked rows [W1; W2] must return exactly the two layers'
    # separate results.  A sweep that mixed rows (a transposed update, a
    # group range taken over the wrong axis) would fail here.
    H, _ = _rand_spd(24, 11)
    p = O.prepare(H, 0.01, desc_act=True)
    g = np.random.default_rng(12)
    W1 = g.standard_normal((5, 24))
    W2 = 3.0 * g.standard_normal((7, 24))
    for static in (False, True):
        both = O.quantize_layer(np.vstack([W1, W2]), p.U, p.perm, 3, 8, False, static)
        a = O.quantize_layer(W1, p.U, p.perm, 3, 8, False, static)
        b = O.quantize_layer(W2, p.U, p.perm, 3, 8, False, static)
        np.testing.assert_array_equal(both.codes, np.vstack([a.codes, b.codes]))
        np.testing.assert_array_equal(both.Q, np.vstack([a.Q, b.Q]))
        np.testing.assert_array_equal(both.scales, np.hstack([a.scales, b.scales]))
        np.testing.assert_array_equal(both.zeros, np.hstack([a.zeros, b.zeros]))


def test_shared_groups_share_x_not_w():
    # the generators' shared groups: one X (the first member's), distinct W
    for cfg in (2, 3, 4):
        for _, members in synth.shared_groups(cfg):
            assert len({(L.seed, L.cfg, L.layer_id, L.d_in, L.n_tokens) for L in members}) == 1
            assert len({L.w_key for L in members}) == len(members)
    q, k, _ = synth.shared_groups(2)[0][1]
    x_q = synth.activation_chunk(q, 0)
    x_k = synth.activation_chunk(k, 0)
    np.testing.assert_array_equal(x_q, x_k)
    assert not np.array_equal(synth.weight(q), synth.weight(k))


def test_quantized_layer_stand_ins():
    # the seeded stand-in tensors of the dequantizing product's long and
    # full-size cases: shapes and dtypes of the stored layer, positive scales,
    # zero points in [0, 2^b), g_idx either k // G or every group exactly G
    # columns (act-order), deterministic in the seed
    for bits, G, act, d_in in [(4, 128, False, 1024), (3, 32, True, 512), (2, 64, True, 320), (8, -1, False, 256)]:
        t = synth.quantized_layer(96, d_in, bits, G, act, seed=5)
        ng = 1 if G == -1 else -(-d_in // G)
        assert t["qweight"].shape == (d_in * bits // 32, 96) and t["qweight"].dtype == np.int32
        assert t["scales"].shape == (ng, 96) and t["scales"].dtype == np.float32 and (t["scales"] > 0).all()
        assert t["zeros"].shape == (ng, 96) and t["zeros"].min() >= 0 and t["zeros"].max() < 2 ** bits
        gi = t["g_idx"]
        assert gi.shape == (d_in,) and gi.dtype == np.int32
        if act:
            assert not np.array_equal(gi, np.arange(d_in) // G)
            counts = np.bincount(gi, minlength=ng)
            assert (counts[:-1] == G).all() and counts[-1] == d_in - G * (ng - 1)
        else:
            np.testing.assert_array_equal(gi, np.arange(d_in) // (d_in if G == -1 else G))
        t2 = synth.quantized_layer(96, d_in, bits, G, act, seed=5)
        for k in t:
            np.testing.assert_array_equal(t[k], t2[k])


# --------------------------------------------------- dequantizing product ---

@pytest.mark.parametrize("bits,G,desc,static", [(4, 8, False, False), (3, 8, True, False), (2, 16, True, True),
                                                (8, -1, False, False)])
def test_dequantize_equals_sweep_q(bits, G, desc, static):
    # the weights rebuilt from the stored tensors (packed codes, per-group
    # scale and zero, g_idx) are the sweep's own dequantized weights, exactly:
    # a wrong group lookup, a transposed parameter table or a bit-order slip
    # in the unpacking changes them
    H, _ = _rand_spd(32, 21)
    p = O.prepare(H, 0.01, desc_act=desc)
    W = np.random.default_rng(22).standard_normal((6, 32))
    sw = O.quantize_layer(W, p.U, p.perm, bits, G, False, static)
    Wq = O.dequantize(O.pack(sw.codes, bits), sw.scales, sw.zeros, sw.g_idx, bits, 32)
    np.testing.assert_array_equal(Wq, sw.Q)
    x = np.random.default_rng(23).standard_normal((3, 32))
    y = O.dequant_matmul(x, O.pack(sw.codes, bits), sw.scales, sw.zeros, sw.g_idx, bits)
    np.testing.assert_allclose(y, np.einsum("mk,nk->mn", x, sw.Q), rtol=1e-12, atol=1e-12)


# ------------------------------------------------ block forward (driver) ---

def test_block_oracle_closed_forms():
    from oracle import block_oracle as B
    g = np.random.default_rng(31)
    # equal keys: every causal attention weight is uniform, so position i gets
    # the mean of the values of positions 0..i
    n_seq, L, heads, d = 2, 5, 2, 8
    q = g.standard_normal((n_seq * L, d))
    k = np.tile(g.standard_normal((1, d)), (n_seq * L, 1))
    v = g.standard_normal((n_seq * L, d))
    out = B.causal_attention(q, k, v, n_seq, L, heads)
    for s in range(n_seq):
        vs = v[s * L:(s + 1) * L]
        np.testing.assert_allclose(out[s * L:(s + 1) * L], np.cumsum(vs, axis=0) / np.arange(1, L + 1)[:, None],
                                   rtol=1e-12, atol=1e-12)
    # the first position attends only to itself
    np.testing.assert_allclose(B.causal_attention(q, g.standard_normal(v.shape), v, n_seq, L, heads)[::L], v[::L],
                               rtol=1e-12, atol=1e-12)
    # zero weights leave the residual stream unchanged; RMSNorm rows have unit RMS
    W = {n: np.zeros((d if n != "gate_proj" and n != "up_proj" else 12, d if n != "down_proj" else 12))
         for n in synth.BLOCK_LINEARS}
    x0 = g.standard_normal((n_seq * L, d))
    st = B.block_stages(W, x0, n_seq, L, heads)
    np.testing.assert_array_equal(st["out"], x0)
    np.testing.assert_allclose(np.sqrt(np.mean(B.rms_norm(x0, 0.0) ** 2, axis=1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(B.silu(np.array([0.0, 40.0, -40.0])), [0.0, 40.0, 0.0], atol=1e-15)


def test_dequant_matmul_channel_order_invariance():
    # the group-ordered product relies on y = x W^T being a sum over the
    # input channels: putting the channels in another order (here the stable
    # sort by group, as the one-time group order does), with x's columns, the
    # codes and g_idx moved alike, leaves y unchanged up to the order of the
    # fp64 sum; after the sort every 32 consecutive channels lie in one group
    for bits, G, d_in in [(4, 32, 384), (3, 32, 256), (8, 128, 512)]:
        t = synth.quantized_layer(40, d_in, bits, G, True, seed=9)
        gi = t["g_idx"]
        order = np.argsort(gi, kind="stable")
        codes = O.unpack(t["qweight"], bits, d_in)
        q_sorted = O.pack(codes[:, order], bits)
        x = np.random.default_rng(bits).standard_normal((3, d_in))
        y = O.dequant_matmul(x, t["qweight"], t["scales"], t["zeros"], gi, bits)
        y_sorted = O.dequant_matmul(x[:, order], q_sorted, t["scales"], t["zeros"], gi[order], bits)
        np.testing.assert_allclose(y_sorted, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
        assert np.all(np.diff(gi[order]) >= 0)
        chunks = gi[order].reshape(-1, 32)
        assert np.all(chunks == chunks[:, :1])
        # and the unsorted act-order layer does have chunks spanning groups
        assert np.any(gi.reshape(-1, 32) != gi.reshape(-1, 32)[:, :1])
