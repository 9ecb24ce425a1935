"""Plain CPU fp64 oracle of the GPTQ per-layer solve.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Every function follows the passage it names.  Page labels used below:

  [guide]  AutoGPTQ examples walkthrough, section 1.4 (BaseQuantizeConfig
           fields and their validation)
  [olmo]   OLMo AutoGPTQ quick-start, section 三 (core API / parameter table)
  [skill]  "gptq" skill card, section 分组量化 (group-wise quantization)
  [blog]   practitioner blog on GPTQ, sections 2.2 (damping) and 2.3 (order)
  [ch5]    GPTQ 实战 chapter 5 (CSDN), sections 5.1.1 (round-to-nearest
           x_q = round(x / s)), 5.1.3 (GPTQ versus plain rounding), 5.1.4
           (reconstruction error), 5.1.7 (Hessian from inputs), 5.1.10
           (group-wise GPTQ),
           5.1.8 ("补偿" closed form; OBS closed form and Cholesky
           acceleration; the implementation-level pseudocode)

Precision: fp64 throughout, inputs taken as their exact fp32/bf16 values.
Where a floating-point value decides an integer (the group scale and zero
point, the rounded code) the decision is taken in fp32, the precision of the
HIP kernels, so both sides round the same quantity the same way.  The pages
fix no precision for it; `decision=np.float64` takes those decisions in fp64
instead (used to measure how many codes the choice moves).

Parity status: every function below is pinned by tests/test_oracle_*.py
(closed forms, brute force, an independent naive-OBS route, hand-derived
worked examples under tests/golden/).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional, Sequence

import numpy as np

VALID_BITS = (2, 3, 4, 8)


class NotSPD(np.linalg.LinAlgError):
    """The damped Hessian is not positive definite (the LinAlgError the blog
    reports in section 2.2 when damp_percent is too small)."""


# ---------------------------------------------------------------------------
# configuration  ([guide] section 1.4, [olmo] section 三 parameter table)
# ---------------------------------------------------------------------------

def validate_config(bits: int, group_size: int, damp_percent: float) -> None:
    """bits must be one of 2/3/4/8; group_size is -1 (one group) or > 0;
    damp_percent lies in the open interval (0, 1).  Raises ValueError."""
    if bits not in VALID_BITS:
        raise ValueError(f"bits must be one of {VALID_BITS}, got {bits}")
    if not (group_size == -1 or group_size > 0):
        raise ValueError(f"group_size must be -1 or > 0, got {group_size}")
    if not (0.0 < damp_percent < 1.0):
        raise ValueError(f"damp_percent must be in (0, 1), got {damp_percent}")


# ---------------------------------------------------------------------------
# Hessian  ([ch5] 5.1.7: H = X X^T up to a constant; the constant is 2/N)
# ---------------------------------------------------------------------------

def hessian_sum(chunks: Iterable[np.ndarray]) -> tuple[np.ndarray, int]:
    """S = sum over token chunks of Xc^T Xc (Xc is tokens x d_in), in fp64."""
    S = None
    n = 0
    for xc in chunks:
        x = np.asarray(xc, dtype=np.float64)
        if S is None:
            S = np.zeros((x.shape[1], x.shape[1]), dtype=np.float64)
        S += x.T @ x
        n += x.shape[0]
    return S, n


def finalize_hessian(S: np.ndarray, n_tokens: int) -> np.ndarray:
    """H = (2 / N) * S."""
    return (2.0 / float(n_tokens)) * np.asarray(S, dtype=np.float64)


def hessian(chunks: Iterable[np.ndarray]) -> tuple[np.ndarray, int]:
    S, n = hessian_sum(chunks)
    return finalize_hessian(S, n), n


# ---------------------------------------------------------------------------
# damping, ordering and the inverse factor
# ---------------------------------------------------------------------------

def damp(H: np.ndarray, damp_percent: float) -> tuple[np.ndarray, float]:
    """[ch5] 5.1.8 damping: H <- H + lambda * mean(diag H) * I with
    lambda = damp_percent ([blog] 2.2 gives the same mean-of-diagonal form)."""
    H = np.asarray(H, dtype=np.float64)
    lam = float(damp_percent) * float(np.mean(np.diag(H)))
    Hd = H + lam * np.eye(H.shape[0])
    return Hd, lam


def act_order(H: np.ndarray) -> np.ndarray:
    """desc_act ([guide] 1.4, [olmo] 三): process columns by descending
    activation energy, read as descending diag(H); ties keep the lower
    original index first (a stable sort)."""
    d = np.asarray(np.diag(H), dtype=np.float64)
    return np.argsort(-d, kind="stable").astype(np.int64)


def inverse_factor(Hp: np.ndarray) -> np.ndarray:
    """[ch5] 5.1.8 "Hinv = Cholesky(inverse(H))": invert once, then take the
    Cholesky factor.  Returned as the upper-triangular U with H^-1 = U^T U,
    whose rows the column sweep reads.  Raises NotSPD when either step fails."""
    Hp = np.asarray(Hp, dtype=np.float64)
    try:
        np.linalg.cholesky(Hp)               # H itself must be SPD
        A = np.linalg.inv(Hp)
        A = 0.5 * (A + A.T)
        L = np.linalg.cholesky(A)
    except np.linalg.LinAlgError as exc:     # pragma: no cover - exercised in tests
        raise NotSPD(str(exc)) from exc
    return np.ascontiguousarray(L.T)


@dataclass
class Prepared:
    H: np.ndarray          # undamped, fp64
    Hd: np.ndarray         # damped, original order
    lam: float
    perm: np.ndarray       # sweep position -> original column
    Hp: np.ndarray         # damped, permuted
    U: np.ndarray          # upper factor of Hp^-1


def prepare(H: np.ndarray, damp_percent: float, desc_act: bool) -> Prepared:
    H = np.asarray(H, dtype=np.float64)
    Hd, lam = damp(H, damp_percent)
    perm = act_order(H) if desc_act else np.arange(H.shape[0], dtype=np.int64)
    Hp = Hd[np.ix_(perm, perm)]
    U = inverse_factor(Hp)
    return Prepared(H=H, Hd=Hd, lam=lam, perm=perm, Hp=Hp, U=U)


# ---------------------------------------------------------------------------
# the group quantizer  ([ch5] 5.1.1: x_q = round(x / s), x_hat = s * x_q;
# [ch5] 5.1.10 and
# [skill] 分组量化: each group carries its own scale and zero point;
# [guide] 1.4: sym selects symmetric quantization)
# ---------------------------------------------------------------------------

def quant_params(v: np.ndarray, bits: int, sym: bool, decision=np.float32, zraw: Optional[np.ndarray] = None
                 ) -> tuple[np.ndarray, np.ndarray]:
    """Scale and zero point of one group for every row; v is rows x m.

    The range always contains 0 (lo = min(0, min v), hi = max(0, max v)).
    sym widens it to [-a, a] with a = max|v| and fixes the zero point at the
    middle code 2^(bits-1).  An all-zero group uses [-1, 1].  Decisions are
    taken in `decision` precision (fp32 by default).  Returns (scale,
    zero integral), both of that dtype; zraw, if given, receives the
    pre-rounding zero point -lo / scale (asymmetric only)."""
    f = decision
    maxq = f(2 ** bits - 1)
    vd = np.asarray(v, dtype=np.float64).astype(f)
    lo = np.minimum(vd.min(axis=1), f(0))
    hi = np.maximum(vd.max(axis=1), f(0))
    if sym:
        a = np.maximum(-lo, hi)
        lo, hi = -a, a
    deg = hi == lo
    lo = np.where(deg, f(-1), lo).astype(f)
    hi = np.where(deg, f(1), hi).astype(f)
    scale = ((hi - lo) / maxq).astype(f)
    if sym:
        zero = np.full(scale.shape, f(2 ** (bits - 1)), dtype=f)
    else:
        zr = ((-lo) / scale).astype(f)
        if zraw is not None:
            zraw[...] = zr
        zero = np.rint(zr).astype(f)
    return scale, zero


def quantize_values(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int, want_v: bool = False):
    """code = clamp(rint(w / s) + z, 0, maxq), decided in the precision of
    `scale` (fp32 unless the caller chose fp64); dequantized value
    s * (code - z) (exact in fp64).  want_v also returns the pre-rounding
    value w / s + z of that precision, as fp64."""
    f = scale.dtype.type
    maxq = f(2 ** bits - 1)
    wd = np.asarray(w, dtype=np.float64).astype(f)
    v = (wd / scale).astype(f) + zero
    q = np.clip(np.rint(wd / scale) + zero, f(0), maxq).astype(f)
    what = scale.astype(np.float64) * (q.astype(np.float64) - zero.astype(np.float64))
    if want_v:
        return q.astype(np.int64), what, v.astype(np.float64)
    return q.astype(np.int64), what


# ---------------------------------------------------------------------------
# the column sweep ([ch5] 5.1.8: quantize, compensate, quantize again;
# OBS closed form; lazy batch of 128 columns)
# ---------------------------------------------------------------------------

@dataclass
class SweepResult:
    codes: np.ndarray      # int64 [d_out, d_in], ORIGINAL column order
    Q: np.ndarray          # fp64  [d_out, d_in], original order
    scales: np.ndarray     # fp32  [n_groups, d_out]
    zeros: np.ndarray      # int64 [n_groups, d_out]
    g_idx: np.ndarray      # int64 [d_in], original column -> group
    err: np.ndarray        # fp64  [d_out, d_in], normalised errors, sweep order
    row_loss: np.ndarray   # fp64  [d_out], sum of err^2 per row
    ties: int = 0          # decisions taken from `follow` at float ties
    vals: Optional[np.ndarray] = None  # [d_out, d_in] pre-rounding w / s + z, sweep order (record_v)
    zvals: Optional[np.ndarray] = None  # [n_groups, d_out] pre-rounding -lo / s of dynamic asym zeros (record_v)


def _n_groups(d_in: int, group_size: int) -> int:
    return 1 if group_size == -1 else -(-d_in // group_size)


def _static_params(W: np.ndarray, bits: int, group_size: int, sym: bool, decision=np.float32):
    """Group parameters fixed before the sweep from the un-updated weights of
    each original group (static_groups, [guide] 1.4 / [olmo] 三)."""
    d_out, d_in = W.shape
    ng = _n_groups(d_in, group_size)
    scales = np.zeros((ng, d_out), dtype=decision)
    zeros = np.zeros((ng, d_out), dtype=decision)
    for g in range(ng):
        sl = slice(0, d_in) if group_size == -1 else slice(g * group_size, min(d_in, (g + 1) * group_size))
        scales[g], zeros[g] = quant_params(W[:, sl], bits, sym, decision)
    return scales, zeros


def _group_plan(d_in: int, perm: np.ndarray, group_size: int, static_groups: bool):
    """(group of sweep position i, g_idx per original column, dynamic?)."""
    if group_size == -1:
        return np.zeros(d_in, dtype=np.int64), np.zeros(d_in, dtype=np.int64), False
    if static_groups:
        gpos = perm // group_size
        g_idx = np.arange(d_in) // group_size
        return gpos.astype(np.int64), g_idx.astype(np.int64), False
    gpos = np.arange(d_in) // group_size
    g_idx = np.empty(d_in, dtype=np.int64)
    g_idx[perm] = gpos
    return gpos.astype(np.int64), g_idx, True


def quantize_layer(W: np.ndarray, U: np.ndarray, perm: np.ndarray, bits: int, group_size: int,
                   sym: bool, static_groups: bool, blocksize: Optional[int] = 128,
                   rows: Optional[Sequence[int]] = None, follow: Optional[np.ndarray] = None,
                   tie_tol: float = 0.0, record_v: bool = False, decision=np.float32) -> SweepResult:
    """GPTQ column sweep.

    Definition ([ch5] 5.1.4 objective, 5.1.8 OBS closed form and its Cholesky
    form): columns are fixed one at a time in sweep order; fixing column i to
    its quantized value changes it by e_i = w_i - q_i, and the remaining
    columns take the OBS compensation that keeps the layer objective minimal,
    -e_i / [H_F^-1]_ii * (H_F^-1)_{i, j} over the not-yet-fixed set F.  With
    H_p^-1 = U^T U (U upper), row i of U restricted to j >= i is
    (H_F^-1)_{i, j} / sqrt([H_F^-1]_ii), so the compensation of column j is
    err_i * U[i, j] with err_i = e_i / U[i, i].  blocksize=None runs exactly
    that, one column after another (the "plain" form); `naive_obq` below
    re-inverts H_F instead of using U, and the two are pinned equal.

    An integer blocksize reorders the same sums (the lazy batches of [ch5]
    5.1.8): the plain form is run on each block of `blocksize` columns alone,
    and the compensations the block's columns owe every later column, err_i *
    U[i, j] summed over the block, are applied at the block's end as one
    matrix product.  Column j of a later block receives the same terms as in
    the plain form, only summed in another order, so the two agree exactly in
    real arithmetic when group_size divides the block or the block divides
    group_size (a dynamic group's range must be read after every earlier
    column's compensation has arrived); pinned equal as well.

    rows selects a subset of output rows (rows are independent given U).

    follow (test use): codes [rows, d_in] in original column order produced by
    another implementation.  Where that code and this sweep's differ by one
    and this sweep's pre-rounding value w/s + z lies within tie_tol (in
    quantization steps) of the rounding boundary between them, both codes are
    correct up to rounding of the running weights; the sweep then takes the
    followed code and continues from it (counted in `ties`).  Every other
    decision is this sweep's own.

    record_v keeps every decision's pre-rounding value w / s + z (sweep
    order) in `vals`; decision=np.float64 decides scales, zeros and codes in
    fp64 instead of fp32."""
    W = np.asarray(W, dtype=np.float64)
    if rows is not None:
        W = W[np.asarray(rows)]
    U = np.asarray(U, dtype=np.float64)
    perm = np.asarray(perm, dtype=np.int64)
    d_out, d_in = W.shape
    maxq = 2 ** bits - 1
    G = group_size
    if blocksize is not None and G != -1:
        if not (blocksize % G == 0 or G % blocksize == 0):
            raise ValueError("blocked sweep needs group_size | blocksize or blocksize | group_size")

    ng = _n_groups(d_in, G)
    gpos, g_idx, dynamic = _group_plan(d_in, perm, G, static_groups)
    if dynamic:
        scales = np.zeros((ng, d_out), dtype=decision)
        zeros = np.zeros((ng, d_out), dtype=decision)
    else:
        # G = -1 uses the whole (un-updated) row; static uses original groups
        scales, zeros = _static_params(W, bits, G, sym, decision)

    Wp = W[:, perm].copy()
    follow_p = None if follow is None else np.asarray(follow, dtype=np.int64)[:, perm]
    n_ties = [0]
    codes_p = np.zeros((d_out, d_in), dtype=np.int64)
    Q_p = np.zeros((d_out, d_in), dtype=np.float64)
    Err = np.zeros((d_out, d_in), dtype=np.float64)
    vals = np.zeros((d_out, d_in), dtype=np.float64) if record_v else None
    zvals = np.full((ng, d_out), np.nan) if record_v else None

    def dyn_params(i: int, grp: np.ndarray):
        zr = np.full(d_out, np.nan) if (zvals is not None and not sym) else None
        scales[gpos[i]], zeros[gpos[i]] = quant_params(grp, bits, sym, decision, zr)
        if zr is not None:
            zvals[gpos[i]] = zr

    def step(i: int, cur: np.ndarray, col: int):
        """Quantize sweep column i held in cur[:, col]; return err column."""
        g = gpos[i]
        w = cur[:, col]
        q, what, v = quantize_values(w, scales[g], zeros[g], bits, want_v=True)
        if vals is not None:
            vals[:, i] = v
        if follow_p is not None:
            f = follow_p[:, i]
            tie = (np.abs(q - f) == 1) & (np.abs(v - (np.minimum(q, f) + 0.5)) <= tie_tol)
            if np.any(tie):
                q = np.where(tie, f, q)
                what = scales[g].astype(np.float64) * (q.astype(np.float64) - zeros[g].astype(np.float64))
                n_ties[0] += int(np.sum(tie))
        codes_p[:, i] = q
        Q_p[:, i] = what
        e = w - what
        return e / U[i, i]

    def plain(cur: np.ndarray, lo: int, hi: int, outer: Optional[np.ndarray] = None):
        """The plain form over sweep columns [lo, hi), held in cur[:, 0 : hi -
        lo]: fix each column and compensate the later columns of the range.
        A dynamic group starting here takes its range from cur, or, for groups
        wider than a block (they start where a block starts, so nothing in
        their range has been touched yet), from `outer`, the whole running
        matrix."""
        for i in range(lo, hi):
            c = i - lo
            if dynamic and i % G == 0:
                wide = outer is not None and G > blocksize
                dyn_params(i, outer[:, i:i + G] if wide else cur[:, c:c + G])
            err = step(i, cur, c)
            Err[:, i] = err
            cur[:, c + 1:] -= np.outer(err, U[i, i + 1:hi])

    if blocksize is None:
        plain(Wp, 0, d_in)
    else:
        B = blocksize
        for b0 in range(0, d_in, B):
            b1 = min(b0 + B, d_in)
            Wb = Wp[:, b0:b1].copy()
            plain(Wb, b0, b1, outer=Wp)
            Wp[:, b0:b1] = Wb
            if b1 < d_in:  # what the block's columns owe the later ones
                Wp[:, b1:] -= Err[:, b0:b1] @ U[b0:b1, b1:]

    codes = np.empty_like(codes_p)
    Q = np.empty_like(Q_p)
    codes[:, perm] = codes_p
    Q[:, perm] = Q_p
    return SweepResult(codes=codes, Q=Q, scales=scales, zeros=zeros.astype(np.int64), g_idx=g_idx,
                       err=Err, row_loss=np.sum(Err * Err, axis=1), ties=n_ties[0], vals=vals, zvals=zvals)


def naive_obq(W: np.ndarray, Hp: np.ndarray, perm: np.ndarray, bits: int, group_size: int,
              sym: bool, static_groups: bool) -> SweepResult:
    """The slow route the chapter contrasts with Cholesky ([ch5] 5.1.8, "朴素
    做法太慢"): before each column is fixed, re-invert the damped Hessian
    restricted to the not-yet-quantized columns and apply the OBS update
    delta = -(w_q - quant(w_q)) / [H_F^-1]_qq * (H_F^-1)_{:,q} to them.
    No Cholesky factor is used.  O(d^4); tiny inputs only."""
    W = np.asarray(W, dtype=np.float64)
    Hp = np.asarray(Hp, dtype=np.float64)
    d_out, d_in = W.shape
    G = group_size
    ng = _n_groups(d_in, G)
    gpos, g_idx, dynamic = _group_plan(d_in, perm, G, static_groups)
    if dynamic:
        scales = np.zeros((ng, d_out), dtype=np.float32)
        zeros = np.zeros((ng, d_out), dtype=np.float32)
    else:
        scales, zeros = _static_params(W, bits, G, sym)
    Wp = W[:, perm].copy()
    codes_p = np.zeros((d_out, d_in), dtype=np.int64)
    Q_p = np.zeros((d_out, d_in))
    dE = np.zeros(d_out)
    for i in range(d_in):
        if dynamic and i % G == 0:
            scales[gpos[i]], zeros[gpos[i]] = quant_params(Wp[:, i:i + G], bits, sym)
        Finv = np.linalg.inv(Hp[i:, i:])
        w = Wp[:, i]
        q, what = quantize_values(w, scales[gpos[i]], zeros[gpos[i]], bits)
        codes_p[:, i] = q
        Q_p[:, i] = what
        e = w - what
        Wp[:, i:] += -(e / Finv[0, 0])[:, None] * Finv[:, 0][None, :]
        dE += e * e / Finv[0, 0]
    codes = np.empty_like(codes_p)
    Q = np.empty_like(Q_p)
    codes[:, perm] = codes_p
    Q[:, perm] = Q_p
    return SweepResult(codes=codes, Q=Q, scales=scales, zeros=zeros.astype(np.int64), g_idx=g_idx,
                       err=np.zeros((d_out, d_in)), row_loss=dE)


def rtn(W: np.ndarray, bits: int, group_size: int, sym: bool):
    """Round-to-nearest on the same group grid, every weight independently
    ([ch5] 5.1.1, 5.1.3): params from the original weights of each group, no
    compensation.  Returns (codes, Q)."""
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    scales, zeros = _static_params(W, bits, group_size, sym)
    g_idx = np.zeros(d_in, dtype=np.int64) if group_size == -1 else np.arange(d_in) // group_size
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    Q = np.zeros((d_out, d_in))
    for c in range(d_in):
        codes[:, c], Q[:, c] = quantize_values(W[:, c], scales[g_idx[c]], zeros[g_idx[c]], bits)
    return codes, Q


# ---------------------------------------------------------------------------
# errors ([ch5] 5.1.4: the objective is ||(W - W_q) X||^2)
# ---------------------------------------------------------------------------

def recon_error(W: np.ndarray, Q: np.ndarray, chunks: Iterable[np.ndarray]) -> float:
    """||(W - Q) X^T||_F^2 with X given as token-major chunks."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(Q, dtype=np.float64)
    tot = 0.0
    for xc in chunks:
        Y = np.asarray(xc, dtype=np.float64) @ D.T
        tot += float(np.sum(Y * Y))
    return tot


def recon_error_from_H(W: np.ndarray, Q: np.ndarray, H: np.ndarray, n_tokens: int) -> float:
    """Same quantity through H = 2 X^T X / N: (N / 2) * tr(D H D^T)."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(Q, dtype=np.float64)
    return 0.5 * n_tokens * float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))


# ---------------------------------------------------------------------------
# packing: 32/bits codes per int32 word along d_in, little-endian bit stream
# ([guide] QuantLinear qweight; [blog] 3.3: 128 INT4 codes occupy 64 bytes)
# ---------------------------------------------------------------------------

def packed_words(d_in: int, bits: int) -> int:
    return -(-d_in * bits // 32)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """qweight[w, n]: bits [32w, 32w+32) of output row n's code stream, where
    code (n, j) occupies stream bits [bits*j, bits*j + bits)."""
    codes = np.asarray(codes, dtype=np.int64)
    d_out, d_in = codes.shape
    nw = packed_words(d_in, bits)
    acc = np.zeros((nw + 1, d_out), dtype=np.uint64)
    for j in range(d_in):
        bit = bits * j
        w, off = divmod(bit, 32)
        v = codes[:, j].astype(np.uint64) << np.uint64(off)
        acc[w] |= v & np.uint64(0xFFFFFFFF)
        acc[w + 1] |= v >> np.uint64(32)
    return acc[:nw].astype(np.uint32).view(np.int32)


def unpack(qweight: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    q = np.asarray(qweight).view(np.uint32).astype(np.uint64)
    nw, d_out = q.shape
    q = np.concatenate([q, np.zeros((1, d_out), dtype=np.uint64)], axis=0)
    mask = np.uint64((1 << bits) - 1)
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    for j in range(d_in):
        w, off = divmod(bits * j, 32)
        v = (q[w] >> np.uint64(off)) | (q[w + 1] << np.uint64(32 - off) if off else np.uint64(0))
        codes[:, j] = (v & mask).astype(np.int64)
    return codes


def dequantize(qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g_idx: np.ndarray, bits: int,
               d_in: int) -> np.ndarray:
    """W_hat[n, k] = scale[g, n] (code(n, k) - zero[g, n]) with g = g_idx[k]
    (ch.5 section 5.1.10: one scale and zero point per group), from the packed
    codes and the per-group parameters, fp64."""
    codes = unpack(qweight, bits, d_in).astype(np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)[g, :].T
    z = np.asarray(zeros, dtype=np.float64)[g, :].T
    return s * (codes - z)


def dequant_matmul(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   g_idx: np.ndarray, bits: int) -> np.ndarray:
    """y = x W_hat^T in fp64 (the quantized layer applied to activations x [m, d_in])."""
    x = np.asarray(x, dtype=np.float64)
    return x @ dequantize(qweight, scales, zeros, g_idx, bits, x.shape[1]).T


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

@dataclass
class LayerResult:
    prep: Prepared
    sweep: SweepResult
    qweight: np.ndarray
    n_tokens: int


def solve_layer(W: np.ndarray, chunks: Iterable[np.ndarray], bits: int, group_size: int,
                sym: bool, desc_act: bool, static_groups: bool, damp_percent: float,
                blocksize: Optional[int] = 128) -> LayerResult:
    validate_config(bits, group_size, damp_percent)
    H, n = hessian(chunks)
    prep = prepare(H, damp_percent, desc_act)
    sw = quantize_layer(W, prep.U, prep.perm, bits, group_size, sym, static_groups, blocksize)
    return LayerResult(prep=prep, sweep=sw, qweight=pack(sw.codes, bits), n_tokens=n)
