"""Shared helpers of the GPU tests (device transfers, tolerances)."""
import numpy as np
import torch

import synth


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """Host fp32 array -> device tensor of the given storage dtype (bf16 by RNE)."""
    if dtype == "bf16":
        bits = synth.bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def banner(msg: str):
    print(f"[gpu-case] {msg}", flush=True)


# A code decision whose pre-rounding value w/s + z lies within TIE_TOL steps of
# a rounding boundary is a float tie: the GPU's running weights carry the fp32
# rounding of up to d_in compensation updates, about sqrt(d_in) * eps32 * (|v| +
# a few) steps (under 1e-4 for d_in <= 28672, |v| <= 255), and the decision may
# go either way.  Measured first-divergence distances are about 1e-6 steps.
TIE_TOL = 2.0 ** -12


def sweep_parity(W_rows, U_g, perm_g, layer_or_kw, gpu_codes):
    """Oracle sweep on the given rows with the GPU's factor and order, following
    the GPU's decisions at float ties; returns (oracle result, fraction of codes
    still differing, fraction of decisions taken at ties)."""
    import oracle as O
    kw = layer_or_kw if isinstance(layer_or_kw, dict) else dict(
        bits=layer_or_kw.bits, group_size=layer_or_kw.group_size, sym=layer_or_kw.sym,
        static_groups=layer_or_kw.static_groups)
    ref = O.quantize_layer(np.asarray(W_rows, dtype=np.float64), np.asarray(U_g, dtype=np.float64), perm_g,
                           kw["bits"], kw["group_size"], kw["sym"], kw["static_groups"],
                           follow=gpu_codes, tie_tol=TIE_TOL)
    mism = float(np.mean(gpu_codes != ref.codes))
    return ref, mism, ref.ties / gpu_codes.size


def independent_parity(W_rows, U_g, perm_g, layer_or_kw, gpu_codes, gpu_zeros=None, rows=None):
    """Oracle sweep on the given rows with the GPU's factor and order and NO
    following: every decision is the oracle's own.  Rows are independent given
    U, so a row either matches the GPU's codes exactly or has a first
    differing decision (in sweep order); that first decision must be a float
    tie -- the oracle's pre-rounding value w/s + z within TIE_TOL steps of the
    rounding boundary between the two codes, or, for a dynamic asymmetric
    group starting there, the zero point's pre-rounding value -lo/s within
    TIE_TOL of a half-integer.  Everything after it in that row follows from a
    different, equally correct decision.  Returns (oracle result, raw fraction
    of codes differing, rows differing, largest first-divergence distance);
    raises AssertionError on a first divergence that is not a tie."""
    import oracle as O
    kw = layer_or_kw if isinstance(layer_or_kw, dict) else dict(
        bits=layer_or_kw.bits, group_size=layer_or_kw.group_size, sym=layer_or_kw.sym,
        static_groups=layer_or_kw.static_groups)
    ref = O.quantize_layer(np.asarray(W_rows, dtype=np.float64), np.asarray(U_g, dtype=np.float64), perm_g,
                           kw["bits"], kw["group_size"], kw["sym"], kw["static_groups"], record_v=True)
    perm_g = np.asarray(perm_g, dtype=np.int64)
    gp = np.asarray(gpu_codes, dtype=np.int64)[:, perm_g]
    rp = ref.codes[:, perm_g]
    diff = gp != rp
    bad_rows = np.nonzero(diff.any(axis=1))[0]
    worst = 0.0
    G = kw["group_size"]
    for r in bad_rows:
        i = int(np.argmax(diff[r]))
        q, f, v = int(rp[r, i]), int(gp[r, i]), float(ref.vals[r, i])
        dist = abs(v - (min(q, f) + 0.5)) if abs(q - f) == 1 else np.inf
        if dist > TIE_TOL and gpu_zeros is not None and G > 0 and not kw["sym"] and not kw["static_groups"]:
            # a dynamic asymmetric group: its zero point may have been the tie
            g = i // G
            col = r if rows is None else rows[r]
            zr = float(ref.zvals[g, r])
            if int(np.asarray(gpu_zeros)[g, col]) != int(ref.zeros[g, r]) and np.isfinite(zr):
                dist = abs(zr - (np.floor(zr) + 0.5))
        assert dist <= TIE_TOL, (f"row {r}: first differing decision at sweep position {i} is not a float tie "
                                 f"(oracle code {q}, GPU code {f}, w/s + z = {v!r}, distance {dist:.3e})")
        worst = max(worst, dist)
    return ref, float(np.mean(diff)), int(len(bad_rows)), worst
