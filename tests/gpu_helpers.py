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
