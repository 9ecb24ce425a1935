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
