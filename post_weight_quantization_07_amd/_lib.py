"""ctypes binding of libgptq.so (include/gptq.h).

Argument marshalling only: every step of the solve runs in the HIP library.
Tensors must live on the current HIP device; PyTorch supplies device memory
and the current stream.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq.so")

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_NOT_SPD, GPTQ_ERR_HIP, GPTQ_ERR_WORKSPACE, GPTQ_ERR_TOO_LARGE = range(6)
GPTQ_F32, GPTQ_BF16 = 0, 1

EXPORTS = ("gptq_config_validate", "gptq_status_string", "gptq_hessian_workspace_size",
           "gptq_hessian_accumulate", "gptq_prepare_workspace_size", "gptq_prepare_hinv",
           "gptq_workspace_size", "gptq_quantize_layer", "gptq_pack", "gptq_dequant_workspace_size",
           "gptq_dequant_matmul", "gptq_dequant_order", "gptq_dequant_ordered_workspace_size",
           "gptq_dequant_matmul_ordered", "gptq_dequant_scratch_bytes", "gptq_dequant_noalloc_need",
           "gptq_dequant_matmul_noalloc", "gptq_phase_timing", "gptq_phase_count", "gptq_phase_name",
           "gptq_phase_read")


class GptqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().gptq_status_string(status).decode()} (status {status})")


class NotPositiveDefinite(GptqError):
    """The damped Hessian failed a Cholesky pivot; retry with a larger damp_percent."""


class NonFiniteHessian(GptqError):
    """diag(H) holds a NaN or an infinity: the calibration inputs are not finite."""


class _CConfig(ctypes.Structure):
    _fields_ = [("bits", c_int32), ("group_size", c_int32), ("damp_percent", c_float),
                ("desc_act", c_int32), ("static_groups", c_int32), ("sym", c_int32),
                ("block_size", c_int32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python -m post_weight_quantization_07_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = c_void_p, c_int64, c_size_t
        cfgp = ctypes.POINTER(_CConfig)
        sig = {
            "gptq_config_validate": (c_int32, [cfgp]),
            "gptq_status_string": (ctypes.c_char_p, [c_int32]),
            "gptq_hessian_workspace_size": (sz, [i64, i64, c_int32]),
            "gptq_hessian_accumulate": (c_int32, [vp, i64, vp, c_int32, i64, i64, vp, sz, vp]),
            "gptq_prepare_workspace_size": (sz, [i64]),
            "gptq_prepare_hinv": (c_int32, [vp, i64, i64, cfgp, vp, vp, vp, vp, sz, vp]),
            "gptq_workspace_size": (sz, [i64, i64, cfgp]),
            "gptq_quantize_layer": (c_int32, [vp, c_int32, i64, i64, vp, vp, cfgp, vp, vp, vp, vp, vp, vp,
                                              vp, sz, vp]),
            "gptq_pack": (c_int32, [vp, i64, i64, c_int32, vp, vp]),
            "gptq_dequant_workspace_size": (sz, [i64, i64, i64]),
            "gptq_dequant_matmul": (c_int32, [vp, c_int32, i64, i64, vp, vp, vp, vp, c_int32, i64, c_int32, vp, vp,
                                              sz, vp]),
            "gptq_dequant_order": (c_int32, [vp, vp, c_int32, i64, i64, vp, vp, vp, vp]),
            "gptq_dequant_ordered_workspace_size": (sz, [i64, i64, i64]),
            "gptq_dequant_matmul_ordered": (c_int32, [vp, c_int32, i64, i64, vp, vp, vp, vp, vp, c_int32, i64,
                                                      c_int32, vp, vp, sz, vp]),
            "gptq_dequant_scratch_bytes": (sz, []),
            "gptq_dequant_noalloc_need": (sz, [i64, c_int32, i64, c_int32, i64]),
            "gptq_dequant_matmul_noalloc": (c_int32, [vp, c_int32, i64, i64, vp, vp, vp, vp, c_int32, i64, c_int32,
                                                      vp, vp]),
            "gptq_phase_timing": (c_int32, [c_int32]),
            "gptq_phase_count": (c_int32, []),
            "gptq_phase_name": (ctypes.c_char_p, [c_int32]),
            "gptq_phase_read": (c_int32, [vp, vp, c_int32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def phase_timing(enable: bool) -> None:
    """Switch the library's per-phase launch timing on (clearing the record) or off."""
    _check(_lib().gptq_phase_timing(1 if enable else 0), "gptq_phase_timing")


def phase_read() -> dict:
    """{phase name: (summed ms, launches)} of the launches recorded since timing was switched on."""
    lib = _lib()
    n = int(lib.gptq_phase_count())
    ms = (c_float * n)()
    cnt = (c_int32 * n)()
    _check(lib.gptq_phase_read(ctypes.cast(ms, c_void_p), ctypes.cast(cnt, c_void_p), n), "gptq_phase_read")
    return {lib.gptq_phase_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(n)}


def library_path() -> str:
    _lib()
    return LIB_PATH


# --------------------------------------------------------------------------
# configuration: the field names and defaults of BaseQuantizeConfig
# (AutoGPTQ examples walkthrough, section 1.4; OLMo quick-start, section 三)
# --------------------------------------------------------------------------

@dataclass
class QuantizeConfig:
    bits: int = 4
    group_size: int = -1
    damp_percent: float = 0.01
    desc_act: bool = True
    static_groups: bool = False
    sym: bool = True
    block_size: int = 128

    def __post_init__(self):
        if self.bits not in (2, 3, 4, 8):
            raise ValueError(f"bits must be one of [2, 3, 4, 8], got {self.bits}")
        if not (self.group_size == -1 or self.group_size > 0):
            raise ValueError(f"group_size must be -1 or > 0, got {self.group_size}")
        if not (0 < self.damp_percent < 1):
            raise ValueError(f"damp_percent must be in (0, 1), got {self.damp_percent}")
        st = _lib().gptq_config_validate(ctypes.byref(self._c()))
        if st != GPTQ_OK:
            raise ValueError(f"configuration rejected by the solver (block_size must be 128; a group "
                             f"must divide 128 or be a multiple of it): {self}")

    def _c(self) -> _CConfig:
        return _CConfig(int(self.bits), int(self.group_size), float(self.damp_percent), int(bool(self.desc_act)),
                        int(bool(self.static_groups)), int(bool(self.sym)), int(self.block_size))

    def n_groups(self, d_in: int) -> int:
        return 1 if self.group_size == -1 else -(-d_in // self.group_size)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(st: int, what: str):
    if st != GPTQ_OK:
        raise GptqError(st, what)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GPTQ_BF16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise ValueError(f"unsupported dtype {t.dtype}: expected bfloat16 or float32")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# the four calls of the C ABI
# --------------------------------------------------------------------------

def gptq_hessian_workspace_size(d_in: int, n_tokens: int, dtype: torch.dtype) -> int:
    code = GPTQ_BF16 if dtype == torch.bfloat16 else GPTQ_F32
    return int(_lib().gptq_hessian_workspace_size(d_in, n_tokens, code))


def gptq_hessian_accumulate(S: torch.Tensor, X: torch.Tensor, ws: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """S += X^T X for X [n_tokens, d_in] (rows may be strided)."""
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    _dev(S)
    if not X.is_cuda:
        raise ValueError("X must be on the GPU")
    n, d = X.shape
    if S.shape != (d, d) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [d_in, d_in]")
    code = _dtype_code(X)
    need = gptq_hessian_workspace_size(d, n, X.dtype)
    if ws is None:
        ws = _workspace(need, X.device)
    _check(_lib().gptq_hessian_accumulate(_ptr(S), d, _ptr(X), code, n, X.stride(0), _ptr(ws), ws.numel(),
                                          _stream(stream)), "gptq_hessian_accumulate")
    return S


def gptq_prepare_workspace_size(d_in: int) -> int:
    return int(_lib().gptq_prepare_workspace_size(d_in))


def gptq_prepare_hinv(S: torch.Tensor, n_total: int, cfg: QuantizeConfig, U: Optional[torch.Tensor] = None,
                      perm: Optional[torch.Tensor] = None, info: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None, check: bool = True):
    """S -> H in place; returns (U, perm, info).  With check=True the stream is
    synchronised and a failed pivot raises NotPositiveDefinite."""
    _dev(S)
    d = S.shape[0]
    dev = S.device
    U = torch.empty((d, d), dtype=torch.float32, device=dev) if U is None else U
    perm = torch.empty(d, dtype=torch.int32, device=dev) if perm is None else perm
    info = torch.empty(1, dtype=torch.int32, device=dev) if info is None else info
    if ws is None:
        ws = _workspace(gptq_prepare_workspace_size(d), dev)
    _check(_lib().gptq_prepare_hinv(_ptr(S), d, int(n_total), ctypes.byref(cfg._c()), _ptr(U), _ptr(perm),
                                    _ptr(info), _ptr(ws), ws.numel(), _stream(stream)), "gptq_prepare_hinv")
    if check:
        k = int(info.item())
        if k == -1:
            raise NonFiniteHessian(GPTQ_ERR_NOT_SPD, "gptq_prepare_hinv: diag(H) is not finite (NaN or infinity "
                                   "in the calibration inputs)")
        if k != 0:
            raise NotPositiveDefinite(GPTQ_ERR_NOT_SPD, "gptq_prepare_hinv: the damped Hessian's trailing block is "
                                      f"not positive definite from sweep position {k - 1}")
    return U, perm, info


def gptq_workspace_size(d_out: int, d_in: int, cfg: QuantizeConfig) -> int:
    return int(_lib().gptq_workspace_size(d_out, d_in, ctypes.byref(cfg._c())))


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: Optional[torch.Tensor], cfg: QuantizeConfig,
                        want_q: bool = True, want_loss: bool = True, out: Optional[dict] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Column sweep; returns codes (uint8, original order), scales, zeros, g_idx
    and optionally Q (dequantized) and row_loss."""
    _dev(W, U, perm)
    d_out, d_in = W.shape
    dev = W.device
    ng = cfg.n_groups(d_in)
    o = dict(out) if out else {}
    o.setdefault("codes", torch.empty((d_out, d_in), dtype=torch.uint8, device=dev))
    o.setdefault("scales", torch.empty((ng, d_out), dtype=torch.float32, device=dev))
    o.setdefault("zeros", torch.empty((ng, d_out), dtype=torch.int32, device=dev))
    o.setdefault("g_idx", torch.empty(d_in, dtype=torch.int32, device=dev))
    if want_q:
        o.setdefault("Q", torch.empty((d_out, d_in), dtype=torch.float32, device=dev))
    if want_loss:
        o.setdefault("row_loss", torch.empty(d_out, dtype=torch.float32, device=dev))
    if ws is None:
        ws = _workspace(gptq_workspace_size(d_out, d_in, cfg), dev)
    _check(_lib().gptq_quantize_layer(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(U), _ptr(perm),
                                      ctypes.byref(cfg._c()), _ptr(o["codes"]), _ptr(o["scales"]),
                                      _ptr(o["zeros"]), _ptr(o["g_idx"]), _ptr(o.get("Q")),
                                      _ptr(o.get("row_loss")), _ptr(ws), ws.numel(), _stream(stream)),
           "gptq_quantize_layer")
    return o


def gptq_pack(codes: torch.Tensor, bits: int, qweight: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(codes)
    d_out, d_in = codes.shape
    if qweight is None:
        qweight = torch.empty((d_in * bits // 32, d_out), dtype=torch.int32, device=codes.device)
    _check(_lib().gptq_pack(_ptr(codes), d_out, d_in, int(bits), _ptr(qweight), _stream(stream)), "gptq_pack")
    return qweight


def gptq_dequant_workspace_size(m: int, d_in: int, d_out: int) -> int:
    return int(_lib().gptq_dequant_workspace_size(m, d_in, d_out))


def gptq_dequant_matmul(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                        g_idx: torch.Tensor, bits: int, y: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y [m, d_out] fp32 = x [m, d_in] (bf16 or fp32) times the transpose of the
    weights dequantized from qweight / scales / zeros / g_idx."""
    _dev(x, qweight, scales, zeros, g_idx)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("gptq_dequant_matmul: x must be a contiguous [m, d_in] matrix")
    m, d_in = x.shape
    d_out = qweight.shape[1]
    n_groups = scales.shape[0]
    if (qweight.shape[0] * 32 != d_in * bits or scales.shape != (n_groups, d_out) or zeros.shape != (n_groups, d_out)
            or g_idx.shape != (d_in,) or qweight.dtype != torch.int32 or scales.dtype != torch.float32
            or zeros.dtype != torch.int32 or g_idx.dtype != torch.int32):
        raise ValueError("gptq_dequant_matmul: qweight / scales / zeros / g_idx do not match x and bits")
    if y is None:
        y = torch.empty((m, d_out), dtype=torch.float32, device=x.device)
    if ws is None:
        need = gptq_dequant_workspace_size(m, d_in, d_out)
        ws = _workspace(need, x.device) if need > 0 else None
    _check(_lib().gptq_dequant_matmul(_ptr(x), _dtype_code(x), m, d_in, _ptr(qweight.contiguous()),
                                      _ptr(scales.contiguous()), _ptr(zeros.contiguous()), _ptr(g_idx.contiguous()),
                                      int(bits), d_out, n_groups, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream(stream)),
           "gptq_dequant_matmul")
    return y


def gptq_dequant_scratch_bytes() -> int:
    return int(_lib().gptq_dequant_scratch_bytes())


def gptq_dequant_noalloc_need(m: int, dtype: torch.dtype, d_in: int, bits: int, d_out: int) -> int:
    code = GPTQ_BF16 if dtype == torch.bfloat16 else GPTQ_F32
    return int(_lib().gptq_dequant_noalloc_need(m, code, d_in, bits, d_out))


def gptq_dequant_matmul_noalloc(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                                g_idx: torch.Tensor, bits: int, y: torch.Tensor, stream=None) -> torch.Tensor:
    """gptq_dequant_matmul with the library's fixed scratch buffer instead of a
    workspace: the call itself allocates nothing (y is the caller's)."""
    _dev(x, qweight, scales, zeros, g_idx, y)
    if x.dim() != 2:
        raise ValueError("gptq_dequant_matmul_noalloc: x must be a contiguous [m, d_in] matrix")
    m, d_in = x.shape
    d_out = qweight.shape[1]
    n_groups = scales.shape[0]
    if (qweight.shape[0] * 32 != d_in * bits or scales.shape != (n_groups, d_out) or zeros.shape != (n_groups, d_out)
            or g_idx.shape != (d_in,) or y.shape != (m, d_out) or qweight.dtype != torch.int32
            or scales.dtype != torch.float32 or zeros.dtype != torch.int32 or g_idx.dtype != torch.int32
            or y.dtype != torch.float32):
        raise ValueError("gptq_dequant_matmul_noalloc: tensors do not match x and bits")
    _check(_lib().gptq_dequant_matmul_noalloc(_ptr(x), _dtype_code(x), m, d_in, _ptr(qweight), _ptr(scales),
                                              _ptr(zeros), _ptr(g_idx), int(bits), d_out, n_groups, _ptr(y),
                                              _stream(stream)),
           "gptq_dequant_matmul_noalloc")
    return y


def gptq_dequant_order(qweight: torch.Tensor, g_idx: torch.Tensor, bits: int, stream=None):
    """An act-order layer put in group order for the dequantizing product:
    returns (qweight_sorted, g_idx_sorted, order), order[j] = the original
    input channel at sorted position j (a stable sort of the channels by
    group), the codes repacked in that order."""
    _dev(qweight, g_idx)
    d_in = g_idx.shape[0]
    d_out = qweight.shape[1]
    if (g_idx.dim() != 1 or qweight.dim() != 2 or qweight.shape[0] * 32 != d_in * bits
            or qweight.dtype != torch.int32 or g_idx.dtype != torch.int32):
        raise ValueError("gptq_dequant_order: qweight / g_idx do not match bits")
    q_out = torch.empty_like(qweight)
    g_out = torch.empty_like(g_idx)
    order = torch.empty_like(g_idx)
    _check(_lib().gptq_dequant_order(_ptr(qweight.contiguous()), _ptr(g_idx.contiguous()), int(bits), d_in, d_out,
                                     _ptr(q_out), _ptr(g_out), _ptr(order), _stream(stream)),
           "gptq_dequant_order")
    return q_out, g_out, order


def gptq_dequant_ordered_workspace_size(m: int, d_in: int, d_out: int) -> int:
    return int(_lib().gptq_dequant_ordered_workspace_size(m, d_in, d_out))


def gptq_dequant_matmul_ordered(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                                g_idx: torch.Tensor, order: torch.Tensor, bits: int, y: Optional[torch.Tensor] = None,
                                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """gptq_dequant_matmul on a layer reordered by gptq_dequant_order; x is
    given in the original channel order."""
    _dev(x, qweight, scales, zeros, g_idx, order)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("gptq_dequant_matmul_ordered: x must be a contiguous [m, d_in] matrix")
    m, d_in = x.shape
    d_out = qweight.shape[1]
    n_groups = scales.shape[0]
    if (qweight.shape[0] * 32 != d_in * bits or scales.shape != (n_groups, d_out) or zeros.shape != (n_groups, d_out)
            or g_idx.shape != (d_in,) or order.shape != (d_in,) or qweight.dtype != torch.int32
            or scales.dtype != torch.float32 or zeros.dtype != torch.int32 or g_idx.dtype != torch.int32
            or order.dtype != torch.int32):
        raise ValueError("gptq_dequant_matmul_ordered: tensors do not match x and bits")
    if y is None:
        y = torch.empty((m, d_out), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _workspace(gptq_dequant_ordered_workspace_size(m, d_in, d_out), x.device)
    _check(_lib().gptq_dequant_matmul_ordered(_ptr(x), _dtype_code(x), m, d_in, _ptr(qweight.contiguous()),
                                              _ptr(scales.contiguous()), _ptr(zeros.contiguous()),
                                              _ptr(g_idx.contiguous()), _ptr(order.contiguous()), int(bits), d_out,
                                              n_groups, _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "gptq_dequant_matmul_ordered")
    return y
