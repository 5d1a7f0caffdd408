"""Python binding of libpwq (ctypes): argument marshalling only.

Each function takes torch tensors that live on the GPU, checks shapes and dtypes,
allocates outputs and the workspace with torch (device memory and streams are all torch
is used for), and calls the C entry point of the same name on the current stream.  Every
step of the computation runs in the HIP kernels of libpwq.so; if the library is missing
the import fails loudly instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpwq.so")

PWQ_OK, PWQ_EINVAL, PWQ_EDTYPE, PWQ_EWORKSPACE, PWQ_EHIP = 0, 1, 2, 3, 4
PWQ_F32, PWQ_F16, PWQ_BF16 = 0, 1, 2

_c_void_p, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float


class PwqParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("act_order", ctypes.c_int32)]


_SIGS = {
    "pwq_version": (ctypes.c_int, []),
    "pwq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pwq_last_hip_error": (ctypes.c_int, []),
    "pwq_hessian_workspace_size": (_sz, [_i64, _i64, ctypes.c_int]),
    "pwq_hessian_accumulate": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_hessian_damp": (ctypes.c_int, [_c_void_p, _i64, _f32, _c_void_p, _c_void_p]),
    "pwq_act_order_perm": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _c_void_p]),
    "pwq_chol_workspace_size": (_sz, [_i64]),
    "pwq_chol_inverse_upper": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_gptq_workspace_size": (_sz, [_i64, _i64, ctypes.POINTER(PwqParams)]),
    "pwq_gptq_quantize_layer": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                               ctypes.POINTER(PwqParams), _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                               _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_rtn_quantize": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p]),
    "pwq_dequant": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i32, _i32, _c_void_p,
                                   ctypes.c_int, _c_void_p]),
    "pwq_gptq_quantize_layer_zp": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                                  ctypes.POINTER(PwqParams), _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                  _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz,
                                                  _c_void_p]),
    "pwq_rtn_quantize_zp": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p,
                                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pwq_dequant_zp": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i32, _i32,
                                      _c_void_p, ctypes.c_int, _c_void_p]),
    "pwq_recon_mse_zp": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, ctypes.c_int, _i64,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                                        _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_channel_abs_mean_workspace_size": (_sz, [_i64, _i64]),
    "pwq_channel_abs_mean": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p, _sz,
                                            _c_void_p]),
    "pwq_awq_search_workspace_size": (_sz, [_i64, _i64]),
    "pwq_awq_search": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _i32, _i32,
                                      _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_tensor_scales_workspace_size": (_sz, []),
    "pwq_tensor_scales": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _i32, _c_void_p, _c_void_p,
                                         _c_void_p, _sz, _c_void_p]),
    "pwq_quantized_matmul_workspace_size": (_sz, [_i64, _i64, _i64]),
    "pwq_quantized_matmul": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                            _i64, _i32, _c_void_p, ctypes.c_int, _i64, _c_void_p, _sz, _c_void_p]),
    "pwq_recon_mse_hessian_workspace_size": (_sz, [_i64, _i64]),
    "pwq_recon_mse_hessian": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, ctypes.c_int, _i64,
                                             _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                                             _c_void_p, _c_void_p, _sz, _c_void_p]),
    "pwq_quantized_matmul_noalloc": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                                    _c_void_p, _i64, _i32, _c_void_p, ctypes.c_int, _i64, _c_void_p]),
    "pwq_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "pwq_profile_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int]),
    "pwq_recon_mse_workspace_size": (_sz, [_i64, _i64, _i64]),
    "pwq_recon_mse": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p, ctypes.c_int, _i64,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p,
                                     _c_void_p, _sz, _c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpwq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (post_weight_quantization_27_amd.build_lib.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class PwqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().pwq_status_string(status).decode()
        if status == PWQ_EHIP:
            msg += f" (hipError {lib().pwq_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(fn: str, status: int):
    if status != PWQ_OK:
        raise PwqError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: PWQ_F32, torch.float16: PWQ_F16, torch.bfloat16: PWQ_BF16}[t.dtype]


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a row-major 2-D device tensor (unit column stride)."""
    if t.dim() != 2 or not t.is_cuda:
        raise ValueError(f"{name}: expected a 2-D GPU tensor")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name}: columns must be contiguous")
    return max(t.stride(0), t.shape[1])


def _ws(nbytes: int, dev) -> Optional[torch.Tensor]:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev) if nbytes else None


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous GPU {dtype} of shape {tuple(shape)}")


# ------------------------------------------------------------------ Hessian
def hessian_accumulate(X: torch.Tensor, H: torch.Tensor) -> torch.Tensor:
    """H += 2 X^T X (X: tokens x d_in, float32 or bfloat16; H float32 d_in x d_in)."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    _need(H, torch.float32, (d_in, d_in), "H")
    code = _dtype_code(X)
    nb = lib().pwq_hessian_workspace_size(n_tok, d_in, code)
    ws = _ws(nb, X.device)
    _check("pwq_hessian_accumulate", lib().pwq_hessian_accumulate(_p(X), code, n_tok, d_in, ldx, _p(H), _p(ws), nb, _stream(X)))
    return H


def hessian_damp(H: torch.Tensor, damp: float, lambda_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(H, torch.float32, (H.shape[0], H.shape[0]), "H")
    _check("pwq_hessian_damp", lib().pwq_hessian_damp(_p(H), H.shape[0], float(damp), _p(lambda_out), _stream(H)))
    return H


def act_order_perm(H: torch.Tensor) -> torch.Tensor:
    n = H.shape[0]
    _need(H, torch.float32, (n, n), "H")
    perm = torch.empty(n, dtype=torch.int32, device=H.device)
    _check("pwq_act_order_perm", lib().pwq_act_order_perm(_p(H), n, _p(perm), _stream(H)))
    return perm


# ------------------------------------------------------------------ factor
def chol_inverse_upper(H: torch.Tensor, perm: Optional[torch.Tensor] = None, U: Optional[torch.Tensor] = None,
                       info: Optional[torch.Tensor] = None):
    """(U, info): U upper with H^-1 = U^T U (of H[perm][:, perm] if perm); info int32 on device."""
    n = H.shape[0]
    _need(H, torch.float32, (n, n), "H")
    if U is None:
        U = torch.empty((n, n), dtype=torch.float32, device=H.device)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=H.device)
    nb = lib().pwq_chol_workspace_size(n)
    ws = _ws(nb, H.device)
    _check("pwq_chol_inverse_upper", lib().pwq_chol_inverse_upper(_p(H), n, _p(perm), _p(U), _p(info), _p(ws), nb, _stream(H)))
    return U, info


# ------------------------------------------------------------------ GPTQ / RTN
def _n_groups(d_in: int, group_size: int) -> int:
    return 1 if group_size == 0 else -(-d_in // group_size)


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, info: torch.Tensor, bits: int = 4, group_size: int = 128,
                        block_size: int = 128, perm: Optional[torch.Tensor] = None,
                        scales_in: Optional[torch.Tensor] = None, want_codes: bool = True, want_packed: bool = True,
                        out: Optional[dict] = None) -> dict:
    """GPTQ column loop.  Returns {codes (int8, original order), packed (uint8), scales (float16,
    groups in processing order), g_idx (int32, act-order only)}."""
    return _gptq(W, U, info, bits, group_size, block_size, perm, scales_in, None, want_codes, want_packed, out, False)


def gptq_quantize_layer_zp(W: torch.Tensor, U: torch.Tensor, info: torch.Tensor, bits: int = 4, group_size: int = 128,
                           block_size: int = 128, perm: Optional[torch.Tensor] = None,
                           scales_in: Optional[torch.Tensor] = None, zeros_in: Optional[torch.Tensor] = None,
                           want_codes: bool = True, want_packed: bool = True, out: Optional[dict] = None) -> dict:
    """GPTQ with zero-points.  As gptq_quantize_layer, with codes uint8 and zeros (uint16 as
    int16 storage, like the scales) in the result."""
    return _gptq(W, U, info, bits, group_size, block_size, perm, scales_in, zeros_in, want_codes, want_packed, out, True)


def _gptq(W, U, info, bits, group_size, block_size, perm, scales_in, zeros_in, want_codes, want_packed, out, zp):
    ldw = _rows(W, "W")
    d_out, d_in = W.shape
    act = perm is not None
    prm = PwqParams(bits, group_size, block_size, 1 if act else 0)
    dev = W.device
    ng = _n_groups(d_in, group_size)
    o = out if out is not None else {}
    if want_codes and o.get("codes") is None:
        o["codes"] = torch.empty((d_out, d_in), dtype=torch.uint8 if zp else torch.int8, device=dev)
    if want_packed and o.get("packed") is None:
        o["packed"] = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    if o.get("scales") is None:
        o["scales"] = torch.empty((d_out, ng), dtype=torch.float16, device=dev)
    if zp and o.get("zeros") is None:
        o["zeros"] = torch.empty((d_out, ng), dtype=torch.int16, device=dev)
    if act and o.get("g_idx") is None:
        o["g_idx"] = torch.empty(d_in, dtype=torch.int32, device=dev)
    nb = lib().pwq_gptq_workspace_size(d_out, d_in, ctypes.byref(prm))
    ws = o.get("_ws")
    if ws is None or ws.numel() < nb:
        ws = _ws(nb, dev)
        o["_ws"] = ws
    codes = _p(o.get("codes") if want_codes else None)
    packed = _p(o.get("packed") if want_packed else None)
    g_idx = _p(o.get("g_idx") if act else None)
    if zp:
        _check("pwq_gptq_quantize_layer_zp", lib().pwq_gptq_quantize_layer_zp(
            _p(W), _dtype_code(W), d_out, d_in, ldw, _p(U), _p(info), ctypes.byref(prm), _p(perm), _p(scales_in),
            _p(zeros_in), codes, packed, _p(o["scales"]), _p(o["zeros"]), g_idx, _p(ws), nb, _stream(W)))
    else:
        _check("pwq_gptq_quantize_layer", lib().pwq_gptq_quantize_layer(
            _p(W), _dtype_code(W), d_out, d_in, ldw, _p(U), _p(info), ctypes.byref(prm), _p(perm), _p(scales_in),
            codes, packed, _p(o["scales"]), g_idx, _p(ws), nb, _stream(W)))
    return o


def rtn_quantize(W: torch.Tensor, bits: int = 4, group_size: int = 128, scales_in: Optional[torch.Tensor] = None,
                 want_codes: bool = True, want_packed: bool = True, out: Optional[dict] = None) -> dict:
    return _rtn(W, bits, group_size, scales_in, None, want_codes, want_packed, out, False)


def rtn_quantize_zp(W: torch.Tensor, bits: int = 4, group_size: int = 128, scales_in: Optional[torch.Tensor] = None,
                    zeros_in: Optional[torch.Tensor] = None, want_codes: bool = True, want_packed: bool = True,
                    out: Optional[dict] = None) -> dict:
    """RTN with zero-points: codes uint8, zeros (uint16 bits in int16 storage) per row and group."""
    return _rtn(W, bits, group_size, scales_in, zeros_in, want_codes, want_packed, out, True)


def _rtn(W, bits, group_size, scales_in, zeros_in, want_codes, want_packed, out, zp):
    ldw = _rows(W, "W")
    d_out, d_in = W.shape
    dev = W.device
    ng = _n_groups(d_in, group_size)
    o = out if out is not None else {}
    if want_codes and o.get("codes") is None:
        o["codes"] = torch.empty((d_out, d_in), dtype=torch.uint8 if zp else torch.int8, device=dev)
    if want_packed and o.get("packed") is None:
        o["packed"] = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    if o.get("scales") is None:
        o["scales"] = torch.empty((d_out, ng), dtype=torch.float16, device=dev)
    if zp and o.get("zeros") is None:
        o["zeros"] = torch.empty((d_out, ng), dtype=torch.int16, device=dev)
    codes = _p(o.get("codes") if want_codes else None)
    packed = _p(o.get("packed") if want_packed else None)
    if zp:
        _check("pwq_rtn_quantize_zp", lib().pwq_rtn_quantize_zp(
            _p(W), _dtype_code(W), d_out, d_in, ldw, bits, group_size, _p(scales_in), _p(zeros_in), codes, packed,
            _p(o["scales"]), _p(o["zeros"]), _stream(W)))
    else:
        _check("pwq_rtn_quantize", lib().pwq_rtn_quantize(
            _p(W), _dtype_code(W), d_out, d_in, ldw, bits, group_size, _p(scales_in), codes, packed, _p(o["scales"]),
            _stream(W)))
    return o


def dequant(scales: torch.Tensor, d_in: int, bits: int = 4, group_size: int = 128, packed: Optional[torch.Tensor] = None,
            codes: Optional[torch.Tensor] = None, g_idx: Optional[torch.Tensor] = None, out_dtype=torch.float16,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    d_out = scales.shape[0]
    src = packed if packed is not None else codes
    if out is None:
        out = torch.empty((d_out, d_in), dtype=out_dtype, device=src.device)
    _check("pwq_dequant", lib().pwq_dequant(_p(packed), _p(codes), _p(scales), _p(g_idx), d_out, d_in, bits, group_size,
                                            _p(out), _dtype_code(out), _stream(src)))
    return out


def dequant_zp(scales: torch.Tensor, zeros: torch.Tensor, d_in: int, bits: int = 4, group_size: int = 128,
               packed: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
               g_idx: Optional[torch.Tensor] = None, out_dtype=torch.float16,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """What = S (code - Z) from unsigned codes or nibbles, scales and zeros."""
    d_out = scales.shape[0]
    src = packed if packed is not None else codes
    if out is None:
        out = torch.empty((d_out, d_in), dtype=out_dtype, device=src.device)
    _check("pwq_dequant_zp", lib().pwq_dequant_zp(_p(packed), _p(codes), _p(scales), _p(zeros), _p(g_idx), d_out, d_in,
                                                  bits, group_size, _p(out), _dtype_code(out), _stream(src)))
    return out


def recon_mse(X: torch.Tensor, W: torch.Tensor, scales: torch.Tensor, bits: int = 4, group_size: int = 128,
              packed: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
              g_idx: Optional[torch.Tensor] = None, mse: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None, zeros: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device float64 scalar: mean over tokens x outputs of (X (W - What)^T)^2.  With
    ``zeros``, the codes are those of the zero-point form (pwq_recon_mse_zp)."""
    ldx, ldw = _rows(X, "X"), _rows(W, "W")
    n_tok, d_in = X.shape
    d_out = W.shape[0]
    if mse is None:
        mse = torch.empty(1, dtype=torch.float64, device=X.device)
    nb = lib().pwq_recon_mse_workspace_size(n_tok, d_in, d_out)
    if ws is None or ws.numel() < nb:
        ws = _ws(nb, X.device)
    if zeros is not None:
        _check("pwq_recon_mse_zp", lib().pwq_recon_mse_zp(
            _p(X), _dtype_code(X), n_tok, d_in, ldx, _p(W), _dtype_code(W), ldw, _p(packed), _p(codes), _p(scales),
            _p(zeros), _p(g_idx), d_out, bits, group_size, _p(mse), _p(ws), nb, _stream(X)))
    else:
        _check("pwq_recon_mse", lib().pwq_recon_mse(
            _p(X), _dtype_code(X), n_tok, d_in, ldx, _p(W), _dtype_code(W), ldw, _p(packed), _p(codes), _p(scales),
            _p(g_idx), d_out, bits, group_size, _p(mse), _p(ws), nb, _stream(X)))
    return mse


def recon_mse_hessian(H: torch.Tensor, n_tok: int, W: torch.Tensor, scales: torch.Tensor, bits: int = 4,
                      group_size: int = 128, packed: Optional[torch.Tensor] = None,
                      codes: Optional[torch.Tensor] = None, g_idx: Optional[torch.Tensor] = None,
                      zeros: Optional[torch.Tensor] = None, shift: Optional[torch.Tensor] = None,
                      mse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device float64 scalar: the same mean square as recon_mse, through H = 2 X^T X formed over
    n_tok tokens (pwq_recon_mse_hessian); ``shift`` (device float32, e.g. hessian_damp's
    lambda_out) is what damping added to H's diagonal."""
    ldh, ldw = _rows(H, "H"), _rows(W, "W")
    d_in = H.shape[0]
    d_out = W.shape[0]
    if H.dtype != torch.float32 or H.shape != (d_in, d_in) or W.shape[1] != d_in:
        raise ValueError("H: float32 d_in x d_in matching W's columns")
    if mse is None:
        mse = torch.empty(1, dtype=torch.float64, device=W.device)
    nb = lib().pwq_recon_mse_hessian_workspace_size(d_in, d_out)
    if ws is None or ws.numel() < nb:
        ws = _ws(nb, W.device)
    _check("pwq_recon_mse_hessian", lib().pwq_recon_mse_hessian(
        _p(H), ldh, d_in, int(n_tok), _p(shift), _p(W), _dtype_code(W), ldw, _p(packed), _p(codes), _p(scales),
        _p(zeros), _p(g_idx), d_out, bits, group_size, _p(mse), _p(ws), nb, _stream(W)))
    return mse


# ------------------------------------------------------------------ activation-aware scaling
def channel_abs_mean(X: torch.Tensor) -> torch.Tensor:
    """float32 d_in: mean over tokens of |X| per input channel."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    a = torch.empty(d_in, dtype=torch.float32, device=X.device)
    nb = lib().pwq_channel_abs_mean_workspace_size(n_tok, d_in)
    ws = _ws(nb, X.device)
    _check("pwq_channel_abs_mean", lib().pwq_channel_abs_mean(_p(X), _dtype_code(X), n_tok, d_in, ldx, _p(a), _p(ws), nb,
                                                              _stream(X)))
    return a


def awq_search(W: torch.Tensor, H: torch.Tensor, n_tok: int, abs_mean: torch.Tensor, bits: int = 4,
               group_size: int = 128, n_alpha: int = 21, zero_point: bool = False, want_codes: bool = True,
               want_packed: bool = True) -> dict:
    """Grid search of s = abs_mean^alpha (H undamped).  Returns {mse (float64 n_alpha), best (int32),
    s (float32 d_in), codes, packed, scales, zeros} with the RTN result of W diag(s)."""
    ldw = _rows(W, "W")
    d_out, d_in = W.shape
    # the library reads H as a dense d_in x d_in float32 matrix (row pitch d_in) and abs_mean
    # as d_in float32 values
    _need(H, torch.float32, (d_in, d_in), "H")
    _need(abs_mean, torch.float32, (d_in,), "abs_mean")
    dev = W.device
    ng = _n_groups(d_in, group_size)
    o = {"mse": torch.empty(n_alpha, dtype=torch.float64, device=dev),
         "best": torch.empty(1, dtype=torch.int32, device=dev),
         "s": torch.empty(d_in, dtype=torch.float32, device=dev),
         "scales": torch.empty((d_out, ng), dtype=torch.float16, device=dev)}
    if want_codes:
        o["codes"] = torch.empty((d_out, d_in), dtype=torch.uint8 if zero_point else torch.int8, device=dev)
    if want_packed:
        o["packed"] = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    if zero_point:
        o["zeros"] = torch.empty((d_out, ng), dtype=torch.int16, device=dev)
    nb = lib().pwq_awq_search_workspace_size(d_out, d_in)
    ws = _ws(nb, dev)
    _check("pwq_awq_search", lib().pwq_awq_search(
        _p(W), _dtype_code(W), d_out, d_in, ldw, _p(H), n_tok, _p(abs_mean), bits, group_size, n_alpha,
        1 if zero_point else 0, _p(o["mse"]), _p(o["best"]), _p(o["s"]), _p(o.get("codes")), _p(o.get("packed")),
        _p(o["scales"]), _p(o.get("zeros")), _p(ws), nb, _stream(W)))
    return o


# ------------------------------------------------------------------ per-tensor quantizer
def tensor_scales(W: torch.Tensor, bits: int = 4, zero_point: bool = False):
    """(scales d_out x 1 float16, zeros d_out x 1 int16 or None): one quantizer for the whole
    matrix, replicated per row; pass them as fixed scales (and zeros) with group_size 0."""
    ldw = _rows(W, "W")
    d_out, d_in = W.shape
    scales = torch.empty((d_out, 1), dtype=torch.float16, device=W.device)
    zeros = torch.empty((d_out, 1), dtype=torch.int16, device=W.device) if zero_point else None
    nb = lib().pwq_tensor_scales_workspace_size()
    ws = _ws(nb, W.device)
    _check("pwq_tensor_scales", lib().pwq_tensor_scales(_p(W), _dtype_code(W), d_out, d_in, ldw, bits, _p(scales),
                                                        _p(zeros), _p(ws), nb, _stream(W)))
    return scales, zeros


# ------------------------------------------------------------------ product with What
def quantized_matmul(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, group_size: int = 128,
                     zeros: Optional[torch.Tensor] = None, out_dtype=torch.float16, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X What^T (X float16 tokens x d_in; What from packed nibbles, scales and optional zeros)."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    d_out = packed.shape[0]
    if out is None:
        out = torch.empty((n_tok, d_out), dtype=out_dtype, device=X.device)
    ldy = _rows(out, "Y") if n_tok > 0 else d_out
    nb = lib().pwq_quantized_matmul_workspace_size(n_tok, d_in, d_out)
    if nb and (ws is None or ws.numel() < nb):
        ws = _ws(nb, X.device)
    _check("pwq_quantized_matmul", lib().pwq_quantized_matmul(
        _p(X), _dtype_code(X), n_tok, d_in, ldx, _p(packed), _p(scales), _p(zeros), d_out, group_size, _p(out),
        _dtype_code(out), ldy, _p(ws) if nb else None, nb, _stream(X)))
    return out


def quantized_matmul_noalloc(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, out: torch.Tensor,
                             group_size: int = 128, zeros: Optional[torch.Tensor] = None) -> torch.Tensor:
    """quantized_matmul into a caller-given ``out`` through the allocation-free entry point
    (the library's static scratch array holds the partial sums; nothing is allocated)."""
    ldx = _rows(X, "X")
    n_tok, d_in = X.shape
    d_out = packed.shape[0]
    ldy = _rows(out, "Y") if n_tok > 0 else d_out
    _check("pwq_quantized_matmul_noalloc", lib().pwq_quantized_matmul_noalloc(
        _p(X), _dtype_code(X), n_tok, d_in, ldx, _p(packed), _p(scales), _p(zeros), d_out, group_size, _p(out),
        _dtype_code(out), ldy, _stream(X)))
    return out


# ------------------------------------------------------------------ one layer, end to end
def gptq_layer(W: torch.Tensor, X: torch.Tensor, bits: int = 4, group_size: int = 128, block_size: int = 128,
               damp: float = 0.01, act_order: bool = False, want_codes: bool = True, want_packed: bool = True,
               sym: bool = True) -> dict:
    """The calls of one layer in order: Hessian, damping, [act-order], factor, GPTQ
    (``sym=False``: the zero-point form)."""
    d_in = W.shape[1]
    H = torch.zeros((d_in, d_in), dtype=torch.float32, device=W.device)
    hessian_accumulate(X, H)
    lam = torch.empty(1, dtype=torch.float32, device=W.device)
    hessian_damp(H, damp, lambda_out=lam)
    perm = act_order_perm(H) if act_order else None
    U, info = chol_inverse_upper(H, perm)
    q = gptq_quantize_layer if sym else gptq_quantize_layer_zp
    res = q(W, U, info, bits, group_size, block_size, perm=perm, want_codes=want_codes, want_packed=want_packed)
    res.update({"H": H, "lambda": lam, "U": U, "info": info, "perm": perm})
    return res


# ------------------------------------------------------------------ kernel timing
PROF_CLASSES = ("xtx", "update", "columns", "rtn", "dequant", "update_split")


def profile_enable(on: bool = True) -> None:
    """Start (or stop) recording HIP events around the library's large kernels."""
    _check("pwq_profile_enable", lib().pwq_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{class: (milliseconds, algorithmic work, launches)} summed since profile_enable; clears the record."""
    n = len(PROF_CLASSES)
    ms, work, cnt = (ctypes.c_double * n)(), (ctypes.c_double * n)(), (ctypes.c_int64 * n)()
    _check("pwq_profile_read", lib().pwq_profile_read(ms, work, cnt, n))
    return {c: (ms[i], work[i], int(cnt[i])) for i, c in enumerate(PROF_CLASSES)}

