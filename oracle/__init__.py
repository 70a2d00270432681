"""CPU oracle for the fused TP epilogue and the MiniMax QK RMSNorm.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path. The arithmetic
lives in ``fusednorm_oracle.c`` (plain C, fp64, OpenMP over tokens); this module
only marshals numpy arrays into it. bf16 data travels as ``uint16`` bit
patterns and e4m3 codes as ``uint8``.

Pages cited: the tokenspeed ``triton.py`` page, section "AMD Triton All-Reduce +
RMSNorm" (the fused kernel), the tokenspeed ``trtllm.py`` page, sections
"Pattern enums" and "MiniMax QK fused AR + RMSNorm", and the vLLM
``minimax_rms_norm/rms_norm_tp`` page (the QK norm under tensor parallelism).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import _build

_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("FUSEDNORM_ORACLE_LIB")   # a test-built variant
    if override:
        lib = ctypes.CDLL(override)
    else:
        if _build.is_stale():
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_bf16_decode.restype = ctypes.c_double
    lib.orc_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_encode.restype = ctypes.c_uint16
    lib.orc_bf16_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_near_tie.restype = ctypes.c_uint8
    lib.orc_e4m3_near_tie.argtypes = [ctypes.c_double]
    lib.orc_bf16_encode_array.argtypes = [_f64p, _u16p, ctypes.c_int64]
    lib.orc_bf16_decode_array.argtypes = [_u16p, _f64p, ctypes.c_int64]
    lib.orc_e4m3_encode_array.argtypes = [_f64p, _u8p, ctypes.c_void_p, ctypes.c_int64]
    lib.orc_e4m3_decode_array.argtypes = [_u8p, _f64p, ctypes.c_int64]
    vp = ctypes.c_void_p
    lib.orc_fused_add_rmsnorm.restype = ctypes.c_int
    lib.orc_fused_add_rmsnorm.argtypes = [
        ctypes.POINTER(vp), ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_qk_means.restype = ctypes.c_int
    lib.orc_qk_means.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, vp]
    lib.orc_qk_rmsnorm.restype = ctypes.c_int
    lib.orc_qk_rmsnorm.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, vp, vp, ctypes.c_float, ctypes.c_int,
                                   vp, vp, vp, vp, vp]
    lib.orc_fused_add_rmsnorm_static.restype = ctypes.c_int
    lib.orc_fused_add_rmsnorm_static.argtypes = [
        ctypes.POINTER(vp), ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_float, vp, vp, vp, vp, vp, vp]
    lib.orc_ag_dual_rmsnorm.restype = ctypes.c_int
    lib.orc_ag_dual_rmsnorm.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, vp, vp, ctypes.c_float, ctypes.c_float,
                                        vp, vp, vp, vp, vp, vp, vp]
    lib.orc_sharded_means.restype = ctypes.c_int
    lib.orc_sharded_means.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp]
    lib.orc_sharded_rmsnorm.restype = ctypes.c_int
    lib.orc_sharded_rmsnorm.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp,
                                        ctypes.c_float, ctypes.c_int, vp, vp, vp]
    _lib = lib
    return lib


def max_threads() -> int:
    """OpenMP threads the oracle's token loops use."""
    return int(_load().orc_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


# ----------------------------------------------------------------------------- codecs

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().orc_bf16_decode_array(bits.reshape(-1), out.reshape(-1), bits.size)
    return out


def bf16_encode(v: np.ndarray) -> np.ndarray:
    v = _c(np.asarray(v, np.float64), np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_bf16_encode_array(v.reshape(-1), out.reshape(-1), v.size)
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().orc_e4m3_decode_array(codes.reshape(-1), out.reshape(-1), codes.size)
    return out


def e4m3_encode(v: np.ndarray, with_near_tie: bool = False):
    v = _c(np.asarray(v, np.float64), np.float64)
    out = np.empty(v.shape, np.uint8)
    tie = np.empty(v.shape, np.uint8) if with_near_tie else None
    _load().orc_e4m3_encode_array(v.reshape(-1), out.reshape(-1), _ptr(tie), v.size)
    return (out, tie.astype(bool)) if with_near_tie else out


# ----------------------------------------------------------------------------- fused epilogue

def fused_add_rmsnorm(partials: Sequence[np.ndarray], residual: np.ndarray, weight: np.ndarray,
                      eps: float, *, quant: Optional[str] = None, group_size: int = 128,
                      want_norm: bool = True, want_pre: bool = False) -> dict:
    """Runs the oracle on bf16 bit arrays.

    partials: P arrays uint16 [T, H]; residual uint16 [T, H]; weight uint16 [H].
    quant: None, "token" (one scale per token) or "block" (one per group_size
    consecutive channels). Returns a dict with ``residual`` (uint16 [T,H]),
    ``norm`` (uint16 [T,H] or None), and for quant ``codes`` (uint8 [T,H]),
    ``scales`` (fp32 [T] or [T, H/group_size]), ``near_tie`` (bool [T,H]);
    with want_pre also ``x`` (fp32 [T,H], the updated residual before its bf16
    rounding), ``y`` (fp64 [T,H], the normalised value before rounding) and
    ``r`` (fp64, the value handed to the e4m3 rounding).
    """
    lib = _load()
    parts = [_c(p, np.uint16) for p in partials]
    residual = _c(residual, np.uint16)
    weight = _c(weight, np.uint16)
    if residual.ndim != 2:
        raise ValueError("residual must be [T, H]")
    T, H = residual.shape
    for p in parts:
        if p.shape != (T, H):
            raise ValueError("partials must match residual's shape")
    if weight.shape != (H,):
        raise ValueError("weight must be [H]")
    P = len(parts)
    arr = (ctypes.c_void_p * P)(*[p.ctypes.data for p in parts])
    res_out = np.empty((T, H), np.uint16)
    norm_out = np.empty((T, H), np.uint16) if want_norm else None
    gs = 0
    codes = scales = tie = None
    if quant is not None:
        if quant == "token":
            gs = 0
            scales = np.empty((T,), np.float32)
        elif quant == "block":
            gs = int(group_size)
            if gs <= 0 or H % gs:
                raise ValueError("H must be a multiple of group_size")
            scales = np.empty((T, H // gs), np.float32)
        else:
            raise ValueError(quant)
        codes = np.empty((T, H), np.uint8)
        tie = np.empty((T, H), np.uint8)
    x = np.empty((T, H), np.float32) if want_pre else None
    y = np.empty((T, H), np.float64) if want_pre else None
    r = np.empty((T, H), np.float64) if (want_pre and quant is not None) else None
    rc = lib.orc_fused_add_rmsnorm(arr, P, _ptr(residual), _ptr(weight), T, H, float(eps), gs,
                                   _ptr(norm_out), _ptr(res_out), _ptr(codes), _ptr(scales),
                                   _ptr(tie), _ptr(x), _ptr(y), _ptr(r))
    if rc != 0:
        raise RuntimeError(f"oracle fused_add_rmsnorm failed with code {rc}")
    out = {"residual": res_out, "norm": norm_out}
    if quant is not None:
        out.update(codes=codes, scales=scales, near_tie=tie.astype(bool))
    if want_pre:
        out["x"] = x
        out["y"] = y
        if r is not None:
            out["r"] = r
    return out


def fused_add_rmsnorm_static(partials: Sequence[np.ndarray], residual: np.ndarray,
                             weight: np.ndarray, eps: float, scale: float, *,
                             want_norm: bool = True, want_pre: bool = False) -> dict:
    """The fused epilogue with one static fp32 FP8 scale s for the whole tensor:
    codes = e4m3(clamp(y / s)). Returns ``residual``, ``norm`` (or None),
    ``codes``, ``near_tie`` and with want_pre ``y`` and ``r`` (= y / s)."""
    lib = _load()
    parts = [_c(p, np.uint16) for p in partials]
    residual = _c(residual, np.uint16)
    weight = _c(weight, np.uint16)
    T, H = residual.shape
    for p in parts:
        if p.shape != (T, H):
            raise ValueError("partials must match residual's shape")
    arr = (ctypes.c_void_p * len(parts))(*[p.ctypes.data for p in parts])
    res_out = np.empty((T, H), np.uint16)
    norm_out = np.empty((T, H), np.uint16) if want_norm else None
    codes = np.empty((T, H), np.uint8)
    tie = np.empty((T, H), np.uint8)
    y = np.empty((T, H), np.float64) if want_pre else None
    r = np.empty((T, H), np.float64) if want_pre else None
    rc = lib.orc_fused_add_rmsnorm_static(arr, len(parts), _ptr(residual), _ptr(weight), T, H,
                                          float(eps), float(scale), _ptr(norm_out),
                                          _ptr(res_out), _ptr(codes), _ptr(tie), _ptr(y),
                                          _ptr(r))
    if rc != 0:
        raise RuntimeError(f"oracle fused_add_rmsnorm_static failed with code {rc}")
    out = {"residual": res_out, "norm": norm_out, "codes": codes, "near_tie": tie.astype(bool)}
    if want_pre:
        out.update(y=y, r=r)
    return out


# ----------------------------------------------------------------------------- reduce-scatter epilogue

# Codes of ReduceScatterFusionPattern (tokenspeed trtllm.py page, section
# "Pattern enums") that this epilogue implements.
RS_RESIDUAL_RMSNORM = 1
RS_RESIDUAL_RMSNORM_FP8 = 2
RS_RESIDUAL_RMSNORM_OUT_FP8 = 4
RS_RESIDUAL_RMSNORM_FP8_BLOCK = 6
RS_ADD_RESIDUAL_RMSNORM_FP8_BLOCK = 7
RS_ADD_RESIDUAL_RMSNORM = 8


def rs_epilogue(pattern: int, partials: Sequence[np.ndarray], token_offset: int,
                add_in: Optional[np.ndarray], residual: np.ndarray, weight: np.ndarray,
                eps: float, scale_factor: Optional[float] = None) -> dict:
    """The epilogue of trtllm_reducescatter_fusion (tokenspeed trtllm.py page,
    section "ReduceScatter fusion") for one rank's token slice: rows
    [token_offset, token_offset + T_local) of the P partial buffers (each
    [token_num, H]) are summed in fp32 in partial order, then add_in (patterns
    7 and 8) and the residual are added, in that order; then RMSNorm and the
    pattern's FP8 step (2 and 4: the static scale_factor; 6 and 7: 1x128
    groups). The reduced slice is the same arithmetic as the all-reduce
    epilogue with add_in as one more addend after the partials."""
    T = residual.shape[0]
    rows = [np.ascontiguousarray(np.asarray(p)[token_offset:token_offset + T]) for p in partials]
    if any(r.shape != residual.shape for r in rows):
        raise ValueError("the token slice runs past a partial buffer")
    needs_add = pattern in (RS_ADD_RESIDUAL_RMSNORM, RS_ADD_RESIDUAL_RMSNORM_FP8_BLOCK)
    if needs_add != (add_in is not None):
        raise ValueError("add_in is given exactly for patterns 7 and 8")
    if add_in is not None:
        rows.append(_c(add_in, np.uint16))
    if pattern in (RS_RESIDUAL_RMSNORM, RS_ADD_RESIDUAL_RMSNORM):
        return fused_add_rmsnorm(rows, residual, weight, eps)
    if pattern in (RS_RESIDUAL_RMSNORM_FP8, RS_RESIDUAL_RMSNORM_OUT_FP8):
        return fused_add_rmsnorm_static(rows, residual, weight, eps, scale_factor,
                                        want_norm=pattern == RS_RESIDUAL_RMSNORM_OUT_FP8)
    if pattern in (RS_RESIDUAL_RMSNORM_FP8_BLOCK, RS_ADD_RESIDUAL_RMSNORM_FP8_BLOCK):
        return fused_add_rmsnorm(rows, residual, weight, eps, quant="block", want_norm=False)
    raise ValueError(f"pattern {pattern} is not implemented")


# ----------------------------------------------------------------------------- all-gather epilogue (MLA)

def ag_dual_rmsnorm(rows: np.ndarray, q_rank: int, kv_rank: int, x_gamma: np.ndarray,
                    y_gamma: np.ndarray, x_eps: float, y_eps: float, quant: bool = False,
                    want_x: bool = True, want_pre: bool = False) -> dict:
    """The all-gather epilogue for MLA (tokenspeed trtllm.py page, section
    "AllGather fusion"): RMSNorm of the q_lora_rank and kv_lora_rank segments of
    each gathered row with their own weights and eps; with quant, 1x128 e4m3 of
    the normalised q part. Returns ``x`` (or None), ``y``, and with quant
    ``codes``, ``scales`` [T, q_rank/128], ``near_tie``."""
    rows, T, stride = _rows(rows, q_rank + kv_rank)
    xg, yg = _c(x_gamma, np.uint16), _c(y_gamma, np.uint16)
    x_out = np.empty((T, q_rank), np.uint16) if want_x else None
    y_out = np.empty((T, kv_rank), np.uint16)
    codes = np.empty((T, q_rank), np.uint8) if quant else None
    scales = np.empty((T, q_rank // 128), np.float32) if quant else None
    tie = np.empty((T, q_rank), np.uint8) if quant else None
    yx = np.empty((T, q_rank), np.float64) if want_pre else None
    yy = np.empty((T, kv_rank), np.float64) if want_pre else None
    rc = _load().orc_ag_dual_rmsnorm(_ptr(rows), T, stride, q_rank, kv_rank, _ptr(xg), _ptr(yg),
                                     float(x_eps), float(y_eps), _ptr(x_out), _ptr(y_out),
                                     _ptr(codes), _ptr(scales), _ptr(tie), _ptr(yx), _ptr(yy))
    if rc != 0:
        raise RuntimeError(f"oracle ag_dual_rmsnorm failed with code {rc}")
    out = {"x": x_out, "y": y_out}
    if quant:
        out.update(codes=codes, scales=scales, near_tie=tie.astype(bool))
    if want_pre:
        out.update(yx=yx, yy=yy)
    return out


# ----------------------------------------------------------------------------- QK norm

def _qk_view(qkv: np.ndarray, q_size: int, kv_size: int):
    qkv = np.asarray(qkv)
    if qkv.dtype != np.uint16 or qkv.ndim != 2:
        raise TypeError("qkv must be uint16 [T, row]")
    if qkv.strides[1] != 2:
        raise ValueError("qkv rows must be contiguous")
    T = qkv.shape[0]
    row_stride = qkv.strides[0] // 2 if T > 1 else qkv.shape[1]
    if qkv.shape[1] < q_size + kv_size:
        raise ValueError("row shorter than q_size + kv_size")
    return qkv, T, row_stride


def qk_means(qkv: np.ndarray, q_size: int, kv_size: int) -> np.ndarray:
    """Local means of squares [T, 2] (fp64) of the q and k segments."""
    qkv, T, stride = _qk_view(qkv, q_size, kv_size)
    out = np.empty((T, 2), np.float64)
    rc = _load().orc_qk_means(_ptr(qkv), T, stride, q_size, kv_size, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle qk_means failed with code {rc}")
    return out


def qk_rmsnorm(qkv: np.ndarray, q_size: int, kv_size: int, q_weight: np.ndarray,
               k_weight: np.ndarray, eps: float, tp_world: int = 1,
               var_in: Optional[np.ndarray] = None, want_pre: bool = False) -> dict:
    """QK RMSNorm on a [T, row] uint16 view whose rows hold q | k | v.

    var_in: None (local means, tp_world must be 1) or fp32 [T, 2], the sum over
    tp_world shards of the shard-local means. Returns ``q`` uint16 [T, q_size]
    and ``k`` uint16 [T, kv_size]; with want_pre also fp64 ``yq`` / ``yk``.
    """
    qkv, T, stride = _qk_view(qkv, q_size, kv_size)
    q_weight = _c(q_weight, np.uint16)
    k_weight = _c(k_weight, np.uint16)
    if var_in is not None:
        var_in = _c(var_in, np.float32)
        if var_in.shape != (T, 2):
            raise ValueError("var_in must be fp32 [T, 2]")
    q_out = np.empty((T, q_size), np.uint16)
    k_out = np.empty((T, kv_size), np.uint16)
    yq = np.empty((T, q_size), np.float64) if want_pre else None
    yk = np.empty((T, kv_size), np.float64) if want_pre else None
    rc = _load().orc_qk_rmsnorm(_ptr(qkv), T, stride, q_size, kv_size, _ptr(q_weight),
                                _ptr(k_weight), float(eps), int(tp_world), _ptr(var_in),
                                _ptr(q_out), _ptr(k_out), _ptr(yq), _ptr(yk))
    if rc != 0:
        raise RuntimeError(f"oracle qk_rmsnorm failed with code {rc}")
    out = {"q": q_out, "k": k_out}
    if want_pre:
        out.update(yq=yq, yk=yk)
    return out


# ----------------------------------------------------------------------------- sharded-hidden RMSNorm

def _rows(x: np.ndarray, H: int):
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("x must be uint16 [T, row]")
    if x.strides[1] != 2:
        raise ValueError("rows must be contiguous")
    if x.shape[1] < H:
        raise ValueError("row shorter than H")
    T = x.shape[0]
    return x, T, (x.strides[0] // 2 if T > 1 else x.shape[1])


def sharded_means(x: np.ndarray, H: int) -> np.ndarray:
    """Local means of squares [T] (fp64) of the first H channels of each row."""
    x, T, stride = _rows(x, H)
    out = np.empty((T,), np.float64)
    rc = _load().orc_sharded_means(_ptr(x), T, stride, H, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle sharded_means failed with code {rc}")
    return out


def sharded_rmsnorm(x: np.ndarray, H: int, weight: np.ndarray, eps: float, tp_world: int = 1,
                    var_in: Optional[np.ndarray] = None, want_pre: bool = False) -> dict:
    """RMSNorm of this rank's H channels of each row; var_in (fp32 [T]) is the sum
    of the ranks' local means, or None for local statistics (tp_world 1)."""
    x, T, stride = _rows(x, H)
    weight = _c(weight, np.uint16)
    if var_in is not None:
        var_in = _c(var_in, np.float32)
        if var_in.shape != (T,):
            raise ValueError("var_in must be fp32 [T]")
    out = np.empty((T, H), np.uint16)
    y = np.empty((T, H), np.float64) if want_pre else None
    rc = _load().orc_sharded_rmsnorm(_ptr(x), T, stride, H, _ptr(weight), float(eps),
                                     int(tp_world), _ptr(var_in), _ptr(out), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle sharded_rmsnorm failed with code {rc}")
    res = {"out": out}
    if want_pre:
        res["y"] = y
    return res


__all__ = [
    "max_threads", "bf16_decode", "bf16_encode", "e4m3_decode", "e4m3_encode",
    "fused_add_rmsnorm", "fused_add_rmsnorm_static", "rs_epilogue", "ag_dual_rmsnorm",
    "qk_means", "qk_rmsnorm",
    "sharded_means", "sharded_rmsnorm",
]
