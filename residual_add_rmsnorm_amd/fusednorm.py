"""Python binding of libfusednorm (C ABI in include/fusednorm.h).

Argument marshalling only: every function takes torch tensors on the GPU,
passes their device pointers, sizes and torch's current HIP stream to the
entry point of the same name, and raises on a non-OK status. Outputs that are
not given are allocated with torch (the pages' wrappers allocate outputs the
caller leaves as None, contiguous even when the inputs are strided views). No
step of the computation runs here.

Loading fails loudly: if the built library is missing, importing this module
raises ``FusedNormLibraryMissing``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfusednorm.so")

FUSEDNORM_OK = 0
FUSEDNORM_ERR_INVALID_ARGUMENT = 1
FUSEDNORM_ERR_UNSUPPORTED = 2
FUSEDNORM_ERR_HIP = 3
FP8_GROUP = 128


class FusedNormLibraryMissing(RuntimeError):
    pass


class FusedNormError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{fn}: {_status_string(status)} ({detail})")


class FusedNormUnsupported(FusedNormError):
    """The library does not handle this input (the caller may take another path)."""


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise FusedNormLibraryMissing(
            f"{_LIB_PATH} is not built; run `python -m residual_add_rmsnorm_amd._build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    vpp = ctypes.POINTER(vp)
    sig = {
        "fused_add_rmsnorm": [vpp, i32, vp, vp, i64, i64, f32, vp, vp, vp],
        "fused_add_rmsnorm_quant_fp8": [vpp, i32, vp, vp, i64, i64, f32, vp, vp, vp, vp, vp],
        "fused_add_rmsnorm_quant_fp8_block": [vpp, i32, vp, vp, i64, i64, f32, i32, vp, vp, vp,
                                              vp, vp],
        "fused_add_rmsnorm_quant_fp8_static": [vpp, i32, vp, vp, i64, i64, f32, vp, vp, vp, vp,
                                               vp],
        "fused_rs_epilogue": [i32, vpp, i32, i64, vp, vp, vp, i64, i64, f32, vp, vp, vp, vp, vp,
                              vp],
        "ag_dual_rmsnorm": [i32, vp, i64, i64, i64, i64, vp, vp, f32, f32, vp, vp, vp, vp, vp],
        "qk_rmsnorm": [vp, i64, i64, i64, i64, vp, vp, f32, i32, vp, vp, vp, vp],
        "qk_rmsnorm_var": [vp, i64, i64, i64, i64, vp, vp],
        "sharded_rmsnorm": [vp, i64, i64, i64, vp, f32, i32, vp, vp, vp],
        "sharded_rmsnorm_var": [vp, i64, i64, i64, vp, vp],
        "fusednorm_e4m3_encode": [vp, vp, i64, vp],
        "fusednorm_stream_read": [vp, i64, vp, vp],
        "fusednorm_stream_copy": [vp, vp, i64, vp],
        "fusednorm_stream_mix": [vpp, i32, i64, i64, vpp, ctypes.POINTER(i64), i32, i64, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = i32
    lib.fusednorm_status_string.argtypes = [i32]
    lib.fusednorm_status_string.restype = ctypes.c_char_p
    lib.fusednorm_last_error.argtypes = []
    lib.fusednorm_last_error.restype = ctypes.c_char_p
    lib.fusednorm_version.argtypes = []
    lib.fusednorm_version.restype = i32
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def version() -> int:
    return int(_lib.fusednorm_version())


def _status_string(status: int) -> str:
    return _lib.fusednorm_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status == FUSEDNORM_OK:
        return
    detail = _lib.fusednorm_last_error().decode()
    cls = FusedNormUnsupported if status == FUSEDNORM_ERR_UNSUPPORTED else FusedNormError
    raise cls(fn, status, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype=torch.bfloat16) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, name: str, shape, itemsize: Optional[int] = None) -> None:
    """The C side sees only pointers: every buffer must cover exactly what the
    kernels read or write, so shapes are checked here before any call."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements")


def _same_device(ts, device) -> None:
    for name, t in ts:
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _partials(partials: Union[Sequence[torch.Tensor], torch.Tensor]):
    if isinstance(partials, torch.Tensor):
        if partials.dim() != 3:
            raise ValueError("stacked partials must be [P, T, H]")
        parts = list(partials.unbind(0))
    else:
        parts = list(partials)
    if not parts:
        raise ValueError("at least one partial buffer is required")
    for i, p in enumerate(parts):
        _need(p, f"partials[{i}]")
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    return parts, arr


def _rows(residual: torch.Tensor):
    """(T, H) of a [T, H] residual."""
    if residual.dim() != 2:
        raise ValueError(f"residual must be [T, H], got shape {tuple(residual.shape)}")
    return residual.shape


def _check_norm_shapes(parts, residual, weight, norm_out, residual_out, quant_out=None,
                       scale_out=None, scale_shape=None) -> None:
    T, H = _rows(residual)
    for i, p in enumerate(parts):
        _shape(p, f"partials[{i}]", (T, H))
    _shape(weight, "weight", (H,))
    _shape(residual_out, "residual_out", (T, H))
    if norm_out is not None:
        _shape(norm_out, "norm_out", (T, H))
    if quant_out is not None:
        _shape(quant_out, "quant_out", (T, H), itemsize=1)
    if scale_out is not None:
        _shape(scale_out, "scale_out", scale_shape)
    _same_device([(f"partials[{i}]", p) for i, p in enumerate(parts)] +
                 [("weight", weight), ("residual_out", residual_out), ("norm_out", norm_out),
                  ("quant_out", quant_out), ("scale_out", scale_out)], residual.device)


def _fp8_out(like: torch.Tensor) -> torch.Tensor:
    return torch.empty(like.shape, dtype=torch.float8_e4m3fn, device=like.device)


def fused_add_rmsnorm(partials, residual: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
                      norm_out: Optional[torch.Tensor] = None,
                      residual_out: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Σ partials (fp32) + residual -> (norm_out, residual_out), both bf16 [T, H].
    ``residual_out`` may be ``residual`` itself (in-place update)."""
    parts, arr = _partials(partials)
    _need(residual, "residual")
    _need(weight, "weight")
    T, H = _rows(residual)
    norm_out = torch.empty_like(residual) if norm_out is None else norm_out
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    _need(norm_out, "norm_out")
    _need(residual_out, "residual_out")
    _check_norm_shapes(parts, residual, weight, norm_out, residual_out)
    _check("fused_add_rmsnorm", _lib.fused_add_rmsnorm(
        arr, len(parts), _ptr(residual), _ptr(weight), T, H, float(eps), _ptr(norm_out),
        _ptr(residual_out), _stream(residual.device, stream)))
    return norm_out, residual_out


def fused_add_rmsnorm_quant_fp8(partials, residual: torch.Tensor, weight: torch.Tensor,
                                eps: float = 1e-6, norm_out: Optional[torch.Tensor] = None,
                                residual_out: Optional[torch.Tensor] = None,
                                quant_out: Optional[torch.Tensor] = None,
                                scale_out: Optional[torch.Tensor] = None, stream=None):
    """Fused epilogue + per-token OCP e4m3. Returns (quant_out e4m3 [T,H],
    scale_out fp32 [T], residual_out bf16 [T,H], norm_out or None)."""
    parts, arr = _partials(partials)
    _need(residual, "residual")
    _need(weight, "weight")
    T, H = _rows(residual)
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    quant_out = _fp8_out(residual) if quant_out is None else quant_out
    scale_out = (torch.empty(T, dtype=torch.float32, device=residual.device)
                 if scale_out is None else scale_out)
    _need(residual_out, "residual_out")
    _need(quant_out, "quant_out", dtype=None)
    _need(scale_out, "scale_out", dtype=torch.float32)
    if norm_out is not None:
        _need(norm_out, "norm_out")
    _check_norm_shapes(parts, residual, weight, norm_out, residual_out, quant_out, scale_out, (T,))
    _check("fused_add_rmsnorm_quant_fp8", _lib.fused_add_rmsnorm_quant_fp8(
        arr, len(parts), _ptr(residual), _ptr(weight), T, H, float(eps), _ptr(norm_out),
        _ptr(residual_out), _ptr(quant_out), _ptr(scale_out), _stream(residual.device, stream)))
    return quant_out, scale_out, residual_out, norm_out


def fused_add_rmsnorm_quant_fp8_block(partials, residual: torch.Tensor, weight: torch.Tensor,
                                      eps: float = 1e-6, group_size: int = FP8_GROUP,
                                      norm_out: Optional[torch.Tensor] = None,
                                      residual_out: Optional[torch.Tensor] = None,
                                      quant_out: Optional[torch.Tensor] = None,
                                      scale_out: Optional[torch.Tensor] = None, stream=None):
    """Fused epilogue + OCP e4m3 with one fp32 scale per 1x128 channel group.
    Returns (quant_out [T,H], scale_out [T, H/128], residual_out, norm_out or None)."""
    parts, arr = _partials(partials)
    _need(residual, "residual")
    _need(weight, "weight")
    T, H = _rows(residual)
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    quant_out = _fp8_out(residual) if quant_out is None else quant_out
    if scale_out is None:
        scale_out = torch.empty(T, max(H // max(int(group_size), 1), 1), dtype=torch.float32,
                                device=residual.device)
    _need(residual_out, "residual_out")
    _need(quant_out, "quant_out", dtype=None)
    _need(scale_out, "scale_out", dtype=torch.float32)
    if norm_out is not None:
        _need(norm_out, "norm_out")
    groups = H // int(group_size) if int(group_size) > 0 and H % int(group_size) == 0 else -1
    _check_norm_shapes(parts, residual, weight, norm_out, residual_out, quant_out, scale_out,
                       (T, groups) if groups > 0 else tuple(scale_out.shape))
    _check("fused_add_rmsnorm_quant_fp8_block", _lib.fused_add_rmsnorm_quant_fp8_block(
        arr, len(parts), _ptr(residual), _ptr(weight), T, H, float(eps), int(group_size),
        _ptr(norm_out), _ptr(residual_out), _ptr(quant_out), _ptr(scale_out),
        _stream(residual.device, stream)))
    return quant_out, scale_out, residual_out, norm_out


def fused_add_rmsnorm_quant_fp8_static(partials, residual: torch.Tensor, weight: torch.Tensor,
                                       scale_factor: Union[torch.Tensor, float],
                                       eps: float = 1e-6, norm_out: Optional[torch.Tensor] = None,
                                       residual_out: Optional[torch.Tensor] = None,
                                       quant_out: Optional[torch.Tensor] = None, stream=None):
    """Fused epilogue + OCP e4m3 with one static dequantisation scale for the
    tensor (a float or a one-element fp32 GPU tensor, as the pages accept; a
    float is copied to the device on every call, so pass a tensor in loops and
    under graph capture). Returns (quant_out e4m3 [T,H], residual_out, norm_out
    or None)."""
    parts, arr = _partials(partials)
    _need(residual, "residual")
    _need(weight, "weight")
    T, H = _rows(residual)
    if not isinstance(scale_factor, torch.Tensor):
        scale_factor = torch.tensor([float(scale_factor)], dtype=torch.float32,
                                    device=residual.device)
    _need(scale_factor, "scale_factor", dtype=torch.float32)
    if scale_factor.numel() != 1:
        raise ValueError("scale_factor must hold one value")
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    quant_out = _fp8_out(residual) if quant_out is None else quant_out
    _need(residual_out, "residual_out")
    _need(quant_out, "quant_out", dtype=None)
    if norm_out is not None:
        _need(norm_out, "norm_out")
    _check_norm_shapes(parts, residual, weight, norm_out, residual_out, quant_out)
    _same_device([("scale_factor", scale_factor)], residual.device)
    _check("fused_add_rmsnorm_quant_fp8_static", _lib.fused_add_rmsnorm_quant_fp8_static(
        arr, len(parts), _ptr(residual), _ptr(weight), T, H, float(eps), _ptr(scale_factor),
        _ptr(norm_out), _ptr(residual_out), _ptr(quant_out), _stream(residual.device, stream)))
    return quant_out, residual_out, norm_out


RS_PATTERNS = {1: "norm", 2: "static", 4: "static+norm", 6: "block", 7: "block", 8: "norm"}


def fused_rs_epilogue(pattern: int, partials, token_offset: int, residual: torch.Tensor,
                      weight: torch.Tensor, eps: float = 1e-6,
                      add_in: Optional[torch.Tensor] = None, scale_factor=None,
                      norm_out: Optional[torch.Tensor] = None,
                      residual_out: Optional[torch.Tensor] = None,
                      quant_out: Optional[torch.Tensor] = None,
                      scale_out: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Reduce-scatter epilogue on rows [token_offset, token_offset + T) of the
    partial buffers (each [token_num, H]); T = residual.shape[0]. Patterns 2
    and 4 take scale_factor as fused_add_rmsnorm_quant_fp8_static does. Returns
    a dict with the outputs the pattern writes."""
    if pattern not in RS_PATTERNS:
        raise FusedNormUnsupported("fused_rs_epilogue", FUSEDNORM_ERR_UNSUPPORTED,
                                   f"pattern {pattern} is not implemented")
    parts, arr = _partials(partials)
    _need(residual, "residual")
    _need(weight, "weight")
    T, H = _rows(residual)
    for i, p in enumerate(parts):
        if p.dim() != 2 or p.shape[1] != H or p.shape[0] < token_offset + T or token_offset < 0:
            raise ValueError(f"partials[{i}] must be [>= token_offset + T, H]")
    kind = RS_PATTERNS[pattern]
    residual_out = torch.empty_like(residual) if residual_out is None else residual_out
    if "norm" in kind and norm_out is None:
        norm_out = torch.empty_like(residual)
    if kind != "norm" and quant_out is None:
        quant_out = _fp8_out(residual)
    if kind == "block" and scale_out is None:
        scale_out = torch.empty(T, max(H // FP8_GROUP, 1), dtype=torch.float32,
                                device=residual.device)
    if kind.startswith("static"):
        if scale_factor is None:
            raise ValueError(f"pattern {pattern} needs scale_factor")
        if not isinstance(scale_factor, torch.Tensor):
            scale_factor = torch.tensor([float(scale_factor)], dtype=torch.float32,
                                        device=residual.device)
        _need(scale_factor, "scale_factor", dtype=torch.float32)
        if scale_factor.numel() != 1:
            raise ValueError("scale_factor must hold one value")
    else:
        scale_factor = None
    for name, t in (("add_in", add_in), ("residual_out", residual_out), ("norm_out", norm_out)):
        if t is not None:
            _need(t, name)
            _shape(t, name, (T, H))
    if quant_out is not None:
        _need(quant_out, "quant_out", dtype=None)
        _shape(quant_out, "quant_out", (T, H), itemsize=1)
    if scale_out is not None:
        _need(scale_out, "scale_out", dtype=torch.float32)
        _shape(scale_out, "scale_out", (T, H // FP8_GROUP) if H % FP8_GROUP == 0
               else tuple(scale_out.shape))
    _shape(weight, "weight", (H,))
    _same_device([("add_in", add_in), ("residual_out", residual_out), ("norm_out", norm_out),
                  ("quant_out", quant_out), ("scale_out", scale_out),
                  ("scale_factor", scale_factor)] +
                 [(f"partials[{i}]", p) for i, p in enumerate(parts)], residual.device)
    _check("fused_rs_epilogue", _lib.fused_rs_epilogue(
        int(pattern), arr, len(parts), int(token_offset), _ptr(add_in), _ptr(residual),
        _ptr(weight), T, H, float(eps), _ptr(scale_factor), _ptr(norm_out), _ptr(residual_out),
        _ptr(quant_out), _ptr(scale_out), _stream(residual.device, stream)))
    return {"residual": residual_out, "norm": norm_out, "codes": quant_out,
            "scales": scale_out if kind == "block" else None}


def _qkv_layout(qkv: torch.Tensor):
    if not isinstance(qkv, torch.Tensor) or not qkv.is_cuda or qkv.dtype != torch.bfloat16:
        raise TypeError("qkv must be a bf16 GPU tensor")
    if qkv.dim() != 2 or (qkv.shape[1] > 1 and qkv.stride(1) != 1):
        raise ValueError("qkv must be [T, row] with contiguous rows")
    T = qkv.shape[0]
    row_stride = qkv.stride(0) if T > 1 else qkv.shape[1]
    return T, row_stride


def _check_qk_shapes(qkv, q_size, kv_size, tensors) -> None:
    if q_size <= 0 or kv_size < 0 or qkv.shape[1] < q_size + kv_size:
        raise ValueError(f"qkv rows ({qkv.shape[1]}) must hold q_size + kv_size "
                         f"({q_size} + {kv_size})")
    if qkv.shape[0] > 1 and qkv.stride(0) < q_size + kv_size:
        raise ValueError("qkv rows overlap")
    for name, t, shape in tensors:
        if t is not None:
            _shape(t, name, shape)
    _same_device([(n, t) for n, t, _ in tensors], qkv.device)


def qk_rmsnorm(qkv: torch.Tensor, q_size: int, kv_size: int, q_weight: torch.Tensor,
               k_weight: torch.Tensor, eps: float = 1e-6, tp_world: int = 1,
               var_in: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
               k_out: Optional[torch.Tensor] = None, stream=None):
    """QK RMSNorm of the q | k segments of each row of ``qkv`` (rows may be
    strided). Returns contiguous (q_out [T, q_size], k_out [T, kv_size])."""
    T, row_stride = _qkv_layout(qkv)
    _need(q_weight, "q_weight")
    _need(k_weight, "k_weight")
    if var_in is not None:
        _need(var_in, "var_in", dtype=torch.float32)
    q_out = torch.empty(T, q_size, dtype=qkv.dtype, device=qkv.device) if q_out is None else q_out
    k_out = torch.empty(T, kv_size, dtype=qkv.dtype, device=qkv.device) if k_out is None else k_out
    _need(q_out, "q_out")
    _need(k_out, "k_out")
    _check_qk_shapes(qkv, q_size, kv_size, [
        ("q_weight", q_weight, (q_size,)), ("k_weight", k_weight, (kv_size,)),
        ("var_in", var_in, (T, 2)), ("q_out", q_out, (T, q_size)),
        ("k_out", k_out, (T, kv_size))])
    _check("qk_rmsnorm", _lib.qk_rmsnorm(
        _ptr(qkv), T, row_stride, int(q_size), int(kv_size), _ptr(q_weight), _ptr(k_weight),
        float(eps), int(tp_world), _ptr(var_in), _ptr(q_out), _ptr(k_out),
        _stream(qkv.device, stream)))
    return q_out, k_out


def qk_rmsnorm_var(qkv: torch.Tensor, q_size: int, kv_size: int,
                   var_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Local means of squares of the q and k segments: fp32 [T, 2]."""
    T, row_stride = _qkv_layout(qkv)
    var_out = (torch.empty(T, 2, dtype=torch.float32, device=qkv.device)
               if var_out is None else var_out)
    _need(var_out, "var_out", dtype=torch.float32)
    _check_qk_shapes(qkv, q_size, kv_size, [("var_out", var_out, (T, 2))])
    _check("qk_rmsnorm_var", _lib.qk_rmsnorm_var(
        _ptr(qkv), T, row_stride, int(q_size), int(kv_size), _ptr(var_out),
        _stream(qkv.device, stream)))
    return var_out


def ag_dual_rmsnorm(rows: torch.Tensor, q_lora_rank: int, kv_lora_rank: int,
                    x_gamma: torch.Tensor, y_gamma: torch.Tensor, x_eps: float = 1e-6,
                    y_eps: float = 1e-6, quant: bool = False, want_x: bool = True,
                    x_norm_out: Optional[torch.Tensor] = None,
                    y_norm_out: Optional[torch.Tensor] = None,
                    quant_out: Optional[torch.Tensor] = None,
                    scale_out: Optional[torch.Tensor] = None, stream=None) -> dict:
    """The MLA all-gather epilogue on gathered rows [T, q_lora_rank |
    kv_lora_rank | rope] (rows may be strided): pattern 1 (quant=False) returns
    ``x`` [T, q_lora_rank] and ``y`` [T, kv_lora_rank] bf16; pattern 2
    (quant=True) also ``codes`` (e4m3 [T, q_lora_rank]) and ``scales`` (fp32
    [T, q_lora_rank/128]), with ``x`` only when want_x."""
    T, row_stride = _qkv_layout(rows)
    q, kv = int(q_lora_rank), int(kv_lora_rank)
    _need(x_gamma, "x_gamma")
    _need(y_gamma, "y_gamma")
    if not quant:
        want_x = True
    if want_x and x_norm_out is None:
        x_norm_out = torch.empty(T, q, dtype=rows.dtype, device=rows.device)
    y_norm_out = torch.empty(T, kv, dtype=rows.dtype, device=rows.device) if y_norm_out is None \
        else y_norm_out
    if quant:
        if quant_out is None:
            quant_out = torch.empty(T, q, dtype=torch.float8_e4m3fn, device=rows.device)
        if scale_out is None:
            scale_out = torch.empty(T, max(q // 128, 1), dtype=torch.float32, device=rows.device)
        _need(quant_out, "quant_out", dtype=None)
        _need(scale_out, "scale_out", dtype=torch.float32)
    for name, t in (("x_norm_out", x_norm_out), ("y_norm_out", y_norm_out)):
        if t is not None:
            _need(t, name)
    tensors = [("x_gamma", x_gamma, (q,)), ("y_gamma", y_gamma, (kv,)),
               ("x_norm_out", x_norm_out, (T, q)), ("y_norm_out", y_norm_out, (T, kv))]
    if quant:
        # a q_lora_rank that is no multiple of 128 is refused by the library
        tensors += [("scale_out", scale_out, (T, q // 128) if q % 128 == 0 else scale_out.shape),
                    ("quant_out", quant_out, (T, q))]
        _shape(quant_out, "quant_out", (T, q), itemsize=1)
    _check_qk_shapes(rows, q, kv, tensors)
    _check("ag_dual_rmsnorm", _lib.ag_dual_rmsnorm(
        2 if quant else 1, _ptr(rows), T, row_stride, q, kv, _ptr(x_gamma), _ptr(y_gamma),
        float(x_eps), float(y_eps), _ptr(x_norm_out), _ptr(y_norm_out),
        _ptr(quant_out if quant else None), _ptr(scale_out if quant else None),
        _stream(rows.device, stream)))
    out = {"x": x_norm_out, "y": y_norm_out}
    if quant:
        out.update(codes=quant_out, scales=scale_out)
    return out


def sharded_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, tp_world: int = 1,
                    var_in: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    H: Optional[int] = None, stream=None) -> torch.Tensor:
    """RMSNorm of this rank's share of a hidden-sharded matrix: the first H
    (default: all) channels of each row of x (rows may be strided). var_in is the
    fp32 [T] sum of the ranks' local means (from sharded_rmsnorm_var plus an
    all-reduce), or None for local statistics. Returns contiguous [T, H]."""
    T, row_stride = _qkv_layout(x)
    H = x.shape[1] if H is None else int(H)
    _need(weight, "weight")
    if var_in is not None:
        _need(var_in, "var_in", dtype=torch.float32)
    out = torch.empty(T, H, dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out")
    _check_qk_shapes(x, H, 0, [("weight", weight, (H,)), ("var_in", var_in, (T,)),
                               ("out", out, (T, H))])
    _check("sharded_rmsnorm", _lib.sharded_rmsnorm(
        _ptr(x), T, row_stride, H, _ptr(weight), float(eps), int(tp_world), _ptr(var_in),
        _ptr(out), _stream(x.device, stream)))
    return out


def sharded_rmsnorm_var(x: torch.Tensor, H: Optional[int] = None,
                        var_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Local mean of squares of the first H channels of each row: fp32 [T]."""
    T, row_stride = _qkv_layout(x)
    H = x.shape[1] if H is None else int(H)
    var_out = (torch.empty(T, dtype=torch.float32, device=x.device)
               if var_out is None else var_out)
    _need(var_out, "var_out", dtype=torch.float32)
    _check_qk_shapes(x, H, 0, [("var_out", var_out, (T,))])
    _check("sharded_rmsnorm_var", _lib.sharded_rmsnorm_var(
        _ptr(x), T, row_stride, H, _ptr(var_out), _stream(x.device, stream)))
    return var_out


def e4m3_encode(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp32 -> OCP e4m3 with the FP8 epilogues' own conversion (saturating, RNE)."""
    _need(x, "x", dtype=torch.float32)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    _need(out, "out", dtype=None)
    _shape(out, "out", tuple(x.shape), itemsize=1)
    _same_device([("out", out)], x.device)
    _check("fusednorm_e4m3_encode", _lib.fusednorm_e4m3_encode(
        _ptr(x), _ptr(out), x.numel(), _stream(x.device, stream)))
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement aid: reads all of ``src`` (nbytes a multiple of 16 KiB) with
    plain 16-byte vector loads; ``sink`` is a 4-byte device buffer."""
    _need(src, "src", dtype=None)
    _need(sink, "sink", dtype=None)
    if sink.nbytes < 4:
        raise ValueError("sink must hold 4 bytes")
    rc = _lib.fusednorm_stream_read(_ptr(src), src.nbytes, _ptr(sink), _stream(src.device, stream))
    if rc != FUSEDNORM_OK:
        raise FusedNormError("fusednorm_stream_read", rc, "")


def stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Measurement aid: copies ``src`` to ``dst`` (same size, a multiple of
    16 KiB) with plain 16-byte vector loads and stores."""
    _need(src, "src", dtype=None)
    _need(dst, "dst", dtype=None)
    if dst.nbytes != src.nbytes:
        raise ValueError("src and dst must have the same size")
    rc = _lib.fusednorm_stream_copy(_ptr(src), _ptr(dst), src.nbytes, _stream(src.device, stream))
    if rc != FUSEDNORM_OK:
        raise FusedNormError("fusednorm_stream_copy", rc, "")


def stream_mix(srcs: Sequence[torch.Tensor], dsts: Sequence[torch.Tensor], rows: int,
               src_row_bytes: int, src_stride: Optional[int] = None, stream=None) -> None:
    """Measurement aid: the bytes of one epilogue launch without its arithmetic.
    For each of ``rows`` rows, reads ``src_row_bytes`` bytes of every source
    (row r of source k at byte ``r * src_stride``, default ``src_row_bytes``)
    and writes one row of every destination; destination k holds ``rows`` rows
    of ``dsts[k].nbytes // rows`` bytes, contiguous."""
    if rows <= 0:
        raise ValueError("rows must be positive")
    stride = src_row_bytes if src_stride is None else src_stride
    for t in list(srcs) + list(dsts):
        _need(t, "stream buffer", dtype=None)
    _same_device([(f"stream buffer {k}", t) for k, t in enumerate(list(srcs) + list(dsts))],
                 srcs[0].device)
    for k, t in enumerate(srcs):
        if t.nbytes < (rows - 1) * stride + src_row_bytes:
            raise ValueError(f"source {k} holds fewer than {rows} rows")
    widths = []
    for k, t in enumerate(dsts):
        if t.nbytes % rows:
            raise ValueError(f"destination {k}: {t.nbytes} bytes is not a whole number of rows")
        widths.append(t.nbytes // rows)
    sp = (ctypes.c_void_p * len(srcs))(*[_ptr(t) for t in srcs])
    dp = (ctypes.c_void_p * len(dsts))(*[_ptr(t) for t in dsts])
    wb = (ctypes.c_int64 * len(dsts))(*widths)
    rc = _lib.fusednorm_stream_mix(sp, len(srcs), src_row_bytes, stride, dp, wb, len(dsts), rows,
                                   _stream(srcs[0].device, stream))
    if rc != FUSEDNORM_OK:
        raise FusedNormError("fusednorm_stream_mix", rc, "")


__all__ = [
    "fused_add_rmsnorm", "fused_add_rmsnorm_quant_fp8", "fused_add_rmsnorm_quant_fp8_block",
    "fused_add_rmsnorm_quant_fp8_static", "fused_rs_epilogue", "ag_dual_rmsnorm",
    "qk_rmsnorm", "qk_rmsnorm_var", "sharded_rmsnorm", "sharded_rmsnorm_var", "e4m3_encode",
    "stream_read", "stream_copy", "stream_mix", "version", "library_path",
    "FusedNormError", "FusedNormUnsupported", "FusedNormLibraryMissing",
]
