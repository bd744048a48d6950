"""Weight-only quantized linear for AMD Instinct MI355X (gfx950): thin Python binding.

Every function here has the name of a C entry point of ``include/qlinear.h`` and only marshals
arguments: it reads shapes, dtypes and data pointers of torch tensors (device memory), passes
torch's current HIP stream, and allocates outputs with torch when none are given.  All
computation runs in the HIP kernels of ``lib/libqlinear.so``; there is no CPU fallback.  If the
library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

__all__ = [
    "QLError",
    "QL_AFFINE",
    "QL_MXFP4",
    "QL_Q8_0",
    "QL_MXFP4_BLOCKS",
    "QL_Q4_K",
    "QL_Q6_K",
    "lib_path",
    "load_library",
    "qlinear_quantize",
    "qlinear_dequant",
    "qlinear_quantize_q8_0",
    "qlinear_take",
    "qlinear_transcode_gptq",
    "qlinear_transcode_gptq_planar",
    "qlinear_gptq_check_g_idx",
    "qlinear_transcode_awq",
    "qlinear_gemv",
    "qlinear_gemm",
    "qlinear_gemm_workspace_size",
    "qlinear_gemm_grouped",
    "qlinear_gemm_grouped_workspace_size",
    "qlinear_gemv_batched",
    "qlinear_gemv_batched_workspace_size",
    "qlinear_problem_list",
    "qlinear_route",
    "qlinear_apply_experts",
    "qlinear_apply_experts_workspace_size",
    "qlinear_apply_experts_noalloc",
    "qlinear_version",
]

QL_AFFINE, QL_MXFP4, QL_Q8_0, QL_MXFP4_BLOCKS, QL_Q4_K, QL_Q6_K = 0, 1, 2, 3, 4, 5
_QL_F32, _QL_F16, _QL_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "lib", "libqlinear.so")


class QLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[ql_status {status}] {message}")
        self.status = status


class _GemmWeight(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("biases", ctypes.c_void_p),
        ("layer_bias", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


class _Problem(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("biases", ctypes.c_void_p),
        ("layer_bias", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("m", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
    ]


_LIB = None
_P, _I64, _INT, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

_SIGNATURES = {
    "qlinear_quantize": (_INT, [_P, _I64, _I64, _INT, _INT, _INT, _P, _P, _P, _P]),
    "qlinear_dequant": (_INT, [_INT, _P, _P, _P, _INT, _I64, _I64, _INT, _INT, _P, _INT, _P]),
    "qlinear_quantize_q8_0": (_INT, [_P, _I64, _I64, _P, _P]),
    "qlinear_take": (_INT, [_P, _I64, _P, _I64, _I64, _P, _P]),
    "qlinear_transcode_gptq": (_INT, [_P, _P, _P, _INT, _I64, _I64, _INT, _INT, _INT, _P, _P, _P, _P]),
    "qlinear_transcode_gptq_planar": (_INT, [_P, _P, _P, _INT, _I64, _I64, _INT, _INT, _P, _P, _P, _P]),
    "qlinear_gptq_check_g_idx": (_INT, [_P, _I64, _INT]),
    "qlinear_transcode_awq": (_INT, [_P, _P, _P, _INT, _I64, _I64, _INT, _INT, _P, _P, _P, _P]),
    "qlinear_gemv": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _INT, _I64, _INT, _INT, _P, _P, _INT, _P]),
    "qlinear_gemm_workspace_size": (_SZ, [_I64, _I64, _I64, _INT, _INT]),
    "qlinear_gemm": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _INT, _I64, _INT, _INT, _P, _P, _INT, _P, _SZ, _P]),
    "qlinear_gemm_grouped_workspace_size": (_SZ, [_I64, _I64, ctypes.POINTER(_GemmWeight), _INT, _INT, _INT]),
    "qlinear_gemm_grouped": (_INT, [_P, _INT, _I64, _I64, ctypes.POINTER(_GemmWeight), _INT, _INT, _INT, _INT, _INT, _P,
                                    _SZ, _P]),
    "qlinear_gemv_batched_workspace_size": (_SZ, [ctypes.POINTER(_Problem), _INT]),
    "qlinear_gemv_batched": (_INT, [ctypes.POINTER(_Problem), _INT, _INT, _INT, _INT, _P, _SZ, _INT, _P]),
    "qlinear_route": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "qlinear_apply_experts_workspace_size": (_SZ, [_I64, _I64]),
    "qlinear_apply_experts": (_INT, [_INT, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _INT, _I64, _P, _INT, _P, _SZ, _P]),
    "qlinear_apply_experts_noalloc": (_INT, [_INT, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _INT, _I64, _P, _INT, _P]),
    "qlinear_last_error": (ctypes.c_char_p, []),
    "qlinear_version": (ctypes.c_char_p, []),
}


def load_library():
    """Load lib/libqlinear.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build the HIP library first (__graft_entry__.build())")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int):
    if status != 0:
        raise QLError(status, load_library().qlinear_last_error().decode())


def _torch():
    import torch

    return torch


def _dt(t) -> int:
    torch = _torch()
    d = t if isinstance(t, torch.dtype) else t.dtype
    if d == torch.float32:
        return _QL_F32
    if d == torch.float16:
        return _QL_F16
    if d == torch.bfloat16:
        return _QL_BF16
    raise QLError(3, f"unsupported dtype {d}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def qlinear_version() -> str:
    return load_library().qlinear_version().decode()


def qlinear_quantize(w, bits: int = 4, group_size: int = 64, param_dtype=None, packed=None, scales=None, biases=None):
    """Affine group quantize + pack of fp32 W [n, k] -> (packed u32 [n, k*bits/32] as int32,
    scales [n, k/g], biases [n, k/g] in param_dtype)."""
    torch = _torch()
    lib = load_library()
    param_dtype = param_dtype or torch.bfloat16
    n, k = w.shape
    if packed is None:
        packed = torch.empty((n, k * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // group_size), dtype=param_dtype, device=w.device)
    if biases is None:
        biases = torch.empty((n, k // group_size), dtype=param_dtype, device=w.device)
    _check(lib.qlinear_quantize(_ptr(w), n, k, bits, group_size, _dt(param_dtype), _ptr(packed), _ptr(scales),
                                _ptr(biases), _stream()))
    return packed, scales, biases


def qlinear_quantize_q8_0(w, blocks=None):
    """quantize_q8_0 of fp32 W [rows, k] -> blocks uint8 [rows, k/32*34]."""
    torch = _torch()
    lib = load_library()
    rows, k = w.shape
    if blocks is None:
        blocks = torch.empty((rows, k // 32 * 34), dtype=torch.uint8, device=w.device)
    _check(lib.qlinear_quantize_q8_0(_ptr(w), rows, k, _ptr(blocks), _stream()))
    return blocks


def qlinear_take(pos, src, dst=None):
    """take: rows of `src` (its first axis; any dtype and trailing shape) at int64 positions
    `pos`, bytes copied with no value decoded; a position out of range gives a zero row."""
    torch = _torch()
    lib = load_library()
    n_pos = pos.numel()
    if dst is None:
        dst = torch.empty((n_pos,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    row_bytes = math.prod(src.shape[1:]) * src.element_size()
    _check(lib.qlinear_take(_ptr(pos), n_pos, _ptr(src), src.shape[0], row_bytes, _ptr(dst), _stream()))
    return dst


def qlinear_gptq_check_g_idx(g_idx, group_size: int):
    """Raise QLError unless g_idx (int32 [k], any device; copied to host) is arange(k) //
    group_size: an activation-order map has no exact affine form."""
    import numpy as np
    lib = load_library()
    h = np.ascontiguousarray(np.asarray(g_idx.cpu() if hasattr(g_idx, "cpu") else g_idx, dtype=np.int32))
    _check(lib.qlinear_gptq_check_g_idx(h.ctypes.data, h.shape[0], group_size))


def qlinear_transcode_gptq(qweight, qzeros, scales, *, bits: int, group_size: int, v1_zeros: bool = False,
                           g_idx=None, packed=None, scales_out=None, biases_out=None):
    """GPTQ (continuous layout, contiguous groups) -> affine (packed [n, k*bits/32] int32, scales and
    biases [n, k/group_size] in scales' dtype).  qweight [k*bits/32, n], qzeros [G, n*bits/32]
    (int32), scales [G, n].  A g_idx, when given, is checked first (qlinear_gptq_check_g_idx)."""
    torch = _torch()
    lib = load_library()
    n = scales.shape[1]
    k = qweight.shape[0] * 32 // bits
    if g_idx is not None:
        qlinear_gptq_check_g_idx(g_idx, group_size)
    if packed is None:
        packed = torch.empty((n, qweight.shape[0]), dtype=torch.int32, device=qweight.device)
    so = scales_out if scales_out is not None else torch.empty((n, scales.shape[0]), dtype=scales.dtype,
                                                                device=qweight.device)
    bo = biases_out if biases_out is not None else torch.empty_like(so)
    _check(lib.qlinear_transcode_gptq(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dt(scales), k, n, bits, group_size,
                                      1 if v1_zeros else 0, _ptr(packed), _ptr(so), _ptr(bo), _stream()))
    return packed, so, bo


def qlinear_transcode_gptq_planar(qweight, qzeros, scales, *, bits: int, group_size: int, g_idx=None, packed=None,
                                  scales_out=None, biases_out=None):
    """GPTQ_P (planar blocks, true zeros) -> affine (packed [n, k*tb/32] int32 with tb = 8 for 7-bit
    sources, else bits; scales and biases [n, k/group_size] in scales' dtype).  qweight
    [k*bits/32, n], qzeros [G, n*bits/32] (int32), scales [G, n].  A g_idx, when given, is checked
    first (qlinear_gptq_check_g_idx)."""
    torch = _torch()
    lib = load_library()
    n = scales.shape[1]
    k = qweight.shape[0] * 32 // bits
    if g_idx is not None:
        qlinear_gptq_check_g_idx(g_idx, group_size)
    tb = 8 if bits == 7 else bits
    if packed is None:
        packed = torch.empty((n, k * tb // 32), dtype=torch.int32, device=qweight.device)
    so = scales_out if scales_out is not None else torch.empty((n, scales.shape[0]), dtype=scales.dtype,
                                                                device=qweight.device)
    bo = biases_out if biases_out is not None else torch.empty_like(so)
    _check(lib.qlinear_transcode_gptq_planar(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dt(scales), k, n, bits,
                                             group_size, _ptr(packed), _ptr(so), _ptr(bo), _stream()))
    return packed, so, bo


def qlinear_transcode_awq(qweight, qzeros, scales, *, bits: int, group_size: int, packed=None, scales_out=None,
                          biases_out=None):
    """AWQ GEMM (codes and zeros packed along the outputs) -> affine (packed [n, k*tb/32] int32 with
    tb = 8 for 7-bit sources, else bits; scales and biases [n, k/group_size] in scales' dtype).
    qweight [k, n*bits/32], qzeros [G, n*bits/32] (int32), scales [G, n]."""
    torch = _torch()
    lib = load_library()
    k, n = qweight.shape[0], scales.shape[1]
    tb = 8 if bits == 7 else bits
    if packed is None:
        packed = torch.empty((n, k * tb // 32), dtype=torch.int32, device=qweight.device)
    so = scales_out if scales_out is not None else torch.empty((n, scales.shape[0]), dtype=scales.dtype,
                                                                device=qweight.device)
    bo = biases_out if biases_out is not None else torch.empty_like(so)
    _check(lib.qlinear_transcode_awq(_ptr(qweight), _ptr(qzeros), _ptr(scales), _dt(scales), k, n, bits, group_size,
                                     _ptr(packed), _ptr(so), _ptr(bo), _stream()))
    return packed, so, bo


def qlinear_dequant(fmt: int, w0, w1=None, w2=None, *, rows: int, k: int, bits: int = 4, group_size: int = 64,
                    out_dtype=None, out=None):
    """dequant of an affine / MXFP4 / Q8_0 / MXFP4-blocks weight into out [rows, k] (out_dtype,
    default fp32)."""
    torch = _torch()
    lib = load_library()
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype, device=w0.device)
    pdt = _dt(w1) if (fmt == QL_AFFINE and w1 is not None) else _QL_BF16
    _check(lib.qlinear_dequant(fmt, _ptr(w0), _ptr(w1), _ptr(w2), pdt, rows, k, bits, group_size, _ptr(out),
                               _dt(out), _stream()))
    return out


def qlinear_gemv(x, packed, scales, biases, *, bits: int, group_size: int, layer_bias=None, y_dtype=None, y=None):
    """y [m, n] = x [m, k] . dequant(W [n, k])^T (+ layer_bias)."""
    torch = _torch()
    lib = load_library()
    m, k = x.shape
    n = packed.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or x.dtype, device=x.device)
    _check(lib.qlinear_gemv(_ptr(x), _dt(x), m, k, _ptr(packed), _ptr(scales), _ptr(biases), _dt(scales), n, bits,
                            group_size, _ptr(layer_bias), _ptr(y), _dt(y), _stream()))
    return y


def qlinear_gemm_workspace_size(m: int, n: int, k: int, bits: int, group_size: int) -> int:
    return int(load_library().qlinear_gemm_workspace_size(m, n, k, bits, group_size))


def qlinear_gemm(x, packed, scales, biases, *, bits: int, group_size: int, layer_bias=None, y_dtype=None, y=None,
                 workspace=None):
    """Prefill product on the matrix cores; same result contract as qlinear_gemv."""
    torch = _torch()
    lib = load_library()
    m, k = x.shape
    n = packed.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or x.dtype, device=x.device)
    need = qlinear_gemm_workspace_size(m, n, k, bits, group_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib.qlinear_gemm(_ptr(x), _dt(x), m, k, _ptr(packed), _ptr(scales), _ptr(biases), _dt(scales), n, bits,
                            group_size, _ptr(layer_bias), _ptr(y), _dt(y), _ptr(workspace), workspace.numel(),
                            _stream()))
    return y


def _gemm_weights(weights):
    arr = (_GemmWeight * max(1, len(weights)))()
    for i, w in enumerate(weights):
        arr[i] = _GemmWeight(_ptr(w["packed"]), _ptr(w["scales"]), _ptr(w["biases"]), _ptr(w.get("layer_bias")),
                             _ptr(w.get("y")), w["packed"].shape[0])
    return arr


def qlinear_gemm_grouped_workspace_size(m: int, k: int, weights: Sequence[dict], bits: int, group_size: int) -> int:
    return int(load_library().qlinear_gemm_grouped_workspace_size(m, k, _gemm_weights(weights), len(weights), bits,
                                                                  group_size))


def qlinear_gemm_grouped(x, weights: Sequence[dict], *, bits: int, group_size: int, y_dtype=None, workspace=None):
    """Prefill products of up to four weights that read the same x: each weight is a dict with
    tensors packed, scales, biases, optional layer_bias and optional output y (allocated here when
    absent).  Returns the list of outputs."""
    torch = _torch()
    lib = load_library()
    m, k = x.shape
    ws_in = [dict(w) for w in weights]
    for w in ws_in:
        if w.get("y") is None:
            w["y"] = torch.empty((m, w["packed"].shape[0]), dtype=y_dtype or x.dtype, device=x.device)
    arr = _gemm_weights(ws_in)
    if workspace is None:
        need = qlinear_gemm_grouped_workspace_size(m, k, ws_in, bits, group_size)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    ydt = ws_in[0]["y"] if ws_in else x
    _check(lib.qlinear_gemm_grouped(_ptr(x), _dt(x), m, k, arr, len(ws_in), _dt(ws_in[0]["scales"]) if ws_in else 2,
                                    bits, group_size, _dt(ydt), _ptr(workspace), workspace.numel(), _stream()))
    return [w["y"] for w in ws_in]


def qlinear_problem_list(problems):
    """Marshal a list of GEMV problems (dicts with tensors x, packed, scales, biases, y, optional
    layer_bias, and ints bits, group_size) into the C array qlinear_gemv_batched takes; pass the
    result instead of the list to skip re-marshalling on every call."""
    return _problem_array(problems)


def _problem_array(problems):
    if isinstance(problems, ctypes.Array):
        return problems
    arr = (_Problem * len(problems))()
    for i, p in enumerate(problems):
        x, packed, y = p["x"], p["packed"], p["y"]
        arr[i] = _Problem(_ptr(x), _ptr(packed), _ptr(p["scales"]), _ptr(p["biases"]), _ptr(p.get("layer_bias")),
                          _ptr(y), x.shape[0], packed.shape[0], x.shape[1], p["bits"], p["group_size"])
    return arr


def qlinear_gemv_batched_workspace_size(problems: Sequence[dict]) -> int:
    return int(load_library().qlinear_gemv_batched_workspace_size(_problem_array(problems), len(problems)))


def qlinear_gemv_batched(problems: Sequence[dict], *, x_dtype, param_dtype, y_dtype, workspace, upload: bool = True):
    """One launch (per class) over a list of GEMVs.  Each problem is a dict with tensors x, packed,
    scales, biases, y, optional layer_bias, and ints bits, group_size."""
    lib = load_library()
    arr = _problem_array(problems)
    _check(lib.qlinear_gemv_batched(arr, len(problems), _dt(x_dtype), _dt(param_dtype), _dt(y_dtype), _ptr(workspace),
                                    workspace.numel(), 1 if upload else 0, _stream()))


def qlinear_route(ids, e: int, offsets=None, perm=None):
    """Stable grouping of positions by expert id -> (offsets int32 [e+1], perm int32 [n_pos])."""
    torch = _torch()
    lib = load_library()
    n_pos = ids.numel()
    if offsets is None:
        offsets = torch.empty(e + 1, dtype=torch.int32, device=ids.device)
    if perm is None:
        perm = torch.full((max(n_pos, 1),), -1, dtype=torch.int32, device=ids.device)
    _check(lib.qlinear_route(_ptr(ids), n_pos, e, _ptr(offsets), _ptr(perm), _stream()))
    return offsets, perm


def qlinear_apply_experts_workspace_size(n_pos: int, e: int) -> int:
    return int(load_library().qlinear_apply_experts_workspace_size(n_pos, e))


def qlinear_apply_experts(fmt: int, w0, w1, ids, x, *, n: int, k: int, pos_per_row: int = 1, y_dtype=None, y=None,
                          workspace=None):
    """y [n_pos, n]: each position's x row through the expert its id names (zeros out of range)."""
    torch = _torch()
    lib = load_library()
    e = w0.shape[0]
    n_pos = ids.numel()
    if y is None:
        y = torch.empty((n_pos, n), dtype=y_dtype or x.dtype, device=x.device)
    need = qlinear_apply_experts_workspace_size(n_pos, e)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib.qlinear_apply_experts(fmt, _ptr(w0), _ptr(w1), e, n, k, _ptr(ids), n_pos, _ptr(x), _dt(x), pos_per_row,
                                     _ptr(y), _dt(y), _ptr(workspace), workspace.numel(), _stream()))
    return y


def qlinear_apply_experts_noalloc(fmt: int, w0, w1, ids, x, *, n: int, k: int, y, pos_per_row: int = 1):
    """qlinear_apply_experts with the routing scratch in the library's built-in device array: no
    workspace, nothing allocated (y is the caller's output tensor [n_pos, n])."""
    lib = load_library()
    e = w0.shape[0]
    _check(lib.qlinear_apply_experts_noalloc(fmt, _ptr(w0), _ptr(w1), e, n, k, _ptr(ids), ids.numel(), _ptr(x), _dt(x),
                                             pos_per_row, _ptr(y), _dt(y), _stream()))
    return y
