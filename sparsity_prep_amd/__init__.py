"""Python binding of the SharQ hot path library (libsharq.so, gfx950).

Argument marshalling only: tensors are allocated with PyTorch on the current
CUDA (HIP) device, their pointers and torch's current stream are handed to
the C ABI declared in include/sharq.h, and every step of the computation runs
in the library's HIP kernels.  There is no fallback: if libsharq.so is
missing, or no GPU is present, the calls raise.

    prep = prepare(x, norm=NORM_RMS, gamma=g, eps=1e-5, n=2, m=4, fmt=MXFP4)
    wq = quantize_weight(w, fmt=MXFP4)
    y = linear(prep, wq)          # float32 [T, nout]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsharq.so")

MXFP4, NVFP4, NVFP4_SP24 = 0, 1, 2  # NVFP4_SP24: NVFP4, backbone in the 2:4 compressed form
NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
_F16, _BF16, _F32 = 0, 1, 2
_DTYPE = {torch.float16: _F16, torch.bfloat16: _BF16}
_OUT_DTYPE = {torch.float32: _F32, torch.bfloat16: _BF16, torch.float16: _F16}


class SharqError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsharq.so (built by ``python -m sparsity_prep_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SharqError(f"{LIB_PATH} is missing: build it with `python -m sparsity_prep_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                ctypes.c_size_t)
        L.sharq_abi_version.restype = ctypes.c_int
        L.sharq_last_hip_error.restype = ctypes.c_int
        L.sharq_status_string.argtypes = [ctypes.c_int]
        L.sharq_status_string.restype = ctypes.c_char_p
        L.sharq_prepare_workspace_size.argtypes = [i64, i64, i32]
        L.sharq_prepare_workspace_size.restype = sz
        L.sharq_prepare.argtypes = [p, i32, i64, i64, i64, i32, p, p, f32, i32, i32, i32,
                                    p, p, p, p, p, p, p, sz, p]
        L.sharq_prepare.restype = ctypes.c_int
        L.sharq_prepare_noalloc.argtypes = [p, i32, i64, i64, i64, i32, p, p, f32, i32, i32, i32,
                                            p, p, p, p, p, p, p]
        L.sharq_prepare_noalloc.restype = ctypes.c_int
        L.sharq_prepare_swiglu.argtypes = [p, i64, i64, i64, i32, i32, i32, p, p, p, p, p, p, p, sz, p]
        L.sharq_prepare_swiglu.restype = ctypes.c_int
        L.sharq_quantize_weight_workspace_size.argtypes = [i64, i64, i64, i32]
        L.sharq_quantize_weight_workspace_size.restype = sz
        L.sharq_quantize_weight.argtypes = [p, i32, i64, i64, i64, i64, i32, p, p, p, p, sz, p]
        L.sharq_quantize_weight.restype = ctypes.c_int
        L.sharq_quantize_weight_gate_up.argtypes = [p, i32, i64, i64, i64, i64, i32, p, p, p, p, sz, p]
        L.sharq_quantize_weight_gate_up.restype = ctypes.c_int
        L.sharq_linear_workspace_size.argtypes = [i64, i64, i64, i64, i32]
        L.sharq_linear_workspace_size.restype = sz
        L.sharq_linear.argtypes = [p, p, p, p, p, i64, i64, i32, p, p, p, i64, i64, p, p, i64,
                                   p, i32, i64, p, sz, p]
        L.sharq_linear.restype = ctypes.c_int
        L.sharq_linear_swiglu.argtypes = [p, p, p, p, i64, i64, p, p, i64, i64, p, p, i64, i32, i32,
                                          p, p, p, p, p, p, i64, p]
        L.sharq_linear_swiglu.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().sharq_status_string(status).decode()
        if status == 8:  # SHARQ_ERR_HIP
            msg += f", hipError {lib().sharq_last_hip_error()}"
        raise SharqError(f"{what}: status {status} ({msg})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None


def block_size(fmt: int) -> int:
    return 32 if fmt == MXFP4 else 16


@dataclass
class Prepared:
    """Output of the fused preparation operator (on the GPU).  Codes and
    scales are K-tiled flat byte arrays (see layout.ktile_to_rows)."""
    b_codes: torch.Tensor     # uint8 [T*K/2] (NVFP4_SP24: [T*K*3/8], the compressed form)
    b_scales: torch.Tensor    # uint8 [T*K/B]
    r_codes: torch.Tensor     # uint8 [T*K/2]
    r_scales: torch.Tensor    # uint8 [T*K/B]
    mask: Optional[torch.Tensor]  # uint8 [T, K/8] row-major bitmap
    global_scale: Optional[torch.Tensor]  # float32 [1] (NVFP4)
    T: int
    K: int
    fmt: int


@dataclass
class QWeight:
    """One FP4 weight payload read by both paths; per expert, K-tiled with
    nout rows."""
    codes: torch.Tensor       # uint8 [E, nout*K/2]
    scales: torch.Tensor      # uint8 [E, nout*K/B]
    global_scale: Optional[torch.Tensor]  # float32 [E] (NVFP4)
    E: int
    nout: int
    K: int
    fmt: int


def alloc_prepared(T: int, K: int, fmt: int, device, with_mask: bool = True) -> Prepared:
    B = block_size(fmt)
    u8 = dict(dtype=torch.uint8, device=device)
    bb = T * K * 3 // 8 if fmt == NVFP4_SP24 else T * K // 2
    return Prepared(
        b_codes=torch.empty(bb, **u8), b_scales=torch.empty(T * K // B, **u8),
        r_codes=torch.empty(T * K // 2, **u8), r_scales=torch.empty(T * K // B, **u8),
        mask=torch.empty((T, K // 8), **u8) if with_mask else None,
        global_scale=torch.empty(1, dtype=torch.float32, device=device) if fmt != MXFP4 else None,
        T=T, K=K, fmt=fmt)


def prepare(x: torch.Tensor, norm: int = NORM_RMS, gamma: Optional[torch.Tensor] = None,
            beta: Optional[torch.Tensor] = None, eps: float = 1e-5, n: int = 2, m: int = 4,
            fmt: int = MXFP4, with_mask: bool = True, out: Optional[Prepared] = None) -> Prepared:
    """Fused norm -> N:M mask -> FP4 backbone -> residual -> FP4 residual."""
    if x.dim() != 2 or x.dtype not in _DTYPE or x.stride(1) != 1:
        raise SharqError("x must be a 2-D row-major float16/bfloat16 tensor")
    T, K = x.shape
    if out is None:
        out = alloc_prepared(T, K, fmt, x.device, with_mask)
    ws = _workspace(lib().sharq_prepare_workspace_size(T, K, fmt), x.device)
    st = lib().sharq_prepare(
        _ptr(x), _DTYPE[x.dtype], T, K, x.stride(0), norm, _ptr(gamma), _ptr(beta), float(eps),
        n, m, fmt, _ptr(out.mask), _ptr(out.b_codes), _ptr(out.b_scales), _ptr(out.r_codes),
        _ptr(out.r_scales), _ptr(out.global_scale), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(x.device))
    _check(st, "sharq_prepare")
    return out


def prepare_noalloc(x: torch.Tensor, out: Prepared, norm: int = NORM_RMS, gamma: Optional[torch.Tensor] = None,
                    beta: Optional[torch.Tensor] = None, eps: float = 1e-5, n: int = 2, m: int = 4) -> Prepared:
    """prepare() into caller-allocated outputs through the allocation-free
    entry point (its scratch is the library's own device array; NVFP4 takes
    at most SHARQ_NOALLOC_MAX_ROWS = 65536 rows; overlapping calls on one GPU
    race)."""
    if x.dim() != 2 or x.dtype not in _DTYPE or x.stride(1) != 1:
        raise SharqError("x must be a 2-D row-major float16/bfloat16 tensor")
    T, K = x.shape
    if out.T != T or out.K != K:
        raise SharqError("out does not match x's shape")
    st = lib().sharq_prepare_noalloc(
        _ptr(x), _DTYPE[x.dtype], T, K, x.stride(0), norm, _ptr(gamma), _ptr(beta), float(eps),
        n, m, out.fmt, _ptr(out.mask), _ptr(out.b_codes), _ptr(out.b_scales), _ptr(out.r_codes),
        _ptr(out.r_scales), _ptr(out.global_scale), _stream(x.device))
    _check(st, "sharq_prepare_noalloc")
    return out


def prepare_swiglu(gate_up: torch.Tensor, K: int, n: int = 2, m: int = 4, fmt: int = MXFP4,
                   with_mask: bool = True, out: Optional[Prepared] = None) -> Prepared:
    """Fused SiLU(gate) * up -> N:M mask -> FP4 backbone -> residual -> FP4
    residual, from float32 rows [gate (K) | up (K) | ...] (the gate/up
    product's output)."""
    if gate_up.dim() != 2 or gate_up.dtype != torch.float32 or gate_up.stride(1) != 1:
        raise SharqError("gate_up must be a 2-D row-major float32 tensor")
    T = gate_up.shape[0]
    if out is None:
        out = alloc_prepared(T, K, fmt, gate_up.device, with_mask)
    ws = _workspace(lib().sharq_prepare_workspace_size(T, K, fmt), gate_up.device)
    st = lib().sharq_prepare_swiglu(
        _ptr(gate_up), T, K, gate_up.stride(0), n, m, fmt, _ptr(out.mask), _ptr(out.b_codes),
        _ptr(out.b_scales), _ptr(out.r_codes), _ptr(out.r_scales), _ptr(out.global_scale), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(gate_up.device))
    _check(st, "sharq_prepare_swiglu")
    return out


def quantize_weight(w: torch.Tensor, fmt: int = MXFP4, gate_up: bool = False) -> QWeight:
    """RTN quantization of W[nout, K] or W[E, nout, K] into one FP4 payload.
    Rows may be strided (a column slice of a wider matrix): unit element
    stride, row stride ldw, expert stride nout * ldw.  NVFP4_SP24 names the
    NVFP4 payload (weights are never compressed).  gate_up: W stacks a
    SwiGLU gate (rows [0, nout/2)) and up (rows [nout/2, nout)) weight; the
    payload holds them interleaved in 32-row groups, the order linear_swiglu
    reads."""
    if fmt == NVFP4_SP24:
        fmt = NVFP4
    if w.dim() == 2:
        w = w.unsqueeze(0)
    if w.dim() != 3 or w.dtype not in _DTYPE or w.stride(2) != 1:
        raise SharqError("w must be a float16/bfloat16 [E, nout, K] tensor with unit element stride")
    E, nout, K = w.shape
    ldw = w.stride(1)
    if E > 1 and w.stride(0) != nout * ldw:
        raise SharqError("w: expert stride must be nout * row stride")
    B = block_size(fmt)
    u8 = dict(dtype=torch.uint8, device=w.device)
    q = QWeight(codes=torch.empty((E, nout * K // 2), **u8), scales=torch.empty((E, nout * K // B), **u8),
                global_scale=torch.empty(E, dtype=torch.float32, device=w.device) if fmt == NVFP4 else None,
                E=E, nout=nout, K=K, fmt=fmt)
    ws = _workspace(lib().sharq_quantize_weight_workspace_size(E, nout, K, fmt), w.device)
    entry = lib().sharq_quantize_weight_gate_up if gate_up else lib().sharq_quantize_weight
    st = entry(_ptr(w), _DTYPE[w.dtype], E, nout, K, ldw, fmt, _ptr(q.codes), _ptr(q.scales),
               _ptr(q.global_scale), _ptr(ws), 0 if ws is None else ws.numel(), _stream(w.device))
    _check(st, "sharq_quantize_weight_gate_up" if gate_up else "sharq_quantize_weight")
    return q


def linear(prep: Prepared, wq: QWeight, group_offsets: Optional[torch.Tensor] = None,
           row_index: Optional[torch.Tensor] = None, rows: Optional[int] = None,
           out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Y = deq(backbone) W^T + deq(residual) W^T, accumulated in float32 and
    stored as float32 (default) or rounded to bfloat16 / float16 (the dtype
    of `out` when given), optionally grouped by expert."""
    if prep.K != wq.K or (NVFP4 if prep.fmt == NVFP4_SP24 else prep.fmt) != wq.fmt:
        raise SharqError("prepared activations and weight disagree on K or format")
    if rows is None:
        rows = row_index.numel() if row_index is not None else prep.T
    dev = prep.b_codes.device
    if out is None:
        if out_dtype not in _OUT_DTYPE:
            raise SharqError("out_dtype must be float32, bfloat16 or float16")
        out = torch.empty((rows, wq.nout), dtype=out_dtype, device=dev)
    elif (out.dim() != 2 or out.dtype not in _OUT_DTYPE or out.shape[0] < rows or out.shape[1] != wq.nout
          or out.stride(1) != 1):
        raise SharqError("out must be a float32/bfloat16/float16 [rows, nout] tensor with unit column stride")
    ws = _workspace(lib().sharq_linear_workspace_size(rows, wq.K, wq.nout, wq.E, prep.fmt), dev)
    st = lib().sharq_linear(
        _ptr(prep.b_codes), _ptr(prep.b_scales), _ptr(prep.r_codes), _ptr(prep.r_scales),
        _ptr(prep.global_scale), prep.T, prep.K, prep.fmt, _ptr(wq.codes), _ptr(wq.scales),
        _ptr(wq.global_scale), wq.E, wq.nout, _ptr(group_offsets), _ptr(row_index), rows,
        _ptr(out), _OUT_DTYPE[out.dtype], out.stride(0), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st, "sharq_linear")
    return out


def linear_swiglu(prep: Prepared, wq: QWeight, n: int = 2, m: int = 4, group_offsets: Optional[torch.Tensor] = None,
                  row_index: Optional[torch.Tensor] = None, rows: Optional[int] = None, with_mask: bool = True,
                  out: Optional[Prepared] = None, y: Optional[torch.Tensor] = None) -> Prepared:
    """The gate/up product (MXFP4, weight from quantize_weight(..., gate_up=True))
    with the down projection's preparation in its epilogue: returns the
    MXFP4 prepared activation SiLU(gate) * up of [rows, nout/2].  y: an
    optional float32 [rows, nout] tensor that also receives the product (in
    the interleaved column order)."""
    if prep.fmt != MXFP4 or wq.fmt != MXFP4 or prep.K != wq.K:
        raise SharqError("linear_swiglu takes MXFP4 activations and weights of the same K")
    if rows is None:
        rows = row_index.numel() if row_index is not None else prep.T
    dev = prep.b_codes.device
    Kd = wq.nout // 2
    if out is None:
        out = alloc_prepared(rows, Kd, MXFP4, dev, with_mask)
    elif out.T != rows or out.K != Kd or out.fmt != MXFP4:
        raise SharqError("out does not match [rows, nout/2] MXFP4")
    if y is not None and (y.dim() != 2 or y.dtype != torch.float32 or y.shape[0] < rows or y.shape[1] != wq.nout
                          or y.stride(1) != 1):
        raise SharqError("y must be a float32 [rows, nout] tensor with unit column stride")
    st = lib().sharq_linear_swiglu(
        _ptr(prep.b_codes), _ptr(prep.b_scales), _ptr(prep.r_codes), _ptr(prep.r_scales), prep.T, prep.K,
        _ptr(wq.codes), _ptr(wq.scales), wq.E, wq.nout, _ptr(group_offsets), _ptr(row_index), rows, n, m,
        _ptr(out.mask), _ptr(out.b_codes), _ptr(out.b_scales), _ptr(out.r_codes), _ptr(out.r_scales),
        _ptr(y), 0 if y is None else y.stride(0), _stream(dev))
    _check(st, "sharq_linear_swiglu")
    return out
