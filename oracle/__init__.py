"""CPU oracle for the SharQ hot path (ctypes wrapper + FP64 reference GEMM).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product library or its
Python binding.  The arithmetic lives in ``sharq_oracle.c`` (plain scalar C,
each step documented there); this module builds and loads it, and adds the
layer product Y = deq(backbone).W^T + deq(residual).W^T in float64 with
numpy (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract: a sparse FP4 product on the
backbone plus a dense FP4 product on the residual, one weight payload).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sharq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT_F16, DT_BF16, DT_F32 = 0, 1, 2
NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
FMT_MXFP4, FMT_NVFP4 = 0, 1
DTYPE_CODE = {"f16": DT_F16, "bf16": DT_BF16, "f32": DT_F32}


def block_size(fmt: int) -> int:
    return 32 if fmt == FMT_MXFP4 else 16


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.or_e2m1_encode.argtypes = [f32]
        L.or_e2m1_encode.restype = ctypes.c_uint8
        L.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.or_e2m1_decode.restype = f32
        L.or_mx_exponent.argtypes = [f32]
        L.or_mx_exponent.restype = i32
        L.or_e4m3_encode.argtypes = [f32]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.or_e4m3_decode.restype = f32
        L.or_nv_global_scale.argtypes = [f32]
        L.or_nv_global_scale.restype = f32
        L.or_select_group.argtypes = [p, i32, i32, p]
        L.or_select_group.restype = None
        L.or_normalize.argtypes = [p, i32, i64, i64, i64, i32, p, p, i32, f32, p]
        L.or_prepare.argtypes = [p, i32, i64, i64, i64, i32, p, p, i32, f32, i32, i32, i32,
                                 p, i64, p, p, p, p, p, p, p, p, p]
        L.or_prepare_swiglu.argtypes = [p, i64, i64, i64, i32, i32, i32, p, i64, p, p, p, p, p, p,
                                        p, p, p]
        L.or_exp32.argtypes = [f32]
        L.or_exp32.restype = f32
        L.or_silu32.argtypes = [f32]
        L.or_silu32.restype = f32
        L.or_silu32_n.argtypes = [p, i64, p]
        L.or_silu32_n.restype = None
        L.or_e2m1_encode_n.argtypes = [p, i64, p]
        L.or_e2m1_encode_n.restype = None
        L.or_e4m3_encode_n.argtypes = [p, i64, p]
        L.or_e4m3_encode_n.restype = None
        L.or_mx_exponent_n.argtypes = [p, i64, p]
        L.or_mx_exponent_n.restype = None
        L.or_quantize_weight.argtypes = [p, i32, i64, i64, i64, i64, i32, p, p, p]
        L.or_dequant.argtypes = [p, p, i64, i64, i32, f32, p]
        L.or_quantize_rows.argtypes = [p, i32, i64, i64, i32, f32, p, p]
        for fn in (L.or_normalize, L.or_prepare, L.or_prepare_swiglu, L.or_quantize_weight, L.or_dequant,
                   L.or_quantize_rows):
            fn.restype = i32
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- scalars

def e2m1_encode(u: float) -> int:
    return int(lib().or_e2m1_encode(float(u)))


def e2m1_encode_array(u: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(u, dtype=np.float32)
    out = np.zeros(a.shape, np.uint8)
    lib().or_e2m1_encode_n(_ptr(a), a.size, _ptr(out))
    return out


def mx_exponent_array(amax: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.zeros(a.shape, np.int16)
    lib().or_mx_exponent_n(_ptr(a), a.size, _ptr(out))
    return out


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(a.shape, np.uint8)
    lib().or_e4m3_encode_n(_ptr(a), a.size, _ptr(out))
    return out


def e2m1_decode(code: int) -> float:
    return float(lib().or_e2m1_decode(int(code)))


def mx_exponent(amax: float) -> int:
    return int(lib().or_mx_exponent(float(amax)))


def e4m3_encode(x: float) -> int:
    return int(lib().or_e4m3_encode(float(x)))


def e4m3_decode(b: int) -> float:
    return float(lib().or_e4m3_decode(int(b)))


def nv_global_scale(amax: float) -> float:
    return float(lib().or_nv_global_scale(float(amax)))


def select_group(v: Sequence[float], n: int) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float32)
    keep = np.zeros(a.size, dtype=np.uint8)
    lib().or_select_group(_ptr(a), a.size, n, _ptr(keep))
    return keep


# ---------------------------------------------------------------- tensors

class Prepared:
    """Oracle outputs for one activation tensor (row-major, see or_prepare)."""

    def __init__(self, rows, K, fmt):
        B = block_size(fmt)
        self.K, self.fmt = K, fmt
        self.mask = np.zeros((rows, K // 8), np.uint8)
        self.b_codes = np.zeros((rows, K // 2), np.uint8)
        self.b_scales = np.zeros((rows, K // B), np.uint8)
        self.r_codes = np.zeros((rows, K // 2), np.uint8)
        self.r_scales = np.zeros((rows, K // B), np.uint8)
        self.gscale = np.zeros(1, np.float32)
        self.xhat = self.deqb = self.resid = None

    @property
    def G(self) -> float:
        return float(self.gscale[0])

    def deq_backbone(self) -> np.ndarray:
        return dequant(self.b_codes, self.b_scales, self.K, self.fmt, self.G)

    def deq_residual(self) -> np.ndarray:
        return dequant(self.r_codes, self.r_scales, self.K, self.fmt, self.G)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def prepare(x: np.ndarray, dtype: str, K: int, norm: int, gamma: Optional[np.ndarray],
            beta: Optional[np.ndarray], eps: float, n: int, m: int, fmt: int,
            rows: Optional[np.ndarray] = None, ldx: Optional[int] = None,
            trace: bool = False) -> Prepared:
    x = np.ascontiguousarray(x)
    T = x.size // (ldx or K) if x.ndim == 1 else x.shape[0]
    ldx = ldx or (x.shape[1] if x.ndim == 2 else K)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = T if r is None else r.size
    out = Prepared(nr, K, fmt)
    g = None if gamma is None else np.ascontiguousarray(gamma)
    b = None if beta is None else np.ascontiguousarray(beta)
    if trace:
        out.xhat = np.zeros((nr, K), np.float32)
        out.deqb = np.zeros((nr, K), np.float32)
        out.resid = np.zeros((nr, K), np.float32)
    rc = lib().or_prepare(_ptr(x), DTYPE_CODE[dtype], T, K, ldx, norm, _ptr(g), _ptr(b),
                          DTYPE_CODE[dtype], float(eps), n, m, fmt, _ptr(r), nr,
                          _ptr(out.mask), _ptr(out.b_codes), _ptr(out.b_scales),
                          _ptr(out.r_codes), _ptr(out.r_scales), _ptr(out.gscale),
                          _ptr(out.xhat), _ptr(out.deqb), _ptr(out.resid))
    _check(rc, "prepare")
    return out


def prepare_swiglu(gu: np.ndarray, K: int, n: int, m: int, fmt: int,
                   rows: Optional[np.ndarray] = None, trace: bool = False) -> Prepared:
    """Prepare SiLU(gate) * up from float32 rows [gate (K) | up (K) | ...]
    (the gate/up product's output), with no normalization."""
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    T, ld = gu.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = T if r is None else r.size
    out = Prepared(nr, K, fmt)
    if trace:
        out.xhat = np.zeros((nr, K), np.float32)
        out.deqb = np.zeros((nr, K), np.float32)
        out.resid = np.zeros((nr, K), np.float32)
    rc = lib().or_prepare_swiglu(_ptr(gu), T, K, ld, n, m, fmt, _ptr(r), nr, _ptr(out.mask),
                                 _ptr(out.b_codes), _ptr(out.b_scales), _ptr(out.r_codes),
                                 _ptr(out.r_scales), _ptr(out.gscale), _ptr(out.xhat), _ptr(out.deqb),
                                 _ptr(out.resid))
    _check(rc, "prepare_swiglu")
    return out


def exp32(y: float) -> float:
    return float(lib().or_exp32(float(y)))


def silu32(g: float) -> float:
    return float(lib().or_silu32(float(g)))


def silu32_array(g: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(a.shape, np.float32)
    lib().or_silu32_n(_ptr(a), a.size, _ptr(out))
    return out


def normalize(x: np.ndarray, dtype: str, K: int, norm: int, gamma, beta, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    out = np.zeros((T, K), np.float32)
    g = None if gamma is None else np.ascontiguousarray(gamma)
    b = None if beta is None else np.ascontiguousarray(beta)
    rc = lib().or_normalize(_ptr(x), DTYPE_CODE[dtype], T, K, x.shape[1], norm, _ptr(g), _ptr(b),
                            DTYPE_CODE[dtype], float(eps), _ptr(out))
    _check(rc, "normalize")
    return out


class QWeight:
    def __init__(self, E, nout, K, fmt):
        B = block_size(fmt)
        self.E, self.nout, self.K, self.fmt = E, nout, K, fmt
        self.codes = np.zeros((E, nout, K // 2), np.uint8)
        self.scales = np.zeros((E, nout, K // B), np.uint8)
        self.gscale = np.ones(E, np.float32)

    def deq(self, e: int = 0, rows: Optional[np.ndarray] = None) -> np.ndarray:
        c, s = self.codes[e], self.scales[e]
        if rows is not None:
            c, s = c[rows], s[rows]
        return dequant(c, s, self.K, self.fmt, float(self.gscale[e]))


def quantize_weight(w: np.ndarray, dtype: str, fmt: int) -> QWeight:
    w = np.ascontiguousarray(w)
    if w.ndim == 2:
        w = w[None]
    E, nout, K = w.shape
    q = QWeight(E, nout, K, fmt)
    rc = lib().or_quantize_weight(_ptr(w), DTYPE_CODE[dtype], E, nout, K, K, fmt,
                                  _ptr(q.codes), _ptr(q.scales), _ptr(q.gscale))
    _check(rc, "quantize_weight")
    return q


def quantize_rows(w_rows: np.ndarray, dtype: str, fmt: int, G: float = 1.0):
    """Quantize a sample of weight rows [n][K] with a known tensor scale G."""
    w_rows = np.ascontiguousarray(w_rows)
    n, K = w_rows.shape
    B = block_size(fmt)
    codes = np.zeros((n, K // 2), np.uint8)
    scales = np.zeros((n, K // B), np.uint8)
    _check(lib().or_quantize_rows(_ptr(w_rows), DTYPE_CODE[dtype], n, K, fmt, float(G),
                                  _ptr(codes), _ptr(scales)), "quantize_rows")
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray, K: int, fmt: int, G: float = 1.0) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows = codes.size // (K // 2)
    out = np.zeros((rows, K), np.float64)
    _check(lib().or_dequant(_ptr(codes), _ptr(scales), rows, K, fmt, float(G), _ptr(out)),
           "dequant")
    return out


# ---------------------------------------------------------------- layer product

def linear(prep: Prepared, wq: QWeight, expert: int = 0,
           out_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = deq(backbone).W^T + deq(residual).W^T in float64 (optionally for a
    subset of output columns ``out_rows`` of W)."""
    dw = wq.deq(expert, out_rows)
    return prep.deq_backbone() @ dw.T + prep.deq_residual() @ dw.T


def linear_grouped(prep: Prepared, wq: QWeight, offsets: np.ndarray,
                   row_index: Optional[np.ndarray]) -> np.ndarray:
    """Grouped (per-expert) product: sorted row r of group e reads prepared row
    row_index[r] (or r itself when row_index is None) and expert e's weight."""
    db, dr = prep.deq_backbone(), prep.deq_residual()
    nrows = int(offsets[-1])
    y = np.zeros((nrows, wq.nout), np.float64)
    for e in range(wq.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        src = np.arange(lo, hi) if row_index is None else row_index[lo:hi]
        dw = wq.deq(e)
        y[lo:hi] = db[src] @ dw.T + dr[src] @ dw.T
    return y


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[.., K/2] bytes -> [.., K] 4-bit codes (even k in the low nibble)."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def unpack_mask(mask: np.ndarray) -> np.ndarray:
    """[.., K/8] bytes -> [.., K] booleans (bit k%8 of byte k/8)."""
    return np.unpackbits(mask, axis=-1, bitorder="little").astype(bool)


# ---------------------------------------------------------------- compressed 2:4 backbone

def sp24_pack(prep: Prepared):
    """The NVFP4 backbone of `prep` (2:4 mask, K % 128 == 0) in the compressed
    form that gfx950's 2:4 sparse f16 matrix instruction takes (the library's
    NVFP4_SP24 format).  A re-arrangement of the oracle's own outputs, written
    from the layout's definition: per row and K tile of 128 elements, 48 bytes
    -- bytes 4c..4c+3 hold chunk c = 4p + 2h + u, the kept codes of elements
    32p + 16u + 8h + [0, 8) and then of 64 + 32p + 16u + 8h + [0, 8), two per
    group of four in ascending position (code v in nibble v % 2 of byte
    v // 2); bytes 32 + 4(2p + h) .. +3 hold, at bits 16u + 2v, the position
    of code v of chunk 4p + 2h + u within its group of four.  Block scales of
    a tile in the order of blocks 0, 1, 4, 5, 2, 3, 6, 7.

    Returns (records [rows, K/128, 48] uint8, scales [rows, K/16] uint8)."""
    codes = unpack_codes(prep.b_codes)
    keep = unpack_mask(prep.mask)
    rows, K = codes.shape
    if K % 128:
        raise ValueError("the compressed backbone needs whole K tiles")
    rec = np.zeros((rows, K // 128, 48), np.uint8)
    r = np.arange(rows)
    for t in range(K // 128):
        for p in (0, 1):
            for h in (0, 1):
                for u in (0, 1):
                    c = 4 * p + 2 * h + u
                    vals, pos = [], []
                    for base in (32 * p + 16 * u + 8 * h, 64 + 32 * p + 16 * u + 8 * h):
                        for g in (0, 1):
                            e0 = t * 128 + base + 4 * g
                            k4 = keep[:, e0:e0 + 4]
                            if not (k4.sum(axis=1) == 2).all():
                                raise ValueError("the compressed backbone needs exactly two kept per group of four")
                            first = np.argsort(~k4, axis=1, kind="stable")[:, :2]  # kept positions, ascending
                            for j in (0, 1):
                                vals.append(codes[r, e0 + first[:, j]])
                                pos.append(first[:, j])
                    for b in range(4):
                        rec[:, t, 4 * c + b] = vals[2 * b] | (vals[2 * b + 1] << 4)
                    word = np.zeros(rows, np.uint32)
                    for v in range(8):
                        word |= pos[v].astype(np.uint32) << np.uint32(16 * u + 2 * v)
                    off = 32 + 4 * (2 * p + h)
                    for b in range(4):
                        rec[:, t, off + b] |= ((word >> np.uint32(8 * b)) & np.uint32(0xFF)).astype(np.uint8)
    order = np.array([0, 1, 4, 5, 2, 3, 6, 7])
    sc = prep.b_scales.reshape(rows, K // 128, 8)[:, :, order].reshape(rows, K // 16)
    return rec, sc


def sp24_unpack(rec: np.ndarray, K: int):
    """Inverse of sp24_pack's code layout: dense backbone codes [rows, K/2]
    (zero at the positions not kept) and the mask bitmap [rows, K/8]."""
    rows = rec.shape[0]
    codes = np.zeros((rows, K), np.uint8)
    keep = np.zeros((rows, K), bool)
    r = np.arange(rows)
    for t in range(K // 128):
        for c in range(8):
            p, h, u = c >> 2, (c >> 1) & 1, c & 1
            word = np.zeros(rows, np.uint32)
            off = 32 + 4 * (2 * p + h)
            for b in range(4):
                word |= rec[:, t, off + b].astype(np.uint32) << np.uint32(8 * b)
            for v in range(8):
                base = (32 * p + 16 * u + 8 * h) if v < 4 else (64 + 32 * p + 16 * u + 8 * h)
                g = (v % 4) // 2
                position = ((word >> np.uint32(16 * u + 2 * v)) & np.uint32(3)).astype(np.int64)
                e = t * 128 + base + 4 * g + position
                nib = (rec[:, t, 4 * c + v // 2] >> (4 * (v % 2))) & 0xF
                codes[r, e] = nib
                keep[r, e] = True
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, np.packbits(keep, axis=1, bitorder="little")
