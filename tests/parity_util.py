"""Helpers shared by the GPU parity tests: host<->device marshalling and the
mismatch accounting for prepared tensors.

Masks, codes and scales must match the oracle bit for bit.  The only
mismatches tolerated are those whose root cause is a near tie in the
oracle's own FP32 values (a selection boundary, an E2M1 rounding midpoint, a
power-of-two block amax for E8M0, an E4M3 midpoint), each within one ulp;
every element downstream of such a root cause (its whole block, in both
paths) counts toward a budget of 1e-5 of the elements.  With FP64 norm sums
and correctly rounded arithmetic on both sides the expected count is 0.
"""
import numpy as np
import torch

import oracle
from sparsity_prep_amd.layout import ktile_to_rows

BUDGET = 1e-5
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def dev16(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def _near(a: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """|bits(a) - bits(t)| <= 1 for some target t (a >= 0, float32)."""
    ab = np.abs(a.astype(np.float32)).view(np.int32).astype(np.int64)
    tb = targets.astype(np.float32).view(np.int32).astype(np.int64)
    return (np.abs(ab[..., None] - tb) <= 1).any(-1)


def _pow2_near(a: np.ndarray) -> np.ndarray:
    ab = np.abs(a.astype(np.float32)).view(np.uint32)
    frac = ab & np.uint32(0x7FFFFF)
    return (frac == 0) | (frac == 0x7FFFFF) | (frac == 1)


def explained_blocks(ora: oracle.Prepared, n: int, m: int) -> np.ndarray:
    """Blocks [rows, K/B] containing a near tie of the oracle's values."""
    xh, R = ora.xhat, ora.resid
    rows, K = xh.shape
    B = oracle.block_size(ora.fmt)
    keys = np.abs(xh).view(np.int32).reshape(rows, K // m, m).astype(np.int64)
    srt = -np.sort(-keys, axis=-1)
    sel_tie = np.zeros((rows, K // m), bool)
    if 0 < n < m:
        sel_tie = np.abs(srt[..., n - 1] - srt[..., n]) <= 1
    sel_tie = np.repeat(sel_tie, m, axis=1)
    keep = oracle.unpack_mask(ora.mask)
    S = np.where(keep, xh, 0).astype(np.float32)
    ties = sel_tie.copy()
    for v, sc in ((S, ora.b_scales), (R, ora.r_scales)):
        if ora.fmt == oracle.FMT_MXFP4:
            E = sc.astype(np.int64) - 127
            u = v / np.exp2(np.repeat(E, B, axis=1)).astype(np.float64)
            ties |= _near(np.abs(u).astype(np.float32), MIDPOINTS)
            amax = np.abs(v.reshape(rows, K // B, B)).max(-1)
            ties |= np.repeat(_pow2_near(amax), B, axis=1)
        else:
            sval = np.array([oracle.e4m3_decode(int(s)) for s in range(256)], np.float32)
            D = (sval[sc] * np.float32(ora.G)).astype(np.float32)
            with np.errstate(divide="ignore", invalid="ignore"):
                u = np.where(np.repeat(D, B, axis=1) > 0, v / np.repeat(D, B, axis=1), 0)
            ties |= _near(np.abs(u).astype(np.float32), MIDPOINTS)
            amax = np.abs(v.reshape(rows, K // B, B)).max(-1)
            t = (amax / (np.float32(6.0) * np.float32(ora.G))).astype(np.float32)
            vals = np.unique(sval[np.isfinite(sval)])
            vals = vals[vals >= 0]
            mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
            ties |= np.repeat(_near(t, mids), B, axis=1)
    return ties.reshape(rows, K // B, B).any(-1)


def compare_prepared(gpu: dict, ora: oracle.Prepared, n: int, m: int, what: str = "") -> dict:
    """Assert parity of GPU prepared outputs (numpy dict) with the oracle's."""
    B = oracle.block_size(ora.fmt)
    rows, K = ora.b_codes.shape[0], ora.K
    bad = np.zeros((rows, K), bool)
    if gpu.get("mask") is not None:
        bad |= oracle.unpack_mask(gpu["mask"]) != oracle.unpack_mask(ora.mask)
    for key in ("b_codes", "r_codes"):
        bad |= oracle.unpack_codes(gpu[key]) != oracle.unpack_codes(getattr(ora, key))
    for key in ("b_scales", "r_scales"):
        bad |= np.repeat(gpu[key] != getattr(ora, key), B, axis=1)
    nbad = int(bad.sum())
    stats = {"elements": rows * K, "mismatched": nbad}
    if nbad == 0:
        return stats
    assert ora.xhat is not None, f"{what}: {nbad} mismatches (no trace to classify them)"
    expl = np.repeat(explained_blocks(ora, n, m), B, axis=1)
    unexplained = bad & ~expl
    first = np.argwhere(bad)[:5]
    assert not unexplained.any(), f"{what}: {int(unexplained.sum())} unexplained mismatches, first {first}"
    counted = int((np.repeat(bad.reshape(rows, K // B, B).any(-1), B, axis=1)).sum())
    stats["counted"] = counted
    assert counted <= BUDGET * rows * K, f"{what}: {counted} tie-explained elements exceed the budget"
    return stats


def prepared_to_host(p) -> dict:
    """Prepared tensors on the host, codes and scales in row-major form."""
    B = 32 if p.fmt == oracle.FMT_MXFP4 else 16
    T, K = p.T, p.K
    return {"mask": None if p.mask is None else host(p.mask),
            "b_codes": ktile_to_rows(host(p.b_codes), T, K, 2), "b_scales": ktile_to_rows(host(p.b_scales), T, K, B),
            "r_codes": ktile_to_rows(host(p.r_codes), T, K, 2), "r_scales": ktile_to_rows(host(p.r_scales), T, K, B),
            "G": None if p.global_scale is None else float(host(p.global_scale)[0])}


def weight_to_host(q):
    """Weight payload on the host: row-major codes [E, nout, K/2], scales [E, nout, K/B]."""
    B = 32 if q.fmt == oracle.FMT_MXFP4 else 16
    c, s = host(q.codes), host(q.scales)
    codes = np.stack([ktile_to_rows(c[e], q.nout, q.K, 2) for e in range(q.E)])
    scales = np.stack([ktile_to_rows(s[e], q.nout, q.K, B) for e in range(q.E)])
    return codes, scales


def rel_fro(y: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y.astype(np.float64) - ref)
    return float(num / den) if den > 0 else float(num)
