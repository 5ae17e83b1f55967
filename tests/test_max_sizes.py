"""The largest shapes at the library's 32-bit addressing limits (MXFP4 2:4
with RMSNorm, K = 4096, bf16 inputs drawn on the GPU from a seeded
generator; every check compares sampled rows with the oracle on the same
input bytes, which is exact because MXFP4 preparation is row-independent):

  * prep at T = 2^21 - 64: code arrays just under 4 GiB, the largest prep
    whose stores use 32-bit offsets;
  * prep at T = 2^21 + 64: code arrays just over 4 GiB, which take the
    64-bit store path;
  * product at T = 2^20 - 64: token code arrays just under 2 GiB, the
    largest product the library accepts; T = 2^20 is refused before any
    launch.

Sampled rows: the first and last 16, rows whose tile bytes straddle the
2 GiB and 4 GiB offsets, and 64 random ones."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import compare_prepared, rel_fro

K = 4096


def _sq():
    import sparsity_prep_amd as sq
    sq.lib()
    return sq


def _inputs(T, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(T, K, device="cuda", dtype=torch.bfloat16, generator=g)
    x[:, ::197] *= 50  # outlier channels
    gamma = (1 + 0.1 * torch.randn(K, device="cuda", generator=g)).to(torch.bfloat16)
    return x, gamma


def _sample_rows(T, seed):
    rng = np.random.default_rng(seed)
    near = []
    for limit in (1 << 31, 1 << 32):
        # K tile t holds every row's 64 code bytes at t*T*64 + row*64: the
        # rows whose bytes straddle `limit` in the tile that crosses it
        t = limit // (T * 64)
        r = (limit - t * T * 64) // 64
        near += [r - 1, r, r + 1]
    rows = np.concatenate([np.arange(16), np.arange(T - 16, T), near, rng.integers(0, T, 64)])
    return np.unique(rows[(rows >= 0) & (rows < T)])


def _rows_of_ktiled(buf, T, per, rows):
    tb = 128 // per
    idx = torch.from_numpy(rows).to(buf.device)
    v = buf.view(K // 128, T, tb)[:, idx, :]
    return v.permute(1, 0, 2).reshape(len(rows), K // per).cpu().numpy()


def _gpu_rows(p, T, rows):
    idx = torch.from_numpy(rows).to(p.b_codes.device)
    return {"mask": p.mask[idx].cpu().numpy(),
            "b_codes": _rows_of_ktiled(p.b_codes, T, 2, rows), "b_scales": _rows_of_ktiled(p.b_scales, T, 32, rows),
            "r_codes": _rows_of_ktiled(p.r_codes, T, 2, rows), "r_scales": _rows_of_ktiled(p.r_scales, T, 32, rows)}


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_prep(sq, T, seed):
    x, gamma = _inputs(T, seed)
    p = sq.prepare(x, norm=sq.NORM_RMS, gamma=gamma, eps=1e-5, n=2, m=4, fmt=sq.MXFP4)
    torch.cuda.synchronize()
    rows = _sample_rows(T, seed)
    xr = _bits(x[torch.from_numpy(rows).cuda()])
    ora = oracle.prepare(xr, "bf16", K, 1, _bits(gamma), None, 1e-5, 2, 4, oracle.FMT_MXFP4, trace=True)
    stats = compare_prepared(_gpu_rows(p, T, rows), ora, 2, 4, what=f"T={T}")
    assert stats["mismatched"] == 0
    return x, gamma, p, rows


@pytest.mark.gpu
@pytest.mark.parametrize("T", [(1 << 21) - 64, (1 << 21) + 64], ids=["codes-below-4GiB", "codes-above-4GiB"])
def test_prep_at_the_offset_limits(T):
    sq = _sq()
    assert (T * K // 2 < (1 << 32)) == (T < (1 << 21))
    _check_prep(sq, T, seed=T % 1000)
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_product_at_the_operand_limit():
    sq = _sq()
    T = (1 << 20) - 64
    nout = 256
    x, gamma, p, rows = _check_prep(sq, T, seed=7)
    del x
    g = torch.Generator(device="cuda").manual_seed(11)
    w = (0.02 * torch.randn(nout, K, device="cuda", generator=g)).to(torch.bfloat16)
    wq = sq.quantize_weight(w, fmt=sq.MXFP4)
    y = sq.linear(p, wq)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    yr = y[idx].cpu().numpy().astype(np.float64)
    gr = _gpu_rows(p, T, rows)
    wc = wq.codes.view(K // 128, nout, 64).permute(1, 0, 2).reshape(nout, K // 2).cpu().numpy()
    ws = wq.scales.view(K // 128, nout, 4).permute(1, 0, 2).reshape(nout, K // 32).cpu().numpy()
    a = oracle.dequant(gr["b_codes"], gr["b_scales"], K, oracle.FMT_MXFP4)
    r = oracle.dequant(gr["r_codes"], gr["r_scales"], K, oracle.FMT_MXFP4)
    wd = oracle.dequant(wc, ws, K, oracle.FMT_MXFP4)
    ref = a @ wd.T + r @ wd.T
    absum = np.abs(a) @ np.abs(wd).T + np.abs(r) @ np.abs(wd).T
    assert rel_fro(yr, ref) <= 1e-3
    assert (np.abs(yr - ref) <= 2.0 * K * 2.0 ** -24 * absum).all()
    del p, y
    torch.cuda.empty_cache()
    # one more row reaches 2 GiB of token codes: refused before any launch
    big = sq.alloc_prepared(1 << 20, K, sq.MXFP4, torch.device("cuda"), with_mask=False)
    with pytest.raises(sq.SharqError, match="status 2"):
        sq.linear(big, wq)
