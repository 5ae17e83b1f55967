"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Prepared masks, codes and scales must be bit-exact (tie allowance in
parity_util); layer outputs must be within relative Frobenius error 1e-3 of
the oracle's FP64 product of the same dequantized codes.  Small cases span
several tiles and ragged tails; full-size workloads (Llama-3.1-8B prefill
and decode, Qwen2.5-7B NVFP4 prefill, Qwen3-30B-A3B MoE experts) are checked
in full for the prepared tensors where the oracle is fast enough, otherwise
on sampled rows, with the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import load as load_golden
from parity_util import compare_prepared, dev16, host, prepared_to_host, rel_fro, weight_to_host

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparsity_prep_amd as sq
    sq.lib()
    return sq


def sq():
    import sparsity_prep_amd
    return sparsity_prep_amd


def gpu_prepare(x_bits, dtype, K, norm, g_bits, b_bits, eps, n, m, fmt, with_mask=True):
    x = dev16(x_bits, dtype)
    g = dev16(g_bits, dtype) if g_bits is not None else None
    b = dev16(b_bits, dtype) if b_bits is not None else None
    p = sq().prepare(x, norm=norm, gamma=g, beta=b, eps=eps, n=n, m=m, fmt=fmt, with_mask=with_mask)
    torch.cuda.synchronize()
    return p


def check_prep(x, dtype, K, norm, g, b, eps, n, m, fmt, rows=None, what=""):
    p = gpu_prepare(x, dtype, K, norm, g, b, eps, n, m, fmt)
    gh = prepared_to_host(p)
    o = oracle.prepare(x, dtype, K, norm, g, b, eps, n, m, fmt, rows=rows, trace=True)
    if rows is not None:
        gh = {k: (v[rows] if isinstance(v, np.ndarray) else v) for k, v in gh.items()}
    stats = compare_prepared(gh, o, n, m, what)
    if fmt == oracle.FMT_NVFP4:
        assert gh["G"] == o.G, (what, gh["G"], o.G)
    return p, gh, o, stats


# ---------------------------------------------------------------- hand-worked rows

@pytest.mark.parametrize("name", ["worked_mxfp4_2of4.txt", "worked_nvfp4_2of4.txt"])
def test_golden_rows(name):
    g = load_golden(name)
    p = gpu_prepare(g["x"], g["dtype"], g["K"], g["norm"], None, None, g["eps"], g["N"], g["M"], g["fmt"])
    gh = prepared_to_host(p)
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
        assert np.array_equal(gh[key], g[key]), (key, gh[key], g[key])
    if g["fmt"] == oracle.FMT_NVFP4:
        assert gh["G"] == g["gscale"]


# ---------------------------------------------------------------- prep sweeps

PREP_CASES = [
    # (fmt, norm, dtype, n, m, T, K)
    (0, 1, "bf16", 2, 4, 5, 256),
    (0, 1, "f16", 2, 4, 16, 256),
    (0, 0, "bf16", 2, 4, 37, 2560),
    (0, 2, "bf16", 2, 4, 7, 1024),
    (0, 1, "bf16", 1, 4, 3, 4096),
    (0, 1, "bf16", 3, 4, 9, 3584),
    (0, 1, "bf16", 4, 8, 4, 512),
    (0, 1, "bf16", 1, 2, 4, 96),
    (0, 1, "bf16", 8, 16, 6, 1536),
    (0, 0, "bf16", 5, 16, 6, 2048 + 32),
    (0, 1, "bf16", 1, 1, 2, 64),
    (0, 1, "bf16", 0, 4, 2, 128),
    (0, 1, "bf16", 4, 4, 3, 800),
    (0, 1, "bf16", 2, 4, 5, 4608),      # norm with a re-read of the row
    (0, 2, "f16", 2, 4, 3, 5120 + 32),
    (0, 0, "f16", 2, 4, 40, 768),
    (1, 1, "bf16", 2, 4, 9, 256),
    (1, 0, "bf16", 2, 4, 33, 2048 + 16),
    (1, 2, "bf16", 2, 4, 4, 1024),
    (1, 1, "f16", 1, 2, 5, 3584),
    (1, 1, "bf16", 8, 16, 3, 4608),
    (1, 0, "bf16", 4, 4, 2, 48),
    (0, 1, "bf16", 2, 4, 3, 8192 + 128),   # MXFP4 norm row beyond one workgroup's registers
    (1, 2, "bf16", 2, 4, 3, 6144),         # NVFP4 statistics: four chunks per wave
    (1, 1, "bf16", 2, 4, 3, 8192 + 512),   # NVFP4 norm statistics, looped row
    (1, 0, "bf16", 2, 4, 5, 12288 + 16),   # NVFP4 amax, eight chunks per wave
    (1, 0, "bf16", 2, 4, 4, 18944),        # NVFP4 amax, sixteen chunks per wave
    (1, 0, "bf16", 2, 4, 2, 32768 + 256),  # NVFP4 amax, looped row
    # MXFP4 norm rows from 2048 on run several rows per workgroup: a ragged last workgroup
    (0, 1, "bf16", 2, 4, 2049, 4096),
    (0, 2, "bf16", 2, 4, 2049, 8192),
    (0, 1, "bf16", 2, 4, 4097, 4096),
    (0, 2, "f16", 2, 4, 4097, 8192),
]


@pytest.mark.parametrize("case", PREP_CASES, ids=lambda c: "fmt%d-norm%d-%s-%d:%d-T%d-K%d" % c)
def test_prep_sweep(case):
    fmt, norm, dtype, n, m, T, K = case
    tag = PREP_CASES.index(case)
    x = synth.small_case(K, T, dtype, outliers=max(1, K // 200), mult=40.0,
                         dist="t" if fmt else "normal", tag=tag)
    g = synth.small_gamma(K, dtype, tag=tag) if norm else None
    b = synth.small_gamma(K, dtype, tag=tag + 1) if norm == 2 else None
    _, _, _, stats = check_prep(x, dtype, K, norm, g, b, 1e-5, n, m, fmt, what=str(case))
    assert stats["mismatched"] == 0, stats


@pytest.mark.parametrize("fmt", [0, 1])
def test_prep_edge_values(fmt):
    K, T = 512, 8
    rng = np.random.default_rng(11)
    x = np.zeros((T, K), np.float32)
    x[1] = rng.standard_normal(K) * 2.0 ** -130           # subnormal range (bf16 keeps them)
    x[2] = rng.standard_normal(K) * 2.0 ** 120             # near the top of the range
    x[3] = 1.0                                              # every magnitude tied
    x[4] = np.where(np.arange(K) % 2, -1.0, 1.0) * 0.75     # E2M1 midpoints everywhere
    x[5, ::7] = 3.0e38
    x[6] = rng.integers(-3, 4, K) * 0.5                     # heavy ties, small integers
    x[7] = -0.0
    bits = synth.to_bits(x, "bf16")
    _, _, _, stats = check_prep(bits, "bf16", K, 0, None, None, 0.0, 2, 4, fmt, what=f"edge fmt{fmt}")
    assert stats["mismatched"] == 0


def test_prep_zero_rows_is_noop():
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    p = sq().prepare(x, norm=0, n=2, m=4, fmt=0)
    assert p.b_codes.numel() == 0 and p.b_scales.numel() == 0


def test_prep_strided_rows():
    K, T, ld = 512, 6, 512 + 64
    x = synth.small_case(ld, T, "bf16", tag=77)
    xt = dev16(x, "bf16")[:, :K]
    p = sq().prepare(xt, norm=0, n=2, m=4, fmt=0)
    torch.cuda.synchronize()
    o = oracle.prepare(np.ascontiguousarray(x[:, :K]), "bf16", K, 0, None, None, 0.0, 2, 4, 0, trace=True)
    compare_prepared(prepared_to_host(p), o, 2, 4, "strided")


# ---------------------------------------------------------------- fused SiLU(gate) * up prep

SWIGLU_CASES = [
    # (fmt, n, m, T, K, ld)
    (0, 2, 4, 5, 256, 512),
    (0, 2, 4, 37, 2560 + 32, 2 * (2560 + 32) + 64),
    (0, 1, 4, 3, 4096, 8192),
    (0, 4, 8, 9, 1024, 2048),
    (0, 2, 4, 2, 14336, 28672),
    (1, 2, 4, 9, 256, 512),
    (1, 2, 4, 33, 2048 + 16, 2 * (2048 + 16)),
    (1, 8, 16, 4, 3584, 7168 + 4),
    (1, 2, 4, 3, 18944, 37888),
]


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=lambda c: "fmt%d-%d:%d-T%d-K%d-ld%d" % c)
def test_prep_swiglu(case):
    fmt, n, m, T, K, ld = case
    tag = SWIGLU_CASES.index(case)
    gu = synth.small_gate_up(K, T, ld, tag=tag)
    p = sq().prepare_swiglu(torch.from_numpy(gu).cuda(), K, n=n, m=m, fmt=fmt)
    torch.cuda.synchronize()
    gh = prepared_to_host(p)
    o = oracle.prepare_swiglu(gu, K, n, m, fmt, trace=True)
    stats = compare_prepared(gh, o, n, m, str(case))
    assert stats["mismatched"] == 0, stats
    if fmt == oracle.FMT_NVFP4:
        assert gh["G"] == float(o.gscale[0])


def test_prep_swiglu_column_slice():
    """The gate/up block may be a column slice of a wider output buffer."""
    K, T = 512, 6
    gu = synth.small_gate_up(K, T, 2 * K + 128, tag=99)
    d = torch.from_numpy(gu).cuda()[:, 64:64 + 2 * K]
    p = sq().prepare_swiglu(d, K, n=2, m=4, fmt=0)
    torch.cuda.synchronize()
    o = oracle.prepare_swiglu(np.ascontiguousarray(gu[:, 64:64 + 2 * K]), K, 2, 4, 0, trace=True)
    assert compare_prepared(prepared_to_host(p), o, 2, 4, "slice")["mismatched"] == 0


def test_prep_swiglu_zero_rows_is_noop():
    p = sq().prepare_swiglu(torch.zeros((0, 512), dtype=torch.float32, device="cuda"), 256, fmt=1)
    assert p.b_codes.numel() == 0


# ---------------------------------------------------------------- weight quantization

@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape", [(1, 48, 256), (3, 40, 640), (1, 257, 4096)])
def test_quantize_weight(fmt, shape):
    E, nout, K = shape
    w = synth.small_weight(nout, K, experts=E, tag=E * 7 + K)
    q = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    torch.cuda.synchronize()
    o = oracle.quantize_weight(w, "bf16", fmt)
    codes, scales = weight_to_host(q)
    assert np.array_equal(codes, o.codes)
    assert np.array_equal(scales, o.scales)
    if fmt == 1:
        assert np.array_equal(host(q.global_scale), o.gscale)


# ---------------------------------------------------------------- layer product

def ref_linear(pg, qw, row_index=None, offsets=None, out_rows=None, expert_of_row=None):
    """Oracle FP64 product of the GPU's own codes (decoded by the oracle)."""
    K, fmt = pg.K, pg.fmt
    G = float(host(pg.global_scale)[0]) if pg.global_scale is not None else 1.0
    gh = prepared_to_host(pg)
    bc, bs, rc, rs = gh["b_codes"], gh["b_scales"], gh["r_codes"], gh["r_scales"]
    wc, ws = weight_to_host(qw)
    wG = host(qw.global_scale) if qw.global_scale is not None else np.ones(qw.E, np.float32)
    rows = np.arange(pg.T if row_index is None and offsets is None else
                     (len(row_index) if row_index is not None else int(offsets[-1])))
    if out_rows is not None:
        rows = np.asarray(out_rows)
    src = rows if row_index is None else row_index[rows]
    if offsets is None:
        ex = np.zeros(len(rows), np.int64)
    else:
        ex = np.searchsorted(offsets, rows, side="right") - 1
    y = np.zeros((len(rows), qw.nout))
    absum = np.zeros((len(rows), qw.nout))
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        a = oracle.dequant(bc[src[sel]], bs[src[sel]], K, fmt, G) + 0.0
        r = oracle.dequant(rc[src[sel]], rs[src[sel]], K, fmt, G)
        w = oracle.dequant(wc[e], ws[e], K, fmt, float(wG[e]))
        y[sel] = a @ w.T + r @ w.T
        absum[sel] = np.abs(a) @ np.abs(w).T + np.abs(r) @ np.abs(w).T
    ref_linear.absum = absum
    return rows, y


def check_product(y: np.ndarray, ref: np.ndarray, K: int, what=""):
    """Product parity: relative Frobenius error <= 1e-3 against the FP64
    product of the same dequantized codes, and every element within the
    FP32 accumulation bound 2*K*2^-24 * sum_k(|b_k w_k| + |r_k w_k|) (the FP4
    products are exact; only the FP32 sums round)."""
    err = rel_fro(y, ref)
    assert err <= TOL, (what, err)
    bound = 2.0 * K * 2.0 ** -24 * ref_linear.absum
    diff = np.abs(y.astype(np.float64) - ref)
    bad = diff > bound
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:5], float((diff - bound).max()))
    return err


def fragment_rows(T: int, rng, frag: int = 32) -> np.ndarray:
    """One random row from every 32-row fragment (every row tile of every
    tile shape), plus the last row."""
    starts = np.arange(0, T, frag)
    rows = np.minimum(starts + rng.integers(0, frag, starts.size), T - 1)
    return np.unique(np.concatenate([rows, [T - 1]]))


LINEAR_CASES = [
    # (fmt, T, K, nout)
    (0, 16, 256, 256), (0, 300, 640, 272), (0, 513, 1024, 520), (0, 1, 512, 64), (0, 5, 768, 48),
    (0, 17, 1280, 100), (0, 64, 4096, 256), (0, 65, 384, 1000), (0, 2, 14336, 64),
    (0, 3, 8320, 40), (0, 48, 4480, 1000),  # small batch: 17 / 9 K chunks over the workgroup's 8 waves
    (0, 2048, 256, 16384),  # 256x256 tiles, two rounds in XCD bands of two row tiles (4 bands)
    (0, 1000, 128, 33000),  # two full rounds in 2 bands (ragged last row tile), remaining columns split off
    (0, 1000, 384, 12200),  # 256x192 tiles (one full round), ragged rows and columns
    (0, 300, 128, 200), (0, 5, 128, 40), (1, 130, 128, 96),  # K = 128: a single stage / chunk
    (0, 64, 1024, 2128), (0, 40, 1024, 3000), (0, 9, 1024, 8240),  # few rows as 64x64 tiles
    (0, 64, 14336, 2050), (0, 24, 14336, 3000), (0, 17, 14336, 4096),  # few rows over 8 / 8 / 4 K ranges, summed
    (1, 16, 256, 256), (1, 300, 640, 272), (1, 1, 512, 64), (1, 70, 1024, 130), (1, 257, 3584, 256),
    (1, 2049, 256, 4224),  # NVFP4 256x224 tiles (64x224 per wave), ragged rows and columns
    (1, 4001, 256, 3500),  # NVFP4 256x224 tiles filling a round, ragged rows and columns
    (1, 4000, 256, 4090),  # NVFP4 256x256 tiles (128x128 per wave), ragged rows and columns
    (1, 2049, 256, 8616),  # NVFP4 column split: 256x256 tiles for full rounds, 64x128 for the rest
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "fmt%d-T%d-K%d-N%d" % c)
def test_linear(case):
    fmt, T, K, nout = case
    x = synth.small_case(K, T, "bf16", outliers=3, mult=40.0, tag=T + K)
    g = synth.small_gamma(K, "bf16", tag=T)
    pg = gpu_prepare(x, "bf16", K, 1, g, None, 1e-5, 2, 4, fmt)
    w = synth.small_weight(nout, K, tag=nout + K)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    y = host(sq().linear(pg, qw))
    _, ref = ref_linear(pg, qw)
    check_product(y, ref, K, case)
    # and against the oracle end to end (its own prep and weight)
    o = oracle.prepare(x, "bf16", K, 1, g, None, 1e-5, 2, 4, fmt)
    ow = oracle.quantize_weight(w, "bf16", fmt)
    assert rel_fro(y, oracle.linear(o, ow)) <= TOL


OUT_DTYPE_CASES = [
    # (fmt, T, K, nout, grouped): one case per dispatch path
    (0, 300, 640, 272, False),     # prefill tiles
    (0, 2048, 256, 16384, False),  # 256x256 tiles
    (0, 5, 768, 48, False),        # small-batch kernel
    (0, 40, 1024, 3000, False),    # few rows as 64x64 tiles
    (0, 24, 14336, 3000, False),   # few rows over K ranges, summed in the output type
    (1, 300, 640, 272, False),     # NVFP4 (tensor scales applied before rounding)
    (0, 90, 640, 96, True),        # grouped, gathered rows
    (1, 90, 640, 96, True),
]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("case", OUT_DTYPE_CASES, ids=lambda c: "fmt%d-T%d-K%d-N%d-g%d" % c)
def test_linear_output_dtype(case, out_dtype):
    """Y stored as BF16 / F16: the FP32 accumulator rounded to nearest even.
    Bit-equal to rounding the library's own FP32 output (same accumulation
    order), and within one unit in the last place of the output type of the
    FP64 product of the same codes."""
    fmt, T, K, nout, grouped = case
    x = synth.small_case(K, T, "bf16", outliers=3, tag=81 + T)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, fmt)
    E = 5 if grouped else 1
    w = synth.small_weight(nout, K, experts=E, tag=82 + nout)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    kw = {}
    row_index = offsets = None
    if grouped:
        offsets = np.array([0, 130, 130, 141, 400, 401], np.int32)
        row_index = np.random.default_rng(83).integers(0, T, offsets[-1]).astype(np.int32)
        kw = dict(group_offsets=torch.from_numpy(offsets).cuda(), row_index=torch.from_numpy(row_index).cuda(),
                  rows=int(offsets[-1]))
    y32 = sq().linear(pg, qw, **kw)
    y16 = sq().linear(pg, qw, out_dtype=out_dtype, **kw)
    assert y16.dtype == out_dtype
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16).cpu(), y32.to(out_dtype).view(torch.int16).cpu())
    _, ref = ref_linear(pg, qw, row_index=row_index, offsets=offsets)
    got = y16.double().cpu().numpy()
    rr16 = torch.from_numpy(ref).to(out_dtype)                       # FP64 product rounded once
    mag = rr16.abs()
    above = (mag.view(torch.int16).to(torch.int32) + 1).to(torch.int16).view(out_dtype)
    ulp = (above.double() - mag.double()).numpy()                    # spacing above |rr| in the type
    diff = np.abs(got - rr16.double().numpy())
    assert np.all(diff <= ulp), (case, int((diff > ulp).sum()))


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_weight_strided_rows(fmt):
    """A weight that is a column slice of a wider matrix (row stride ldw > K):
    the payload equals the oracle's on the slice."""
    E, nout, K, ld = 2, 40, 512, 768
    wide = synth.small_weight(nout, ld, experts=E, tag=84 + fmt)
    wd = dev16(wide, "bf16")
    q = sq().quantize_weight(wd[:, :, 128:128 + K], fmt=fmt)
    torch.cuda.synchronize()
    o = oracle.quantize_weight(np.ascontiguousarray(wide[:, :, 128:128 + K]), "bf16", fmt)
    codes, scales = weight_to_host(q)
    assert np.array_equal(codes, o.codes)
    assert np.array_equal(scales, o.scales)
    if fmt == 1:
        assert np.array_equal(host(q.global_scale), o.gscale)


GATHER_CASES = [
    # (fmt, T, K, nout, rows): one weight, output rows gathered through row_index
    (0, 50, 1024, 64, 40),     # small-batch kernel
    (0, 50, 1024, 3000, 40),   # few rows as 64x64 tiles
    (0, 70, 14336, 2050, 40),  # few rows over K ranges, summed
    (0, 90, 640, 272, 300),    # prefill tiles, rows repeated
    (1, 90, 640, 272, 300),
    (1, 30, 512, 128, 7),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=lambda c: "fmt%d-T%d-K%d-N%d-rows%d" % c)
def test_linear_dense_gather(case):
    """A single weight with gathered token rows (no expert groups): output row
    m is the product of prepared row row_index[m], on every dispatch path."""
    fmt, T, K, nout, rows = case
    x = synth.small_case(K, T, "bf16", outliers=3, tag=7 + rows)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, fmt)
    w = synth.small_weight(nout, K, tag=8 + nout)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    row_index = np.random.default_rng(rows).integers(0, T, rows).astype(np.int32)
    y = host(sq().linear(pg, qw, row_index=torch.from_numpy(row_index).cuda(), rows=rows))
    _, ref = ref_linear(pg, qw, row_index=row_index)
    assert y.shape == (rows, nout)
    check_product(y, ref, K, case)


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_grouped(fmt):
    K, nout, E, T = 640, 96, 5, 90
    x = synth.small_case(K, T, "bf16", outliers=3, tag=5)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, fmt)
    w = synth.small_weight(nout, K, experts=E, tag=6)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    offsets = np.array([0, 130, 130, 141, 400, 401], np.int32)   # an empty expert, ragged sizes
    rng = np.random.default_rng(3)
    row_index = rng.integers(0, T, offsets[-1]).astype(np.int32)
    y = host(sq().linear(pg, qw, group_offsets=torch.from_numpy(offsets).cuda(),
                         row_index=torch.from_numpy(row_index).cuda(), rows=int(offsets[-1])))
    _, ref = ref_linear(pg, qw, row_index=row_index, offsets=offsets)
    check_product(y, ref, K, "grouped gathered")
    # contiguous grouped rows, no gather
    pg2 = gpu_prepare(synth.small_case(K, 401, "bf16", tag=9), "bf16", K, 0, None, None, 0.0, 2, 4, fmt)
    y2 = host(sq().linear(pg2, qw, group_offsets=torch.from_numpy(offsets).cuda(), rows=401))
    _, ref2 = ref_linear(pg2, qw, offsets=offsets)
    check_product(y2, ref2, K, "grouped contiguous")


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_grouped_many_experts(fmt):
    """More experts than one wave has lanes (the tile lookup takes two
    passes), empty experts first, last and in between, gathered rows."""
    K, nout, E, T = 256, 64, 80, 120
    x = synth.small_case(K, T, "bf16", outliers=2, tag=41)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, fmt)
    w = synth.small_weight(nout, K, experts=E, tag=42)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    rng = np.random.default_rng(43)
    counts = rng.integers(0, 19, E)
    counts[[0, 1, 37, 63, 64, E - 1]] = 0
    counts[65] = 300  # one expert with several row tiles, right after the first pass
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_index = rng.integers(0, T, offsets[-1]).astype(np.int32)
    y = host(sq().linear(pg, qw, group_offsets=torch.from_numpy(offsets).cuda(),
                         row_index=torch.from_numpy(row_index).cuda(), rows=int(offsets[-1])))
    _, ref = ref_linear(pg, qw, row_index=row_index, offsets=offsets)
    check_product(y, ref, K, "many experts")


def test_linear_grouped_ragged_experts():
    """Persistent grouped MXFP4 product (16 experts or more, workgroups
    walking their XCD's expert tiles) over ragged experts: 260 rows (three
    128-row tiles, the last holding 4 rows), 129, 65, 33, 32, 31, 1 and 0
    rows, gathered rows."""
    K, nout, E, T = 384, 320, 24, 200
    x = synth.small_case(K, T, "bf16", outliers=2, tag=51)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, 0)
    w = synth.small_weight(nout, K, experts=E, tag=52)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0)
    rng = np.random.default_rng(53)
    counts = rng.integers(0, 40, E)
    counts[[2, 5, 9, 11, 16, 17, 20, 23]] = [260, 129, 65, 33, 32, 31, 1, 0]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_index = rng.integers(0, T, offsets[-1]).astype(np.int32)
    y = host(sq().linear(pg, qw, group_offsets=torch.from_numpy(offsets).cuda(),
                         row_index=torch.from_numpy(row_index).cuda(), rows=int(offsets[-1])))
    _, ref = ref_linear(pg, qw, row_index=row_index, offsets=offsets)
    check_product(y, ref, K, "ragged experts")


@pytest.mark.parametrize("T", [4, 300], ids=["short", "tiled"])
def test_nvfp4_every_block_scale(T):
    """NVFP4 product where the 16-element blocks take every finite E4M3
    block scale (subnormal ones included) and a one-hot weight picks one
    element per block: every output is a single exact product, so the GPU
    must match the oracle's decoding of the same codes and scales exactly."""
    K, nout = 2048, 128
    e4m3 = np.array([oracle.e4m3_decode(c) for c in range(127)], np.float64)
    x = np.zeros((T, K), np.float32)
    for t in range(T):
        codes = 1 + (np.arange(K // 16) + 7 * t) % 126          # 1..126: all finite non-zero scales
        x[t, ::16] = (6.0 * e4m3[codes]).astype(np.float32)      # block amax = 6 * scale, code 6
        x[t, 16 * (t % (K // 16))] = 2688.0                        # tensor amax: G = 1
    w = np.zeros((nout, K), np.float32)
    w[np.arange(nout), 16 * np.arange(nout)] = 2688.0            # weight tensor scale 1, code 6 x 448
    xb, wb = synth.to_bits(x, "bf16"), synth.to_bits(w, "bf16")
    pg = gpu_prepare(xb, "bf16", K, 0, None, None, 0.0, 2, 4, 1)
    assert float(host(pg.global_scale)[0]) == 1.0
    qw = sq().quantize_weight(dev16(wb, "bf16"), fmt=1)
    y = host(sq().linear(pg, qw))
    _, ref = ref_linear(pg, qw)
    assert np.array_equal(y, ref.astype(np.float32))
    assert float(host(qw.global_scale)[0]) == 1.0
    assert np.array_equal(y, x[:, ::16][:, :nout] * np.float32(2688.0))


@pytest.mark.parametrize("T", [300, 5], ids=["tiled", "small"])
def test_linear_strided_unaligned_output(T):
    """Y written into a column window of a wider buffer, 12 bytes past a
    16-byte boundary (scalar stores); the columns around it stay untouched."""
    K, nout = 512, 72
    x = synth.small_case(K, T, "bf16", tag=51)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, 0)
    w = synth.small_weight(nout, K, tag=52)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0)
    buf = torch.full((T, nout + 13), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[:, 3:3 + nout]
    sq().linear(pg, qw, out=out)
    torch.cuda.synchronize()
    full = host(buf)
    _, ref = ref_linear(pg, qw)
    check_product(full[:, 3:3 + nout], ref, K, "strided")
    assert np.isnan(full[:, :3]).all() and np.isnan(full[:, 3 + nout:]).all()
    dense = host(sq().linear(pg, qw))
    assert np.array_equal(full[:, 3:3 + nout], dense)


def test_determinism():
    K, T, nout = 4096, 512, 512
    x = synth.small_case(K, T, "bf16", tag=21)
    g = synth.small_gamma(K, "bf16", tag=21)
    w = synth.small_weight(nout, K, tag=21)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0)
    outs = []
    for _ in range(2):
        pg = gpu_prepare(x, "bf16", K, 1, g, None, 1e-5, 2, 4, 0)
        outs.append((prepared_to_host(pg), host(sq().linear(pg, qw))))
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
        assert np.array_equal(outs[0][0][key], outs[1][0][key])
    assert np.array_equal(outs[0][1], outs[1][1])


def _check_graph_replays(step, out, y):
    """Run step eagerly, capture it in one HIP graph, then replay the graph
    three times with eager work and synchronizations in between; every
    replay must reproduce the eager prepared tensors and product bit for bit
    (every sum is taken in a fixed order)."""
    step()
    torch.cuda.synchronize()
    ref_p, ref_y = prepared_to_host(out), host(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        y.fill_(float("nan"))
        out.b_codes.zero_()
        out.r_scales.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = prepared_to_host(out)
        for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales", "G"):
            assert np.array_equal(got[key], ref_p[key]), (rep, key)
        assert np.array_equal(host(y), ref_y), rep
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,T", [(0, 8), (1, 8), (0, 300), (1, 300)],
                         ids=["mx-decode8", "nv-decode8", "mx-T300", "nv-T300"])
def test_graph_replay_matches_eager(fmt, T):
    """The whole path (normalized prep + product) captured in one HIP graph."""
    K, nout = 2048, 384
    w = synth.small_weight(nout, K, tag=31 + fmt)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=fmt)
    x = dev16(synth.small_case(K, T, "bf16", tag=32 + fmt), "bf16")
    g = dev16(synth.small_gamma(K, "bf16", tag=33), "bf16")
    out = sq().alloc_prepared(T, K, fmt, x.device)
    y = torch.empty((T, nout), dtype=torch.float32, device="cuda")

    def step():
        sq().prepare(x, norm=1, gamma=g, eps=1e-5, n=2, m=4, fmt=fmt, out=out)
        sq().linear(out, qw, out=y)

    _check_graph_replays(step, out, y)


def test_graph_replay_k_split_matches_eager():
    """A few-row product that runs over K ranges (partial products in a
    workspace allocated during capture, then summed) captured in one graph."""
    K, nout, T = 14336, 3000, 24
    w = synth.small_weight(nout, K, tag=37)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0)
    assert sq().lib().sharq_linear_workspace_size(T, K, nout, 1, 0) > 0   # this shape takes the K split
    x = dev16(synth.small_case(K, T, "bf16", tag=38), "bf16")
    out = sq().alloc_prepared(T, K, 0, x.device)
    y = torch.empty((T, nout), dtype=torch.float32, device="cuda")

    def step():
        sq().prepare(x, norm=0, n=2, m=4, fmt=0, out=out)
        sq().linear(out, qw, out=y)

    _check_graph_replays(step, out, y)


def test_graph_replay_grouped_matches_eager():
    """A grouped expert product over gathered rows, after a prep without a
    norm, captured in one HIP graph."""
    K, nout, E, T = 768, 256, 6, 200
    w = synth.small_weight(nout, K, experts=E, tag=34)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0)
    x = dev16(synth.small_case(K, T, "bf16", tag=35), "bf16")
    rng = np.random.default_rng(36)
    counts = rng.integers(0, 160, E)
    counts[2] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    offs = torch.from_numpy(offsets).cuda()
    ridx = torch.from_numpy(rng.integers(0, T, rows).astype(np.int32)).cuda()
    out = sq().alloc_prepared(T, K, 0, x.device)
    y = torch.empty((rows, nout), dtype=torch.float32, device="cuda")

    def step():
        sq().prepare(x, norm=0, n=2, m=4, fmt=0, out=out)
        sq().linear(out, qw, group_offsets=offs, row_index=ridx, rows=rows, out=y)

    _check_graph_replays(step, out, y)


@pytest.mark.parametrize("grouped", [False, True], ids=["dense", "grouped"])
def test_graph_replay_swiglu_matches_eager(grouped):
    """The MLP half of a layer as the benchmark runs it -- gate_up prep, the
    gate_up product with the down projection's preparation in its epilogue,
    the down product -- captured in one HIP graph."""
    K, nout, T = 512, 768, 300
    E = 20 if grouped else 1
    w = synth.small_weight(nout, K, experts=E, tag=37)
    qgu = sq().quantize_weight(dev16(w, "bf16"), fmt=0, gate_up=True)
    qd = sq().quantize_weight(dev16(synth.small_weight(K, nout // 2, experts=E, tag=38), "bf16"), fmt=0)
    x = dev16(synth.small_case(K, T, "bf16", tag=39), "bf16")
    g = dev16(synth.small_gamma(K, tag=40), "bf16")
    offs = ridx = None
    rows = T
    if grouped:
        rng = np.random.default_rng(41)
        counts = rng.integers(0, 60, E)
        counts[3] = 0
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        rows = int(offsets[-1])
        offs = torch.from_numpy(offsets).cuda()
        ridx = torch.from_numpy(rng.integers(0, T, rows).astype(np.int32)).cuda()
    p = sq().alloc_prepared(T, K, 0, x.device)
    pd = sq().alloc_prepared(rows, nout // 2, 0, x.device)
    y = torch.empty((rows, K), dtype=torch.float32, device="cuda")

    def step():
        sq().prepare(x, norm=1, gamma=g, eps=1e-5, n=2, m=4, fmt=0, out=p)
        sq().linear_swiglu(p, qgu, n=2, m=4, group_offsets=offs, row_index=ridx, rows=rows, out=pd)
        sq().linear(pd, qd, group_offsets=offs, rows=rows, out=y)

    _check_graph_replays(step, pd, y)


# ---------------------------------------------------------------- full-size workloads

def _weight_sample_check(wl, lin, qw, w_bits, nrows=128, seed=0):
    rng = np.random.default_rng(seed)
    E = qw.E
    codes, scales = weight_to_host(qw)
    for e in sorted(set([0, E - 1])):
        rows = np.sort(rng.choice(qw.nout, size=min(nrows, qw.nout), replace=False))
        G = 1.0
        if wl.fmt == oracle.FMT_NVFP4:
            amax = float(np.abs(synth.bits_to_f32(w_bits[e], wl.dtype)).max())
            G = oracle.nv_global_scale(amax)
            assert host(qw.global_scale)[e] == np.float32(G)
        c, s = oracle.quantize_rows(w_bits[e][rows], wl.dtype, wl.fmt, G)
        assert np.array_equal(codes[e][rows], c), (lin.name, e)
        assert np.array_equal(scales[e][rows], s), (lin.name, e)


def _run_layer(wl, lin, tokens, prep_rows=None, out_rows=64, seed=0):
    x = synth.activation(wl, lin, tokens)
    g = synth.gamma(wl, lin) if lin.norm else None
    p, gh, o, stats = check_prep(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt,
                                 rows=prep_rows, what=f"{wl.name}/{lin.name}/T{tokens}")
    assert stats["mismatched"] <= 1e-5 * stats["elements"]
    w = synth.weight(wl, lin)
    qw = sq().quantize_weight(dev16(w, wl.dtype), fmt=wl.fmt)
    torch.cuda.synchronize()
    _weight_sample_check(wl, lin, qw, w)
    y = host(sq().linear(p, qw))
    rng = np.random.default_rng(seed)
    rows = np.arange(tokens) if tokens <= out_rows else fragment_rows(tokens, rng)
    rows, ref = ref_linear(p, qw, out_rows=rows)
    err = check_product(y[rows], ref, lin.k, f"{wl.name}/{lin.name}")
    print(f"{wl.name}/{lin.name} T={tokens}: prep mismatches {stats['mismatched']} "
          f"of {stats['elements']}, GEMM rel err {err:.2e} on {rows.size} rows", flush=True)
    return err


def _linear(wl, name):
    return next(L for L in wl.linears if L.name == name)


# Every linear of the layer on a drawn input (down too: the prep without norm
# on a bf16 activation); the fused SiLU(gate)*up path of the layer step is
# checked separately below.
@pytest.mark.parametrize("name", ["qkv", "o_proj", "gate_up", "down"])
def test_llama8b_prefill_full(name):
    wl = synth.WORKLOADS[1]
    _run_layer(wl, _linear(wl, name), wl.tokens)


@pytest.mark.parametrize("tokens", synth.DECODE_TOKENS)
@pytest.mark.parametrize("name", ["qkv", "o_proj", "gate_up", "down"])
def test_llama8b_decode_full(name, tokens):
    wl = synth.WORKLOADS[2]
    _run_layer(wl, _linear(wl, name), tokens)


@pytest.mark.parametrize("name", ["qkv", "o_proj", "gate_up", "down"])
def test_qwen25_7b_nvfp4_full(name):
    wl = synth.WORKLOADS[3]
    rng = np.random.default_rng(len(name))
    rows = np.unique(np.concatenate([[0, wl.tokens - 1], rng.choice(wl.tokens, 254, replace=False)]))
    _run_layer(wl, _linear(wl, name), wl.tokens, prep_rows=rows)


def _run_fused_down(wl, tokens, seed=0):
    """The layer step's MLP half as the benchmark runs it: gate_up prep and
    product on the GPU, then the down projection prepared straight from
    gate_up's FP32 output (SiLU(gate) * up inside the prep kernel) and
    multiplied.  The oracle prepares the same FP32 rows (sampled rows; the
    NVFP4 tensor scale over all rows) and multiplies the GPU's codes."""
    gu_lin, down = _linear(wl, "gate_up"), _linear(wl, "down")
    assert down.swiglu_of == "gate_up" and gu_lin.nout == 2 * down.k
    x = synth.activation(wl, gu_lin, tokens)
    g = synth.gamma(wl, gu_lin)
    pg = gpu_prepare(x, wl.dtype, gu_lin.k, gu_lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
    qgu = sq().quantize_weight(dev16(synth.weight(wl, gu_lin), wl.dtype), fmt=wl.fmt)
    ygu = sq().linear(pg, qgu)
    pd = sq().prepare_swiglu(ygu, down.k, n=wl.n, m=wl.m, fmt=wl.fmt)
    torch.cuda.synchronize()
    gu_host = host(ygu)
    rng = np.random.default_rng(seed)
    rows = np.arange(tokens) if tokens <= 64 else np.unique(np.concatenate(
        [fragment_rows(tokens, rng), rng.choice(tokens, 192, replace=False)]))
    o = oracle.prepare_swiglu(gu_host, down.k, wl.n, wl.m, wl.fmt, rows=rows, trace=True)
    gh = prepared_to_host(pd)
    gh = {k: (v[rows] if isinstance(v, np.ndarray) else v) for k, v in gh.items()}
    stats = compare_prepared(gh, o, wl.n, wl.m, f"{wl.name}/down fused T{tokens}")
    assert stats["mismatched"] == 0, stats
    if wl.fmt == oracle.FMT_NVFP4:
        assert gh["G"] == o.G
    qd = sq().quantize_weight(dev16(synth.weight(wl, down), wl.dtype), fmt=wl.fmt)
    y = host(sq().linear(pd, qd))
    out_rows = np.arange(tokens) if tokens <= 64 else fragment_rows(tokens, rng)
    out_rows, ref = ref_linear(pd, qd, out_rows=out_rows)
    err = check_product(y[out_rows], ref, down.k, f"{wl.name}/down fused")
    print(f"{wl.name}/down fused T={tokens}: prep rows {rows.size} bit-exact, GEMM rel err {err:.2e}", flush=True)


def test_llama8b_prefill_fused_down():
    wl = synth.WORKLOADS[1]
    _run_fused_down(wl, wl.tokens)


@pytest.mark.parametrize("tokens", synth.DECODE_TOKENS)
def test_llama8b_decode_fused_down(tokens):
    _run_fused_down(synth.WORKLOADS[2], tokens)


def test_qwen25_7b_nvfp4_fused_down():
    wl = synth.WORKLOADS[3]
    _run_fused_down(wl, wl.tokens)


def test_single_linear_c0():
    wl = synth.WORKLOADS[0]
    _run_layer(wl, wl.linears[0], wl.tokens)


def test_qwen3_moe_full():
    wl = synth.WORKLOADS[4]
    route = synth.moe_routing(wl)
    offs = torch.from_numpy(route.offsets).cuda()
    ridx = torch.from_numpy(route.row_index).cuda()
    nrows = int(route.offsets[-1])
    rng = np.random.default_rng(4)
    # one row from every 32-row fragment of the sorted rows, and each expert's first and last row
    nonempty = np.nonzero(np.diff(route.offsets))[0]
    sample = np.unique(np.concatenate([fragment_rows(nrows, rng), route.offsets[nonempty],
                                       route.offsets[nonempty + 1] - 1]))
    # gate_up: RMSNorm on the unique tokens, grouped product gathers rows
    lin = wl.linears[0]
    x = synth.activation(wl, lin, wl.tokens)
    g = synth.gamma(wl, lin)
    p, gh, o, stats = check_prep(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt,
                                 what="moe gate_up")
    w = synth.weight(wl, lin)
    qw = sq().quantize_weight(dev16(w, wl.dtype), fmt=wl.fmt)
    _weight_sample_check(wl, lin, qw, w, nrows=32)
    y = host(sq().linear(p, qw, group_offsets=offs, row_index=ridx, rows=nrows))
    _, ref = ref_linear(p, qw, row_index=route.row_index, offsets=route.offsets, out_rows=sample)
    err = check_product(y[sample], ref, lin.k, "moe gate_up")
    print(f"moe gate_up rel err {err:.2e} on {sample.size} rows", flush=True)
    # down: rows already sorted by expert, no norm
    lin = wl.linears[1]
    x = synth.activation(wl, lin, nrows)
    rows = np.unique(np.concatenate([[0, nrows - 1], rng.choice(nrows, 510, replace=False)]))
    p, gh, o, stats = check_prep(x, wl.dtype, lin.k, lin.norm, None, None, wl.eps, wl.n, wl.m, wl.fmt,
                                 rows=rows, what="moe down")
    w = synth.weight(wl, lin)
    qw = sq().quantize_weight(dev16(w, wl.dtype), fmt=wl.fmt)
    _weight_sample_check(wl, lin, qw, w, nrows=32)
    y = host(sq().linear(p, qw, group_offsets=offs, rows=nrows))
    _, ref = ref_linear(p, qw, offsets=route.offsets, out_rows=sample)
    err = check_product(y[sample], ref, lin.k, "moe down")
    print(f"moe down rel err {err:.2e} on {sample.size} rows", flush=True)


# ---------------------------------------------------------------- SwiGLU epilogue (sharq_linear_swiglu)

def gate_up_source_rows(nout: int) -> np.ndarray:
    """Source row (of the stacked [gate; up] weight) of every payload row of
    sharq_quantize_weight_gate_up: payload row 64p + c is gate row 32p + c,
    payload row 64p + 32 + c is up row 32p + c."""
    r = np.arange(nout)
    p, c = r // 64, r % 64
    return np.where(c < 32, 32 * p + c, nout // 2 + 32 * p + c - 32)


def deinterleave(y: np.ndarray) -> np.ndarray:
    """Columns of a product in payload order -> [gate | up] rows."""
    out = np.empty_like(y)
    out[:, gate_up_source_rows(y.shape[1])] = y
    return out


def test_quantize_weight_gate_up():
    """The interleaved payload equals the oracle's RTN of the reordered rows."""
    K, nout, E = 384, 320, 3
    w = synth.small_weight(nout, K, experts=E, tag=71)
    q = sq().quantize_weight(dev16(w, "bf16"), fmt=0, gate_up=True)
    torch.cuda.synchronize()
    wc, ws = weight_to_host(q)
    src = gate_up_source_rows(nout)
    for e in range(E):
        o = oracle.quantize_weight(np.ascontiguousarray(w[e][src]), "bf16", 0)
        assert np.array_equal(wc[e], o.codes[0]) and np.array_equal(ws[e], o.scales[0]), e


def _check_swiglu(pg, qw, n, m, what, row_index=None, offsets=None, rows=None, out_rows=None):
    """linear_swiglu against (1) the oracle's FP64 product of the same codes
    (its optional FP32 product output, within the FP32 accumulation bound)
    and (2) the oracle's SiLU(gate) * up preparation of that FP32 product
    (bit-exact); the prepared output without the product output, and the
    library's own two-kernel chain (product, then sharq_prepare_swiglu), must
    give identical bytes."""
    ri = None if row_index is None else torch.from_numpy(row_index).cuda()
    go = None if offsets is None else torch.from_numpy(offsets).cuda()
    if rows is None:
        rows = len(row_index) if row_index is not None else (int(offsets[-1]) if offsets is not None else pg.T)
    y = torch.full((rows, qw.nout), float("nan"), dtype=torch.float32, device="cuda")
    pd = sq().linear_swiglu(pg, qw, n=n, m=m, group_offsets=go, row_index=ri, rows=rows, y=y)
    pd2 = sq().linear_swiglu(pg, qw, n=n, m=m, group_offsets=go, row_index=ri, rows=rows)
    chain = sq().prepare_swiglu(torch.from_numpy(deinterleave(host(y))).cuda(), qw.nout // 2, n=n, m=m, fmt=0)
    torch.cuda.synchronize()
    yh = host(y)
    sel, ref = ref_linear(pg, qw, row_index=row_index, offsets=offsets, out_rows=out_rows)
    err = check_product(yh[sel], ref, pg.K, what)
    gh = prepared_to_host(pd)
    for other in (pd2, chain):
        oh = prepared_to_host(other)
        for k in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
            assert np.array_equal(gh[k], oh[k]), (what, k)
    gu = deinterleave(yh[sel])
    o = oracle.prepare_swiglu(gu, qw.nout // 2, n, m, 0, trace=True)
    gh = {k: (v[sel] if isinstance(v, np.ndarray) else v) for k, v in gh.items()}
    stats = compare_prepared(gh, o, n, m, what)
    assert stats["mismatched"] == 0, (what, stats)
    return err


SWIGLU_LINEAR_CASES = [
    # (T, K, nout, n, m): tile shapes 256x256, 128x256, 128x128, the column
    # split, ragged rows, every in-lane mask width
    (300, 640, 512, 2, 4), (513, 1024, 768, 2, 4), (1, 256, 256, 2, 4), (64, 384, 1280, 1, 4),
    (257, 512, 2304, 2, 2), (130, 256, 512, 1, 1), (96, 256, 512, 4, 4), (2049, 256, 8448, 2, 4),
    (40, 256, 512, 0, 4), (4096, 128, 1024, 3, 4),
    (2100, 128, 16384, 2, 4),  # two or more rounds of 128x256 tiles at two workgroups per CU, ragged rows
    (1024, 128, 32768, 2, 4),  # the same tiles in two XCD bands of 512 token rows
]


@pytest.mark.parametrize("case", SWIGLU_LINEAR_CASES, ids=[str(c) for c in SWIGLU_LINEAR_CASES])
def test_linear_swiglu(case):
    T, K, nout, n, m = case
    tag = SWIGLU_LINEAR_CASES.index(case)
    x = synth.small_case(K, T, "bf16", outliers=3, tag=700 + tag)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, 0)
    w = synth.small_weight(nout, K, tag=800 + tag)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0, gate_up=True)
    out_rows = None if T <= 600 else fragment_rows(T, np.random.default_rng(tag))
    _check_swiglu(pg, qw, n, m, str(case), out_rows=out_rows)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 2)])
def test_linear_swiglu_large_gates(n, m):
    """Gate values far outside [-80, 80] in part of the tile (weights scaled
    by 2^9, products of a few hundred): waves whose gates all lie inside that
    range and waves that take the general SiLU sequence in one launch."""
    T, K, nout = 300, 512, 1024
    x = synth.small_case(K, T, "bf16", outliers=3, tag=95)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, 0)
    wf = synth.bits_to_f32(synth.small_weight(nout, K, tag=96), "bf16")
    wf[:, : nout // 4] *= 512.0  # gate rows of the first half of the hidden columns
    qw = sq().quantize_weight(dev16(synth.to_bits(wf, "bf16"), "bf16"), fmt=0, gate_up=True)
    _check_swiglu(pg, qw, n, m, f"large gates {n}:{m}")


@pytest.mark.parametrize("E", [5, 24], ids=["grouped", "persistent"])
def test_linear_swiglu_grouped(E):
    """Expert products over gathered rows (five experts: one workgroup per
    tile; 24: persistent workgroups walking their XCD's experts), ragged and
    empty experts."""
    K, nout, T = 384, 512, 200
    x = synth.small_case(K, T, "bf16", outliers=2, tag=91)
    pg = gpu_prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, 0)
    w = synth.small_weight(nout, K, experts=E, tag=92)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=0, gate_up=True)
    rng = np.random.default_rng(93)
    counts = rng.integers(0, 60, E)
    counts[0], counts[E - 1] = 0, 260
    counts[E // 2] = 129
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_index = rng.integers(0, T, offsets[-1]).astype(np.int32)
    _check_swiglu(pg, qw, 2, 4, f"grouped E={E}", row_index=row_index, offsets=offsets)


def test_llama8b_gate_up_swiglu_full():
    """Llama-3.1-8B gate_up (2048 x 28672 x 4096) with the down projection's
    preparation in its epilogue, in the benchmark's launch configuration;
    product and prepared rows from every 32-row fragment checked."""
    wl = synth.WORKLOADS[1]
    gu_lin, down = _linear(wl, "gate_up"), _linear(wl, "down")
    x = synth.activation(wl, gu_lin, wl.tokens)
    g = synth.gamma(wl, gu_lin)
    pg = gpu_prepare(x, wl.dtype, gu_lin.k, gu_lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
    qw = sq().quantize_weight(dev16(synth.weight(wl, gu_lin), wl.dtype), fmt=wl.fmt, gate_up=True)
    rows = fragment_rows(wl.tokens, np.random.default_rng(5))
    err = _check_swiglu(pg, qw, wl.n, wl.m, "llama gate_up swiglu", out_rows=rows)
    assert qw.nout // 2 == down.k
    print(f"llama gate_up swiglu: rows {rows.size}, GEMM rel err {err:.2e}", flush=True)


def test_qwen3_moe_gate_up_swiglu_full():
    """Qwen3-30B-A3B expert gate_up (32768 gathered rows, 128 experts) with
    the expert down projection's preparation in its epilogue."""
    wl = synth.WORKLOADS[4]
    route = synth.moe_routing(wl)
    nrows = int(route.offsets[-1])
    lin = wl.linears[0]
    x = synth.activation(wl, lin, wl.tokens)
    g = synth.gamma(wl, lin)
    pg = gpu_prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
    qw = sq().quantize_weight(dev16(synth.weight(wl, lin), wl.dtype), fmt=wl.fmt, gate_up=True)
    rng = np.random.default_rng(6)
    nonempty = np.nonzero(np.diff(route.offsets))[0]
    rows = np.unique(np.concatenate([fragment_rows(nrows, rng), route.offsets[nonempty],
                                     route.offsets[nonempty + 1] - 1]))
    err = _check_swiglu(pg, qw, wl.n, wl.m, "moe gate_up swiglu", row_index=route.row_index,
                        offsets=route.offsets, out_rows=rows)
    print(f"moe gate_up swiglu: rows {rows.size}, GEMM rel err {err:.2e}", flush=True)
