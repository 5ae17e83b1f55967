"""GPU parity of NVFP4_SP24: NVFP4 with the backbone stored in the compressed
form of gfx950's 2:4 sparse f16 matrix instruction and multiplied on it
(SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
Inference, Abstract: a sparse FP4 product on the backbone).

The compressed backbone must equal the oracle's NVFP4 backbone re-arranged by
oracle.sp24_pack byte for byte (records and block-scale order); the residual,
mask and tensor scale must equal the oracle's NVFP4 outputs.  Products are
checked against the FP64 product of the oracle's dequantized codes (which the
prep check has just shown equal to the GPU's) with the FP32 accumulation bound
per element and the 1e-3 relative Frobenius bound; they also agree with the
dense NVFP4 product of the same input within that bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import dev16, host, rel_fro, weight_to_host
from sparsity_prep_amd.layout import ktile_to_rows

SP, NV = 2, 1


def sq():
    import sparsity_prep_amd
    sparsity_prep_amd.lib()
    return sparsity_prep_amd


def sp_to_host(p):
    T, K = p.T, p.K
    return {"rec": host(p.b_codes).reshape(K // 128, T, 48).transpose(1, 0, 2),
            "b_scales": ktile_to_rows(host(p.b_scales), T, K, 16),
            "r_codes": ktile_to_rows(host(p.r_codes), T, K, 2),
            "r_scales": ktile_to_rows(host(p.r_scales), T, K, 16),
            "mask": None if p.mask is None else host(p.mask),
            "G": float(host(p.global_scale)[0])}


def check_sp(gh, o, what, rows=None):
    if rows is not None:
        gh = {k: (v[rows] if isinstance(v, np.ndarray) else v) for k, v in gh.items()}
    rec, sc = oracle.sp24_pack(o)
    for key, got, want in (("records", gh["rec"], rec), ("backbone scales", gh["b_scales"], sc),
                           ("residual codes", gh["r_codes"], o.r_codes), ("residual scales", gh["r_scales"], o.r_scales),
                           ("mask", gh["mask"], o.mask)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, (what, key, len(bad), bad[:5])
    assert gh["G"] == o.G, (what, gh["G"], o.G)


def reference(o, qw, rows=None):
    """FP64 product of the oracle's dequantized codes and the GPU weight
    payload, with sum |a w| per element for the accumulation bound."""
    K = o.K
    bc, bs, rc, rs = o.b_codes, o.b_scales, o.r_codes, o.r_scales
    if rows is not None:
        bc, bs, rc, rs = bc[rows], bs[rows], rc[rows], rs[rows]
    a = oracle.dequant(bc, bs, K, NV, o.G)
    r = oracle.dequant(rc, rs, K, NV, o.G)
    wc, ws = weight_to_host(qw)
    w = oracle.dequant(wc[0], ws[0], K, NV, float(host(qw.global_scale)[0]))
    return a @ w.T + r @ w.T, np.abs(a) @ np.abs(w).T + np.abs(r) @ np.abs(w).T


def check_product(y, ref, absum, K, what):
    err = rel_fro(y, ref)
    assert err <= 1e-3, (what, err)
    diff = np.abs(y.astype(np.float64) - ref)
    bad = diff > 2.0 * K * 2.0 ** -24 * absum
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:5])
    return err


PREP_CASES = [
    # (T, K, norm, ldx extra)
    (1, 128, 1, 0), (5, 256, 1, 0), (33, 640, 2, 0), (257, 1024, 0, 0), (300, 3584, 1, 0), (9, 18944, 1, 0),
    (130, 512, 1, 8),  # strided rows
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", PREP_CASES, ids=lambda c: "T%d-K%d-norm%d-pad%d" % c)
def test_prepare_sp24(case):
    T, K, norm, pad = case
    ld = K + pad
    x = synth.small_case(ld, T, "bf16", outliers=3, mult=40.0, tag=T + K)
    g = synth.small_gamma(K, "bf16", tag=K)
    b = synth.small_gamma(K, "bf16", tag=K + 1) if norm == 2 else None
    xd = dev16(x, "bf16")[:, :K]
    p = sq().prepare(xd, norm=norm, gamma=dev16(g, "bf16") if norm else None,
                     beta=dev16(b, "bf16") if b is not None else None, eps=1e-6, n=2, m=4, fmt=SP)
    torch.cuda.synchronize()
    o = oracle.prepare(np.ascontiguousarray(x[:, :K]), "bf16", K, norm, g, b, 1e-6, 2, 4, NV)
    check_sp(sp_to_host(p), o, f"prep T{T} K{K}")
    # the same call through the allocation-free entry point
    p2 = sq().alloc_prepared(T, K, SP, xd.device)
    sq().prepare_noalloc(xd, p2, norm=norm, gamma=dev16(g, "bf16") if norm else None,
                         beta=dev16(b, "bf16") if b is not None else None, eps=1e-6, n=2, m=4)
    torch.cuda.synchronize()
    check_sp(sp_to_host(p2), o, f"noalloc T{T} K{K}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", [(3, 128), (40, 1536), (257, 3584)], ids=lambda c: "T%d-K%d" % c)
def test_prepare_swiglu_sp24(case):
    T, K = case
    gu = synth.small_gate_up(K, T, ld=2 * K + 4, tag=K)
    p = sq().prepare_swiglu(torch.from_numpy(gu).cuda(), K, n=2, m=4, fmt=SP)
    torch.cuda.synchronize()
    o = oracle.prepare_swiglu(gu, K, 2, 4, NV)
    check_sp(sp_to_host(p), o, f"swiglu T{T} K{K}")


def _sp_and_dense(T, K, nout, tag, norm=1):
    x = synth.small_case(K, T, "bf16", outliers=3, mult=40.0, tag=tag)
    g = synth.small_gamma(K, "bf16", tag=tag + 1)
    xd, gd = dev16(x, "bf16"), dev16(g, "bf16")
    psp = sq().prepare(xd, norm=norm, gamma=gd, eps=1e-6, n=2, m=4, fmt=SP)
    pnv = sq().prepare(xd, norm=norm, gamma=gd, eps=1e-6, n=2, m=4, fmt=NV)
    w = synth.small_weight(nout, K, tag=tag + 2)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=SP)
    assert qw.fmt == NV
    torch.cuda.synchronize()
    o = oracle.prepare(x, "bf16", K, norm, g, None, 1e-6, 2, 4, NV)
    check_sp(sp_to_host(psp), o, f"linear prep T{T} K{K}")
    return psp, pnv, qw, o


LINEAR_CASES = [
    # (T, K, nout)
    (16, 256, 256), (300, 640, 272), (1, 512, 64), (70, 1024, 130), (257, 3584, 256), (5, 128, 40),
    (2049, 256, 4224),  # 256x256 tiles, ragged rows and columns
    (2049, 256, 8616),  # column split: 256x256 tiles for full rounds, 128x128 for the rest
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "T%d-K%d-N%d" % c)
def test_linear_sp24(case):
    T, K, nout = case
    psp, pnv, qw, o = _sp_and_dense(T, K, nout, tag=T + nout)
    y = host(sq().linear(psp, qw))
    ydense = host(sq().linear(pnv, qw))
    ref, absum = reference(o, qw)
    check_product(y, ref, absum, K, f"sp T{T} K{K} N{nout}")
    check_product(ydense, ref, absum, K, f"dense T{T} K{K} N{nout}")


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_linear_sp24_16bit_output(dt):
    """16-bit outputs of the transposed epilogue: the FP32 accumulator rounded
    to nearest even, i.e. torch's rounding of the FP32 output of the same
    product, bit for bit."""
    psp, _, qw, _ = _sp_and_dense(300, 640, 272, tag=7)
    y32 = sq().linear(psp, qw)
    y16 = sq().linear(psp, qw, out_dtype=dt)
    assert torch.equal(y32.to(dt), y16)


@pytest.mark.gpu
def test_linear_sp24_grouped():
    """Grouped expert products over gathered rows and over contiguous rows
    (an empty expert, ragged sizes)."""
    K, nout, E, T = 640, 96, 5, 90
    x = synth.small_case(K, T, "bf16", outliers=3, tag=5)
    p = sq().prepare(dev16(x, "bf16"), norm=0, n=2, m=4, fmt=SP)
    o = oracle.prepare(x, "bf16", K, 0, None, None, 0.0, 2, 4, NV)
    w = synth.small_weight(nout, K, experts=E, tag=6)
    qw = sq().quantize_weight(dev16(w, "bf16"), fmt=SP)
    torch.cuda.synchronize()
    check_sp(sp_to_host(p), o, "grouped prep")
    offsets = np.array([0, 130, 130, 141, 400, 401], np.int32)
    rng = np.random.default_rng(3)
    row_index = rng.integers(0, T, offsets[-1]).astype(np.int32)
    y = host(sq().linear(p, qw, group_offsets=torch.from_numpy(offsets).cuda(),
                         row_index=torch.from_numpy(row_index).cuda(), rows=int(offsets[-1])))
    wc, ws = weight_to_host(qw)
    wG = host(qw.global_scale)
    a = oracle.dequant(o.b_codes, o.b_scales, K, NV, o.G)
    r = oracle.dequant(o.r_codes, o.r_scales, K, NV, o.G)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        wd = oracle.dequant(wc[e], ws[e], K, NV, float(wG[e]))
        src = row_index[lo:hi]
        ref = a[src] @ wd.T + r[src] @ wd.T
        absum = np.abs(a[src]) @ np.abs(wd).T + np.abs(r[src]) @ np.abs(wd).T
        check_product(y[lo:hi], ref, absum, K, f"grouped expert {e}")


@pytest.mark.gpu
def test_graph_replay_sp24():
    """Prep and product captured in one HIP graph and replayed three times
    with eager work in between, every replay equal to the eager result."""
    K, nout, T = 2048, 384, 300
    qw = sq().quantize_weight(dev16(synth.small_weight(nout, K, tag=51), "bf16"), fmt=SP)
    x = dev16(synth.small_case(K, T, "bf16", tag=52), "bf16")
    g = dev16(synth.small_gamma(K, "bf16", tag=53), "bf16")
    out = sq().alloc_prepared(T, K, SP, x.device)
    y = torch.empty((T, nout), dtype=torch.float32, device="cuda")

    def step():
        sq().prepare(x, norm=1, gamma=g, eps=1e-6, n=2, m=4, fmt=SP, out=out)
        sq().linear(out, qw, out=y)

    step()
    torch.cuda.synchronize()
    ref_b, ref_y = out.b_codes.clone(), y.clone()
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.b_codes, ref_b), rep
        assert torch.equal(y, ref_y), rep
        step()
        torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["qkv", "gate_up"])
def test_qwen25_7b_sp24_full(name):
    """Full-size Qwen2.5-7B linears (T = 4096) in NVFP4_SP24: sampled rows of
    the prep (the tensor scale over all rows) and of the product, one row
    from every 32-row fragment."""
    wl = synth.WORKLOADS[3]
    lin = next(L for L in wl.linears if L.name == name)
    x = synth.activation(wl, lin, wl.tokens)
    g = synth.gamma(wl, lin)
    p = sq().prepare(dev16(x, wl.dtype), norm=lin.norm, gamma=dev16(g, wl.dtype), eps=wl.eps, n=2, m=4, fmt=SP)
    qw = sq().quantize_weight(dev16(synth.weight(wl, lin), wl.dtype), fmt=SP)
    y = sq().linear(p, qw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(len(name))
    starts = np.arange(0, wl.tokens, 32)
    rows = np.unique(np.concatenate([starts + rng.integers(0, 32, starts.size), [wl.tokens - 1]]))
    o = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, 2, 4, NV, rows=rows)
    check_sp(sp_to_host(p), o, f"qwen {name}", rows=rows)
    ref, absum = reference(o, qw)
    err = check_product(host(y)[rows], ref, absum, lin.k, f"qwen {name}")
    print(f"qwen {name} SP24: {rows.size} rows bit-exact, GEMM rel err {err:.2e}", flush=True)
