"""Check mode (SHARQ_DEBUG=1): every entry point waits for its own launches
and reports their errors, except while its stream is being captured into a
HIP graph.  The results must not change: the MXFP4 and NVFP4 preps and
products give the same bytes with and without the check mode, and the whole
path still captures into a graph and replays with it on."""
import os

import pytest


def _run(sq, torch, fmt):
    g = torch.Generator(device="cpu").manual_seed(3)
    x = torch.randn(96, 512, generator=g).to(torch.bfloat16).cuda()
    gamma = (1 + 0.1 * torch.randn(512, generator=g)).to(torch.bfloat16).cuda()
    w = (0.02 * torch.randn(384, 512, generator=g)).to(torch.bfloat16).cuda()
    wq = sq.quantize_weight(w, fmt=fmt)
    p = sq.prepare(x, norm=sq.NORM_RMS, gamma=gamma, eps=1e-5, n=2, m=4, fmt=fmt)
    y = sq.linear(p, wq)
    torch.cuda.synchronize()
    return p, y, (x, gamma, wq)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [0, 1])
def test_check_mode_keeps_results(monkeypatch, fmt):
    import torch
    import sparsity_prep_amd as sq
    monkeypatch.delenv("SHARQ_DEBUG", raising=False)
    p0, y0, _ = _run(sq, torch, fmt)
    monkeypatch.setenv("SHARQ_DEBUG", "1")
    p1, y1, _ = _run(sq, torch, fmt)
    assert sq.lib().sharq_last_hip_error() == 0
    for a in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
        assert torch.equal(getattr(p0, a), getattr(p1, a)), a
    assert torch.equal(y0, y1)


@pytest.mark.gpu
def test_check_mode_under_graph_capture(monkeypatch):
    import torch
    import sparsity_prep_amd as sq
    monkeypatch.setenv("SHARQ_DEBUG", "1")
    p, y, (x, gamma, wq) = _run(sq, torch, 0)
    out = sq.alloc_prepared(x.shape[0], x.shape[1], 0, x.device)
    yg = torch.empty_like(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            sq.prepare(x, norm=sq.NORM_RMS, gamma=gamma, eps=1e-5, n=2, m=4, fmt=0, out=out)
            sq.linear(out, wq, out=yg)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(2):
        yg.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y)
    assert sq.lib().sharq_last_hip_error() == 0
    assert os.environ["SHARQ_DEBUG"] == "1"
