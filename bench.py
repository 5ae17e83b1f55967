"""Benchmark of the SharQ hot path on one MI355X.

One step = the whole hot path over one batch: for each linear layer of a
Llama-3.1-8B-shaped prefill layer (2048 tokens; qkv 4096->6144 and gate_up
4096->28672 with RMSNorm, down 14336->4096 without norm), the fused
preparation (norm, 2:4 mask, MXFP4 backbone, residual, MXFP4 residual)
followed by the dual-path MXFP4 product.  Inputs are seeded synthetic
tensors of that shape, resident in HBM before the timed region; several
copies of every input and weight are rotated so that the 256 MB Infinity
Cache cannot serve a step from the previous one.

Prints one JSON line: whole-step dual-product throughput (algorithmic
TFLOP/s, 2*T*Nout*K*(1+N/M) per linear), prep GB/s, the roofline of the
dominant kernel (the dual product) measured with HIP events on the launch
stream, and the CPU oracle timed on a bounded sample on the host.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--workload llama|decode1|decode8|decode64|qwen|moe]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama")
    ap.add_argument("--rotate", type=int, default=3, help="copies of every input rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def prep_bytes(T, K, fmt):
    """Algorithmic bytes of one prep: read X (bf16) once, write codes, scales and mask."""
    per_row = 2 * K + K + (K // 16 if fmt == 0 else K // 8) + K // 8
    return T * per_row


def gemm_flops(rows, K, nout, n, m):
    """Algorithmic flops of the dual product: backbone (N/M dense) + residual."""
    return 2.0 * rows * nout * K * (1.0 + n / m)


class Layer:
    """One linear of the workload with its device buffers (rotated copies)."""

    def __init__(self, sq, torch, wl, lin, tokens, rotate, synth, dev):
        import synth as _s
        self.lin, self.tokens, self.wl = lin, tokens, wl
        x = _s.activation(wl, lin, tokens)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        self.x = [xt] + [xt.clone() for _ in range(rotate - 1)]
        self.g = None
        if lin.norm:
            self.g = torch.from_numpy(_s.gamma(wl, lin).view(np.int16)).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(_s.weight(wl, lin).view(np.int16)).view(torch.bfloat16).to(dev)
        q = sq.quantize_weight(w, fmt=wl.fmt)
        del w
        self.w = [q] + [sq.QWeight(q.codes.clone(), q.scales.clone(),
                                   None if q.global_scale is None else q.global_scale.clone(),
                                   q.E, q.nout, q.K, q.fmt) for _ in range(rotate - 1)]
        self.prep = [sq.alloc_prepared(tokens, lin.k, wl.fmt, dev) for _ in range(rotate)]
        self.y = [torch.empty((tokens, lin.nout), dtype=torch.float32, device=dev) for _ in range(rotate)]
        self.x_host = x

    def run(self, sq, i, ev=None):
        r = i % len(self.x)
        if ev is not None:
            ev[0].record()
        sq.prepare(self.x[r], norm=self.lin.norm, gamma=self.g, eps=self.wl.eps, n=self.wl.n, m=self.wl.m,
                   fmt=self.wl.fmt, out=self.prep[r])
        if ev is not None:
            ev[1].record()
        sq.linear(self.prep[r], self.w[r], out=self.y[r])
        if ev is not None:
            ev[2].record()


def cpu_baseline(layers, sample_rows=32):
    """The oracle (C prep + float64 numpy product) on a bounded sample: the
    first `sample_rows` tokens of every linear of the step."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    t_prep = t_gemm = 0.0
    flops = 0.0
    pbytes = 0
    for L in layers:
        wl, lin = L.wl, L.lin
        x = L.x_host[:sample_rows]
        g = synth.gamma(wl, lin) if lin.norm else None
        t0 = time.perf_counter()
        p = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
        t1 = time.perf_counter()
        ow = oracle_weight(L)  # offline on both sides: not timed
        t2 = time.perf_counter()
        dw = ow.deq(0)
        _ = p.deq_backbone() @ dw.T + p.deq_residual() @ dw.T
        t3 = time.perf_counter()
        t_prep += t1 - t0
        t_gemm += t3 - t2
        flops += gemm_flops(x.shape[0], lin.k, lin.nout, wl.n, wl.m)
        pbytes += prep_bytes(x.shape[0], lin.k, wl.fmt)
    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    total = t_prep + t_gemm
    return {
        "value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": f"first {sample_rows} tokens of qkv, gate_up and down (full weights); prep in "
                  f"single-threaded C ({pbytes / t_prep / 1e9:.3f} GB/s), product in float64 numpy "
                  f"({flops / t_gemm / 1e9:.2f} GFLOP/s on {blas_threads} BLAS threads)",
        "seconds": total, "prep_GBps": pbytes / t_prep / 1e9, "gemm_GFLOPs": flops / t_gemm / 1e9,
    }


_ORACLE_W = {}


def oracle_weight(L):
    """The oracle's own RTN payload of the layer's weight (host, cached)."""
    import oracle
    import synth
    key = (L.wl.name, L.lin.name)
    if key not in _ORACLE_W:
        _ORACLE_W[key] = oracle.quantize_weight(synth.weight(L.wl, L.lin), L.wl.dtype, L.wl.fmt)
    return _ORACLE_W[key]


def error_report(sq, torch, layers, sample_rows=32):
    """Relative Frobenius error of the layer output vs an unquantized reference
    (normalized activation times the bf16 weight, in float64), for SharQ on
    the GPU and for plain MXFP4 round-to-nearest (N = M, no residual)."""
    import oracle
    import synth
    out = {}
    for L in layers:
        wl, lin = L.wl, L.lin
        x = L.x_host[:sample_rows]
        g = synth.gamma(wl, lin) if lin.norm else None
        xh = oracle.normalize(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps).astype(np.float64)
        wf = synth.bits_to_f32(synth.weight(wl, lin)[0], wl.dtype).astype(np.float64)
        ref = xh @ wf.T
        dw = oracle_weight(L).deq(0)
        ysh = L.y[0][:sample_rows].double().cpu().numpy()
        rtn = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.m, wl.m, wl.fmt)
        yrtn = rtn.deq_backbone() @ dw.T
        e_sh = float(np.linalg.norm(ysh - ref) / np.linalg.norm(ref))
        e_rtn = float(np.linalg.norm(yrtn - ref) / np.linalg.norm(ref))
        out[lin.name] = {"sharq_gpu": e_sh, "mxfp4_rtn": e_rtn, "gap_closed": 1.0 - e_sh / e_rtn}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); "
              "the path is single-GPU by design, see the sharding notes in the design document.",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import sparsity_prep_amd as sq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sq.lib()
    if args.workload == "llama":
        wl, tokens = synth.WORKLOADS[1], synth.WORKLOADS[1].tokens
    elif args.workload.startswith("decode"):
        wl, tokens = synth.WORKLOADS[2], int(args.workload[len("decode"):])
    elif args.workload == "qwen":
        wl, tokens = synth.WORKLOADS[3], synth.WORKLOADS[3].tokens
    else:
        raise SystemExit(f"unknown workload {args.workload}")
    layers = [Layer(sq, torch, wl, lin, tokens, args.rotate, synth, dev) for lin in wl.linears]
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for i in range(args.warmup):
        for L in layers:
            L.run(sq, i)
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for li, L in enumerate(layers):
            L.run(sq, s, evs[s][li])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    prep_ms = [0.0] * len(layers)
    gemm_ms = [0.0] * len(layers)
    for s in range(args.steps):
        for li in range(len(layers)):
            e = evs[s][li]
            prep_ms[li] += e[0].elapsed_time(e[1]) / args.steps
            gemm_ms[li] += e[1].elapsed_time(e[2]) / args.steps
    flops = [gemm_flops(tokens, L.lin.k, L.lin.nout, wl.n, wl.m) for L in layers]
    pbytes = [prep_bytes(tokens, L.lin.k, wl.fmt) for L in layers]
    gemm_tflops = sum(flops) / (sum(gemm_ms) * 1e-3) / 1e12
    prep_gbps = sum(pbytes) / (sum(prep_ms) * 1e-3) / 1e9
    value = sum(flops) / (ms_step * 1e-3) / 1e12
    peak = MXFP4_PEAK_TFLOPS if wl.fmt == 0 else BF16_PEAK_TFLOPS

    result = {
        "metric": "prep GB/s + dual-GEMM TFLOP/s, % of HBM / MXFP4 MFMA peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1 (mxfp4) x fp4 -> fp32" if wl.fmt == 0 else "fp4-e2m1 (nvfp4) -> bf16 mfma -> fp32",
        "data": "synthetic (seeded; Llama-3.1-8B-shaped activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": f"{wl.name}" + ("" if tokens == wl.tokens else f"_T{tokens}"),
                   "tokens": tokens, "linears": {L.lin.name: [L.lin.k, L.lin.nout] for L in layers},
                   "mask": f"{wl.n}:{wl.m}", "format": "MXFP4" if wl.fmt == 0 else "NVFP4",
                   "rotated_copies": args.rotate},
        "prep_GBps": round(prep_gbps, 1),
        "prep_frac_hbm": round(prep_gbps / HBM_PEAK_GBPS, 4),
        "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_peak": round(gemm_tflops / peak, 4),
        "per_linear": {L.lin.name: {"prep_us": round(prep_ms[i] * 1e3, 2), "gemm_us": round(gemm_ms[i] * 1e3, 2),
                                    "prep_GBps": round(pbytes[i] / (prep_ms[i] * 1e-3) / 1e9, 1),
                                    "gemm_TFLOPs": round(flops[i] / (gemm_ms[i] * 1e-3) / 1e12, 1)}
                       for i, L in enumerate(layers)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / peak, 4), "traffic": None,
                     "kernel": "k_dual_gemm_mx (dual-path product)",
                     "per_launch": "algorithmic 2*T*Nout*K*(1+N/M) flops / HIP-event launch time, "
                                   "summed over the three linears"},
        "roofline_prep": {"bound": "hbm", "achieved": round(prep_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(prep_gbps / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers)
        result["error_report"] = error_report(sq, torch, layers)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
