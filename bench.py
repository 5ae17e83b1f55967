"""Benchmark of the SharQ hot path on one MI355X.

One step = the whole hot path over one batch: for each linear layer of the
workload, the fused preparation (norm, 2:4 mask, FP4 backbone, residual, FP4
residual) followed by the dual-path FP4 product.  The default workload is a
Llama-3.1-8B-shaped prefill layer (2048 tokens; qkv 4096->6144 and gate_up
4096->28672 with RMSNorm, down 14336->4096 without norm) in MXFP4.  Inputs
are seeded synthetic tensors of the models' shapes, resident in HBM before
the timed region; several copies of every input and weight are rotated so
that the 256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line: whole-step dual-product throughput (algorithmic
TFLOP/s, 2*T*Nout*K*(1+N/M) per linear) with every timed step run as one
captured HIP graph (--graph off: eager launches), prep GB/s, the roofline of
the dominant kernel (the dual product) from per-launch times taken with HIP
events on the launch stream (eager steps around every launch; for decode
batches, graphs holding one phase over the rotated copies), with its
HBM-side traffic from the committed counter summary under profiles/ while
the kernel sources match it, the CPU oracle timed on a bounded sample on
the host, the operator-level error of SharQ next to plain FP4
round-to-nearest, the fused SiLU(gate)*up prep of the down projection next
to the unfused chain, and the same linears as bf16 / FP8 GEMMs.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5]
                    [--workload llama|decode1|decode8|decode64|qwen|moe]
                    [--graph on|off] [--no-extras] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
F16_PEAK_TFLOPS = 2500.0        # MI355X dense f16 / bf16 MFMA
# 32x32x64 block-scaled FP4 MFMA issued back to back from registers with
# random operands (no memory traffic), measured on MI355X: the chip lowers its
# clock under that load (about 1.6 GHz, against 2.1-2.3 GHz with constant operands)
MFMA_RANDOM_FP4_TFLOPS = 6250.0
SAMPLE_ROWS = 32                # rows per linear in the CPU baseline and the error report


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama")
    ap.add_argument("--rotate", type=int, default=None,
                    help="copies of every input and weight rotated across steps (default: 3, and 8 for "
                         "decode batches, so that the rotated set outgrows the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="run every timed step as one captured HIP graph (off: eager launches "
                         "from the host, with HIP events around every launch)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fused SiLU(gate)*up prep and the bf16 / fp8 GEMM comparisons")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def block_of(fmt):
    return 32 if fmt == 0 else 16


def prep_bytes(T, K, fmt):
    """Algorithmic bytes of one prep: read X (bf16) once, write codes, scales and mask."""
    per_row = 2 * K + K + 2 * K // block_of(fmt) + K // 8
    return T * per_row


def gemm_flops(rows, K, nout, n, m):
    """Algorithmic flops of the dual product: backbone (N/M dense) + residual."""
    return 2.0 * rows * nout * K * (1.0 + n / m)


def weight_bytes(E, nout, K, fmt):
    """FP4 weight payload (codes and block scales), read once per product."""
    return E * nout * K * (0.5 + 1.0 / block_of(fmt))


class Layer:
    """One linear of the workload with its device buffers (rotated copies).

    prep_tokens rows are prepared; the product writes `rows` output rows
    (more than prep_tokens when a grouped product gathers rows of an MoE
    expert batch through row_index)."""

    def __init__(self, sq, torch, synth, wl, lin, prep_tokens, rotate, dev, route=None, gather=False):
        self.lin, self.wl = lin, wl
        self.prep_tokens = prep_tokens
        x = synth.activation(wl, lin, prep_tokens)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        self.x = [xt] + [xt.clone() for _ in range(rotate - 1)]
        self.x_host = x
        self.g = None
        if lin.norm:
            self.g = torch.from_numpy(synth.gamma(wl, lin).view(np.int16)).view(torch.bfloat16).to(dev)
        w_bits = synth.weight(wl, lin)
        w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q = sq.quantize_weight(w, fmt=wl.fmt)
        del w
        self.w = [q] + [sq.QWeight(q.codes.clone(), q.scales.clone(),
                                   None if q.global_scale is None else q.global_scale.clone(),
                                   q.E, q.nout, q.K, q.fmt) for _ in range(rotate - 1)]
        self.E = q.E
        self.offs = self.ridx = None
        self.rows = prep_tokens
        S = min(SAMPLE_ROWS, prep_tokens)
        self.sample_tokens = np.arange(S)          # host rows of x feeding the sampled outputs
        self.sample_experts = np.zeros(S, np.int64)
        if route is not None:
            self.offs = torch.from_numpy(route.offsets).to(dev)
            self.rows = int(route.offsets[-1])
            if gather:
                self.ridx = torch.from_numpy(route.row_index).to(dev)
                self.sample_tokens = route.row_index[:S].astype(np.int64)
            self.sample_experts = route.expert_of_row[:S].astype(np.int64)
        experts = sorted(set(self.sample_experts.tolist()) | {0})
        self.w_host = {e: w_bits[e] for e in experts}  # weight rows the host-side reports need
        del w_bits
        self.prep = [sq.alloc_prepared(prep_tokens, lin.k, wl.fmt, dev) for _ in range(rotate)]
        self.y = [torch.empty((self.rows, lin.nout), dtype=torch.float32, device=dev) for _ in range(rotate)]

    def run_prep(self, sq, i):
        r = i % len(self.x)
        sq.prepare(self.x[r], norm=self.lin.norm, gamma=self.g, eps=self.wl.eps, n=self.wl.n, m=self.wl.m,
                   fmt=self.wl.fmt, out=self.prep[r])

    def run_gemm(self, sq, i):
        r = i % len(self.x)
        sq.linear(self.prep[r], self.w[r], group_offsets=self.offs, row_index=self.ridx, rows=self.rows,
                  out=self.y[r])

    def run(self, sq, i, ev=None):
        r = i % len(self.x)
        if ev is not None:
            ev[0].record()
        sq.prepare(self.x[r], norm=self.lin.norm, gamma=self.g, eps=self.wl.eps, n=self.wl.n, m=self.wl.m,
                   fmt=self.wl.fmt, out=self.prep[r])
        if ev is not None:
            ev[1].record()
        sq.linear(self.prep[r], self.w[r], group_offsets=self.offs, row_index=self.ridx, rows=self.rows,
                  out=self.y[r])
        if ev is not None:
            ev[2].record()


_ORACLE_W = {}


def oracle_weight(L, e):
    """The oracle's own RTN payload of expert e of the layer's weight (host, cached)."""
    import oracle
    key = (L.wl.name, L.lin.name, e)
    if key not in _ORACLE_W:
        _ORACLE_W[key] = oracle.quantize_weight(L.w_host[e], L.wl.dtype, L.wl.fmt)
    return _ORACLE_W[key]


def host_info():
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count()
    model = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)"
            for d in threadpool_info() if d.get("user_api") == "blas"]
    return {"cpus_usable": ncpu, "cpu_model": model, "blas": blas}


def cpu_baseline(layers):
    """The oracle (C prep + float64 numpy product) on a bounded sample: the
    first SAMPLE_ROWS tokens of every linear of the step (MoE: against expert
    0).  The prep also runs on all usable cores (rows split over threads that
    each call the same single-threaded oracle)."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    t_prep = t_gemm = t_prep_all = 0.0
    flops = 0.0
    pbytes = pbytes_all = 0
    cores = host_info()["cpus_usable"]
    for L in layers:
        wl, lin = L.wl, L.lin
        S = min(SAMPLE_ROWS, L.prep_tokens)
        x = L.x_host[:S]
        g = synth.gamma(wl, lin) if lin.norm else None
        dw = oracle_weight(L, 0).deq(0)  # offline on both sides: not timed
        t0 = time.perf_counter()
        p = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
        t1 = time.perf_counter()
        _ = p.deq_backbone() @ dw.T + p.deq_residual() @ dw.T
        t2 = time.perf_counter()
        t_prep += t1 - t0
        t_gemm += t2 - t1
        flops += gemm_flops(S, lin.k, lin.nout, wl.n, wl.m)
        pbytes += prep_bytes(S, lin.k, wl.fmt)
        # all cores: S rows per thread
        n_all = min(S * cores, L.prep_tokens)
        chunks = [c for c in np.array_split(np.arange(n_all), cores) if c.size]
        t3 = time.perf_counter()
        with ThreadPoolExecutor(len(chunks)) as ex:
            list(ex.map(lambda r: oracle.prepare(L.x_host, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n,
                                                 wl.m, wl.fmt, rows=r), chunks))
        t_prep_all += time.perf_counter() - t3
        pbytes_all += prep_bytes(n_all, lin.k, wl.fmt)
    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    total = t_prep + t_gemm
    return {
        "value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": f"first {SAMPLE_ROWS} tokens of every linear (full weights); prep in single-threaded C "
                  f"({pbytes / t_prep / 1e9:.3f} GB/s), product in float64 numpy "
                  f"({flops / t_gemm / 1e9:.2f} GFLOP/s on {blas_threads} BLAS threads)",
        "seconds": total, "prep_GBps_1thread": pbytes / t_prep / 1e9,
        "prep_GBps_all_cores": pbytes_all / t_prep_all / 1e9, "gemm_GFLOPs": flops / t_gemm / 1e9,
        "host": host_info(),
    }


def error_report(layers):
    """Relative Frobenius error of sampled output rows against an unquantized
    reference (the FP32 normalized activation times the bf16 weight, in
    float64): SharQ on the GPU, SharQ in the oracle, plain FP4 round to
    nearest (N = M, no residual), the N = M ablation (residual kept, no
    mask), and SharQ's activation side alone (unquantized weight)."""
    import oracle
    import synth
    out = {}
    for L in layers:
        wl, lin = L.wl, L.lin
        S = L.sample_tokens.size
        x = L.x_host[L.sample_tokens]
        g = synth.gamma(wl, lin) if lin.norm else None
        xh = oracle.normalize(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps).astype(np.float64)
        sh = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
        rtn = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.m, wl.m, wl.fmt)
        xs = sh.deq_backbone() + sh.deq_residual()
        xa = rtn.deq_backbone() + rtn.deq_residual()
        ref = np.zeros((S, lin.nout))
        y = {k: np.zeros((S, lin.nout)) for k in ("sharq_oracle", "rtn", "nm_ablation", "activation_only")}
        for e in sorted(set(L.sample_experts.tolist())):
            sel = np.nonzero(L.sample_experts == e)[0]
            wf = synth.bits_to_f32(L.w_host[e], wl.dtype).astype(np.float64)
            dw = oracle_weight(L, e).deq(0)
            ref[sel] = xh[sel] @ wf.T
            y["sharq_oracle"][sel] = xs[sel] @ dw.T
            y["rtn"][sel] = rtn.deq_backbone()[sel] @ dw.T
            y["nm_ablation"][sel] = xa[sel] @ dw.T
            y["activation_only"][sel] = xs[sel] @ wf.T
        ysh = L.y[0][:S].double().cpu().numpy()
        den = np.linalg.norm(ref)
        e = {"sharq_gpu": float(np.linalg.norm(ysh - ref) / den)}
        e.update({k: float(np.linalg.norm(v - ref) / den) for k, v in y.items()})
        e["gap_closed"] = 1.0 - e["sharq_gpu"] / e["rtn"]
        out[lin.name] = e
    return out


def _event_ms(torch, fn, reps=20):
    """Mean time of fn() over reps launches on the current stream (HIP events)."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _replay_ms(torch, graph):
    """Time of one replay of a captured graph (HIP events, after one warm replay)."""
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def swiglu_report(sq, torch, wl, layers):
    """The down projection's prep from the gate/up product's float32 output:
    fused (SiLU(gate)*up computed inside the prep kernel) against an unfused
    chain (torch SiLU*up to a bf16 tensor, then the bf16 prep)."""
    gu_layer = next((L for L in layers if L.lin.name == "gate_up"), None)
    down = next((L for L in layers if L.lin.name == "down"), None)
    if gu_layer is None or down is None or gu_layer.rows != down.prep_tokens:
        return None
    Ys = gu_layer.y                     # rotated copies, so the Infinity Cache cannot hold the input
    T, K = Ys[0].shape[0], Ys[0].shape[1] // 2
    out = sq.alloc_prepared(T, K, wl.fmt, Ys[0].device)
    it = [0]

    def nxt():
        it[0] += 1
        return Ys[it[0] % len(Ys)]

    fused = _event_ms(torch, lambda: sq.prepare_swiglu(nxt(), K, n=wl.n, m=wl.m, fmt=wl.fmt, out=out))
    act = torch.empty((T, K), dtype=torch.bfloat16, device=Ys[0].device)

    def unfused_chain():
        Y = nxt()
        act.copy_(torch.nn.functional.silu(Y[:, :K]) * Y[:, K:])
        sq.prepare(act, norm=0, n=wl.n, m=wl.m, fmt=wl.fmt, out=out)

    chain = _event_ms(torch, unfused_chain)
    B = block_of(wl.fmt)
    algo = T * (8 * K + K + 2 * K // B + K // 8)   # read gate and up (f32), write the prepared tensors
    return {"rows": T, "K": K, "fused_us": round(fused * 1e3, 2), "fused_GBps": round(algo / (fused * 1e-3) / 1e9, 1),
            "unfused_torch_silu_bf16_then_prep_us": round(chain * 1e3, 2),
            "speedup": round(chain / fused, 3),
            "bytes_note": "fused algorithmic bytes = read 2K f32 + write codes, scales, mask"}


def gemm_baselines(torch, synth, wl, layers, sharq_ms):
    """The same linears as plain bf16 GEMMs (torch.matmul, hipBLASLt) and as
    per-tensor-scaled FP8 e4m3 GEMMs (torch._scaled_mm), activation
    quantization not included; times next to SharQ's prep + product."""
    if wl.experts > 1:
        return None
    res = {}
    tot = {"bf16": 0.0, "fp8": 0.0}
    for L in layers:
        w = torch.from_numpy(np.ascontiguousarray(L.w_host[0]).view(np.int16)).view(torch.bfloat16).to(L.x[0].device)
        x = L.x[0]
        bf = _event_ms(torch, lambda: torch.matmul(x, w.t()))
        r = {"bf16_us": round(bf * 1e3, 2)}
        tot["bf16"] += bf
        try:
            f8 = torch.float8_e4m3fn
            xq, wq = x.to(f8), w.to(f8)
            one = torch.ones((), dtype=torch.float32, device=x.device)
            fp8 = _event_ms(torch, lambda: torch._scaled_mm(xq, wq.t(), scale_a=one, scale_b=one,
                                                            out_dtype=torch.bfloat16))
            r["fp8_us"] = round(fp8 * 1e3, 2)
            tot["fp8"] += fp8
        except Exception as e:  # no FP8 GEMM in this torch build
            r["fp8_error"] = str(e)[:120]
            tot["fp8"] = None
        res[L.lin.name] = r
        del w
    res["total_us"] = {"sharq_prep_plus_product": round(sharq_ms * 1e3, 2),
                       "bf16_gemm": round(tot["bf16"] * 1e3, 2),
                       "fp8_gemm": None if tot["fp8"] is None else round(tot["fp8"] * 1e3, 2)}
    return res


def measured_traffic(name):
    """HBM-side bytes per step of a kernel family from the committed counter
    summary under profiles/ (FETCH_SIZE / WRITE_SIZE scaled by a plain copy),
    or None when the kernel sources changed after the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", name)
    try:
        with open(path) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for src in t["sources"]:
            with open(os.path.join(root, src), "rb") as f:
                h.update(f.read())
    except (OSError, ValueError, KeyError):
        return None
    return t if h.hexdigest() == t["source_sha256"] else None


def build_layers(args, sq, torch, synth, dev):
    if args.rotate is None and not args.workload.startswith("decode"):
        args.rotate = 3
    if args.workload == "llama":
        wl = synth.WORKLOADS[1]
        return wl, [Layer(sq, torch, synth, wl, lin, wl.tokens, args.rotate, dev) for lin in wl.linears]
    if args.workload.startswith("decode"):
        wl, tokens = synth.WORKLOADS[2], int(args.workload[len("decode"):])
        if args.rotate is None:
            args.rotate = 8
        return wl, [Layer(sq, torch, synth, wl, lin, tokens, args.rotate, dev) for lin in wl.linears]
    if args.workload == "qwen":
        wl = synth.WORKLOADS[3]
        return wl, [Layer(sq, torch, synth, wl, lin, wl.tokens, args.rotate, dev) for lin in wl.linears]
    if args.workload == "moe":
        wl = synth.WORKLOADS[4]
        route = synth.moe_routing(wl)
        rows = int(route.offsets[-1])
        # gate_up: prep the unique tokens, the product gathers each expert's rows;
        # down: prep the expert-sorted rows themselves
        return wl, [Layer(sq, torch, synth, wl, wl.linears[0], wl.tokens, args.rotate, dev, route, gather=True),
                    Layer(sq, torch, synth, wl, wl.linears[1], rows, args.rotate, dev, route)]
    raise SystemExit(f"unknown workload {args.workload}")


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
    wl, layers = build_layers(args, sq, torch, synth, dev)
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

    use_graph = args.graph == "on"
    decode = layers[0].prep_tokens <= 64
    prep_ms = [0.0] * len(layers)
    gemm_ms = [0.0] * len(layers)

    def eager_steps(evs):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            for li, L in enumerate(layers):
                L.run(sq, s, None if evs is None else evs[s][li])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    if use_graph:
        # one captured graph per rotated copy, holding the whole step
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(2):
                for L in layers:
                    L.run(sq, i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        step_graphs = []
        for r in range(args.rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for L in layers:
                    L.run(sq, r)
            step_graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            step_graphs[i % args.rotate].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step_graphs[s % args.rotate].replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    if use_graph and decode:
        # per-launch times of decode kernels (a few microseconds each, shorter
        # than a host launch): one graph per phase holding that phase once per
        # timed step over the rotated copies, timed with HIP events around a replay
        for li, L in enumerate(layers):
            gp, gg = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gp):
                for i in range(args.steps):
                    L.run_prep(sq, i)
            with torch.cuda.graph(gg):
                for i in range(args.steps):
                    L.run_gemm(sq, i)
            prep_ms[li] = _replay_ms(torch, gp) / args.steps
            gemm_ms[li] = _replay_ms(torch, gg) / args.steps
    else:
        # per-launch times from eager steps with HIP events around every launch
        # (same order and cache state as the step; each interval also holds the
        # gap after the preceding launch)
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers]
               for _ in range(args.steps)]
        t_eager = eager_steps(evs)
        if not use_graph:
            ms_step = t_eager * 1e3 / args.steps
        for s in range(args.steps):
            for li in range(len(layers)):
                e = evs[s][li]
                prep_ms[li] += e[0].elapsed_time(e[1]) / args.steps
                gemm_ms[li] += e[1].elapsed_time(e[2]) / args.steps
    flops = [gemm_flops(L.rows, L.lin.k, L.lin.nout, wl.n, wl.m) for L in layers]
    pbytes = [prep_bytes(L.prep_tokens, L.lin.k, wl.fmt) for L in layers]
    wbytes = [weight_bytes(L.E, L.lin.nout, L.lin.k, wl.fmt) for L in layers]
    gemm_tflops = sum(flops) / (sum(gemm_ms) * 1e-3) / 1e12
    prep_gbps = sum(pbytes) / (sum(prep_ms) * 1e-3) / 1e9
    value = sum(flops) / (ms_step * 1e-3) / 1e12
    nv = wl.fmt != 0
    tokens = layers[0].prep_tokens

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
        "dtype": "fp4-e2m1 (nvfp4) -> f16 mfma -> fp32" if nv else "fp4-e2m1 (mxfp4) x fp4 -> fp32",
        "data": "synthetic (seeded; model-shaped activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": f"{wl.name}" + ("" if tokens == wl.tokens else f"_T{tokens}"),
                   "tokens": tokens, "linears": {L.lin.name: [L.lin.k, L.lin.nout] for L in layers},
                   "mask": f"{wl.n}:{wl.m}", "format": "NVFP4" if nv else "MXFP4",
                   "rotated_copies": args.rotate,
                   "launch": "one HIP graph per step" if use_graph else "eager launches"},
        "prep_GBps": round(prep_gbps, 1),
        "prep_frac_hbm": round(prep_gbps / HBM_PEAK_GBPS, 4),
        "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_peak": round(gemm_tflops / MXFP4_PEAK_TFLOPS, 4),
        "per_linear": {L.lin.name: {"rows": L.rows, "prep_us": round(prep_ms[i] * 1e3, 2),
                                    "gemm_us": round(gemm_ms[i] * 1e3, 2),
                                    "prep_GBps": round(pbytes[i] / (prep_ms[i] * 1e-3) / 1e9, 1),
                                    "gemm_TFLOPs": round(flops[i] / (gemm_ms[i] * 1e-3) / 1e12, 1),
                                    "weight_stream_GBps": round(wbytes[i] / (gemm_ms[i] * 1e-3) / 1e9, 1)}
                       for i, L in enumerate(layers)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": MXFP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MXFP4_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_dual_gemm<NVFP4> (dual-path product, f16 MFMA)" if nv else "k_dual_gemm<MXFP4> (dual-path product)",
                     "per_launch": "algorithmic 2*rows*Nout*K*(1+N/M) flops / HIP-event launch time, "
                                   "summed over the linears",
                     "timing": ("graphs of one phase over the rotated copies, HIP events around a replay"
                                if use_graph and decode else "eager steps, HIP events around every launch")},
        "roofline_prep": {"bound": "hbm", "achieved": round(prep_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(prep_gbps / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if nv:
        result["roofline"]["frac_of_f16_peak"] = round(gemm_tflops / F16_PEAK_TFLOPS, 4)
    if wl.name == "llama3.1-8b_prefill_T2048_mxfp4" and tokens == wl.tokens:
        for key, fname in (("roofline", "k_dual_gemm_mxfp4_llama3.1-8b_prefill_T2048.traffic.json"),
                           ("roofline_prep", "k_prep_mxfp4_llama3.1-8b_prefill_T2048.traffic.json")):
            t = measured_traffic(fname)
            if t is not None:
                result[key]["traffic"] = t["bytes_per_step"]
                result[key]["traffic_unit"] = "bytes per step (all launches of the kernel in one step)"
                result[key]["algorithmic_bytes_per_step"] = t["algorithmic_bytes_per_step"]
    result["roofline"]["mfma_ceiling_random_fp4_TFLOPs"] = MFMA_RANDOM_FP4_TFLOPS
    if not args.no_extras:
        result["swiglu_prep"] = swiglu_report(sq, torch, wl, layers)
        result["gemm_baselines"] = gemm_baselines(torch, synth, wl, layers, sum(prep_ms) + sum(gemm_ms))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers)
        result["error_report"] = error_report(layers)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
