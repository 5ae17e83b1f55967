"""Benchmark of the SharQ hot path on one MI355X.

One step = the whole hot path over one batch: for each linear layer of the
workload, the fused preparation (norm, 2:4 mask, FP4 backbone, residual, FP4
residual) followed by the dual-path FP4 product.  The default workload is a
Llama-3.1-8B-shaped prefill layer (2048 tokens) in MXFP4 with the layer's
four linears in order: qkv 4096->6144 (RMSNorm), o_proj 4096->4096 (no norm),
gate_up 4096->28672 (RMSNorm) and down 14336->4096, whose preparation reads
gate_up's FP32 output and forms SiLU(gate)*up inside the prep kernel.
Inputs are seeded synthetic tensors of the models' shapes, resident in HBM
before the timed region; several copies of every input, weight and output are
rotated so that the 256 MB Infinity Cache cannot serve a step from the
previous one.

Prints one JSON line: whole-step dual-product throughput (algorithmic
TFLOP/s, 2*T*Nout*K*(1+N/M) per linear) over the K timed steps, captured as
one HIP graph after the W warmup steps (--graph off: eager launches); per-launch kernel times
from graphs that hold one phase (one linear's preps, or its products) over
rotated copies, timed with HIP events around a replay on the launch stream
(prep inputs rotated over enough copies to exceed twice the Infinity Cache);
the roofline of the dominant kernel (the dual product) and of the prep from
those times, with HBM-side traffic from the committed counter summaries under
profiles/ while the kernel sources match them; the products with BF16
output; the CPU oracle timed on a bounded sample on the host; the
operator-level error of SharQ next to plain FP4 round-to-nearest; the fused
SiLU(gate)*up prep against the unfused chain; and the same linears as bf16 /
FP8 GEMMs.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5]
                    [--workload llama|decode1|decode8|decode64|qwen|moe]
                    [--graph on|off] [--no-extras] [--no-cpu-baseline]
                    [--no-other-workloads]

The default workload's line also carries other_workloads: the step and
roofline figures of the decode, Qwen2.5-7B NVFP4 and Qwen3-30B-A3B MoE
workloads, each from a child run of this script after the timed region.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
F16_PEAK_TFLOPS = 2500.0        # MI355X dense f16 / bf16 MFMA
INFINITY_CACHE_BYTES = 256 << 20
# 32x32x64 block-scaled FP4 MFMA issued back to back from registers with
# random operands (no memory traffic), measured on MI355X: the chip lowers its
# clock under that load (about 1.6 GHz, against 2.1-2.3 GHz with constant operands)
MFMA_RANDOM_FP4_TFLOPS = 6250.0
ERROR_ROWS = 32                 # rows per linear in the error report
CPU_ROWS = 2048                 # rows per linear (per thread for the threaded prep) in the CPU baseline


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama")
    ap.add_argument("--rotate", type=int, default=None,
                    help="copies of every input, weight and output rotated across steps (default: 3, and 8 "
                         "for decode batches, so that the rotated set outgrows the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="run every timed step as one captured HIP graph (off: eager launches)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the BF16-output products, the unfused SiLU chain and the bf16 / fp8 GEMMs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter calibration)")
    ap.add_argument("--swiglu-epilogue", choices=["on", "off", "all"], default="on",
                    help="MXFP4 batches of more than 32 tokens: the gate_up product prepares the down "
                         "projection's input in its epilogue (sharq_linear_swiglu); off: gate_up's FP32 output, "
                         "then the SiLU(gate)*up prep; all: the epilogue at every batch size")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="default workload only: skip the short runs of the other workloads that the line "
                         "reports under other_workloads")
    ap.add_argument("--nv-backbone", choices=["sp24", "dense"], default="sp24",
                    help="NVFP4 2:4 workloads: store the backbone in the compressed 2:4 form and multiply it on "
                         "the sparse f16 matrix instruction (sp24), or zero-filled on the dense one (dense)")
    return ap.parse_args()


FMT_NVFP4_SP24 = 2  # the library's NVFP4 preparation with the backbone in the compressed 2:4 form


def block_of(fmt):
    return 32 if fmt == 0 else 16


def prep_bytes(T, K, fmt, swiglu=False):
    """Algorithmic bytes of one prep: read the input once (bf16 X, or the FP32
    gate and up halves for the SiLU(gate)*up prep), write codes, scales and
    mask.  The compressed 2:4 backbone holds K/4 code bytes and K/8 bytes of
    2-bit positions per row instead of K/2 code bytes."""
    read = 8 * K if swiglu else 2 * K
    codes = K // 2 + (3 * K // 8 if fmt == FMT_NVFP4_SP24 else K // 2)
    return T * (read + codes + 2 * K // block_of(fmt) + K // 8)


def gate_up_source_rows(nout):
    """Row of the stacked [gate; up] weight held by each payload row of
    sharq_quantize_weight_gate_up (groups of 32 interleaved)."""
    r = np.arange(nout)
    p, c = r // 64, r % 64
    return np.where(c < 32, 32 * p + c, nout // 2 + 32 * p + c - 32)


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
    expert batch through row_index).  When `src` is given, the prep input is
    src's FP32 output [gate | up] (SiLU(gate)*up formed in the prep kernel)."""

    def __init__(self, sq, torch, synth, wl, lin, prep_tokens, rotate, dev, route=None, gather=False,
                 src=None, prep_copies=None, pfmt=None, gate_up_order=False):
        self.lin, self.wl, self.src = lin, wl, src
        # SwiGLU epilogue: this layer's product prepares epi_dst's input
        # (its weight rows interleaved as sharq_quantize_weight_gate_up
        # stores them); epi_src: this layer's input comes from that epilogue
        self.gate_up_order = gate_up_order
        self.epi_dst = None
        self.epi_src = None
        self.pfmt = wl.fmt if pfmt is None else pfmt  # preparation format (weights: wl.fmt)
        self.prep_tokens = prep_tokens
        self.rotate = rotate
        self.x = None
        self.x_host = None
        n_in = rotate if prep_copies is None else max(rotate, prep_copies)
        if src is None:
            x = synth.activation(wl, lin, prep_tokens)
            xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            self.x = [xt] + [xt.clone() for _ in range(n_in - 1)]
            self.x_host = x
        else:
            n_in = rotate  # src's rotated outputs (each larger than the Infinity Cache)
        self.n_in = n_in
        self.g = None
        if lin.norm:
            self.g = torch.from_numpy(synth.gamma(wl, lin).view(np.int16)).view(torch.bfloat16).to(dev)
        w_bits = synth.weight(wl, lin)
        w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q = sq.quantize_weight(w, fmt=wl.fmt, gate_up=gate_up_order)
        del w
        self.w = [q] + [sq.QWeight(q.codes.clone(), q.scales.clone(),
                                   None if q.global_scale is None else q.global_scale.clone(),
                                   q.E, q.nout, q.K, q.fmt) for _ in range(rotate - 1)]
        self.E = q.E
        self.offs = self.ridx = None
        self.rows = prep_tokens
        self.sample_tokens = np.arange(prep_tokens)  # host rows of the prep input feeding output row r
        self.sample_experts = np.zeros(prep_tokens, np.int64)
        if route is not None:
            self.offs = torch.from_numpy(route.offsets).to(dev)
            self.rows = int(route.offsets[-1])
            if gather:
                self.ridx = torch.from_numpy(route.row_index).to(dev)
                self.sample_tokens = route.row_index.astype(np.int64)
            else:
                self.sample_tokens = np.arange(self.rows)
            self.sample_experts = route.expert_of_row.astype(np.int64)
        experts = sorted(set(self.sample_experts[:max(ERROR_ROWS, CPU_ROWS)].tolist()) | {0})
        self.w_host = {e: w_bits[e] for e in experts}  # weight rows the host-side reports need
        del w_bits
        self.prep = [sq.alloc_prepared(prep_tokens, lin.k, self.pfmt, dev) for _ in range(n_in)]
        self.y = [torch.empty((self.rows, lin.nout), dtype=torch.float32, device=dev) for _ in range(rotate)]
        self.y16 = None

    @property
    def swiglu(self):
        return self.src is not None

    def run_prep(self, sq, i):
        r = i % self.n_in
        if self.epi_src is not None:
            return  # prepared by the epilogue of epi_src's product
        self.run_prep_kernel(sq, i)

    def run_prep_kernel(self, sq, i):
        """This linear's preparation as its own kernel (the SiLU(gate)*up prep
        on src's FP32 output for a down projection)."""
        r = i % self.n_in
        if self.src is not None:
            sq.prepare_swiglu(self.src.y[i % self.src.rotate], self.lin.k, n=self.wl.n, m=self.wl.m,
                              fmt=self.pfmt, out=self.prep[r])
        else:
            sq.prepare(self.x[r], norm=self.lin.norm, gamma=self.g, eps=self.wl.eps, n=self.wl.n, m=self.wl.m,
                       fmt=self.pfmt, out=self.prep[r])

    def run_gemm(self, sq, i, bf16=False):
        r = i % self.rotate
        if self.epi_dst is not None and not bf16:
            d = self.epi_dst
            sq.linear_swiglu(self.prep[r], self.w[r], n=self.wl.n, m=self.wl.m, group_offsets=self.offs,
                             row_index=self.ridx, rows=self.rows, out=d.prep[i % d.n_in])
            return
        out = self.y16[r] if bf16 else self.y[r]
        sq.linear(self.prep[r], self.w[r], group_offsets=self.offs, row_index=self.ridx, rows=self.rows, out=out)

    def fill_outputs(self, sq, torch):
        """SwiGLU-epilogue layers: their FP32 products in the usual [gate | up]
        column order in self.y (for the host-side reports and the stand-alone
        SiLU prep timing), from the epilogue's optional product output."""
        if self.epi_dst is None:
            return
        src = torch.from_numpy(gate_up_source_rows(self.lin.nout)).to(self.y[0].device)
        tmp = torch.empty_like(self.y[0])
        for r in range(self.rotate):
            sq.linear_swiglu(self.prep[r], self.w[r], n=self.wl.n, m=self.wl.m, group_offsets=self.offs,
                             row_index=self.ridx, rows=self.rows, out=self.epi_dst.prep[r % self.epi_dst.n_in],
                             y=tmp)
            self.y[r][:, src] = tmp
        del tmp

    def run(self, sq, i, ev=None):
        """Prep then product of rotated copy i % rotate (events around each, if given)."""
        i = i % self.rotate
        if ev is not None:
            ev[0].record()
        self.run_prep(sq, i)
        if ev is not None:
            ev[1].record()
        self.run_gemm(sq, i)
        if ev is not None:
            ev[2].record()

    def prep_input_host(self, rows):
        """Host copy of the prep input rows (bf16 bits, or FP32 [gate | up] rows of src's output)."""
        if self.src is None:
            return self.x_host[rows]
        return self.src.y[0][rows].cpu().numpy()


_ORACLE_W = {}


def oracle_weight(L, e):
    """The oracle's own RTN payload of expert e of the layer's weight (host, cached)."""
    import oracle
    key = (L.wl.name, L.lin.name, e)
    if key not in _ORACLE_W:
        _ORACLE_W[key] = oracle.quantize_weight(L.w_host[e], L.wl.dtype, L.wl.fmt)
    return _ORACLE_W[key]


def usable_cores():
    """CPUs this process may run on: the affinity mask, limited by a cgroup CPU quota if one is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    quota = None
    for path in ("/sys/fs/cgroup/cpu.max",):
        try:
            q, per = open(path).read().split()[:2]
            if q != "max":
                quota = float(q) / float(per)
        except (OSError, ValueError):
            pass
    if quota is not None:
        n = max(1, min(n, int(math.floor(quota))))
    return n, quota


def host_info():
    n, quota = usable_cores()
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
    return {"cpus_usable": n, "cgroup_cpu_quota": quota, "cpu_count": os.cpu_count(), "cpu_model": model,
            "blas": blas}


def oracle_prep(L, rows):
    """The oracle's preparation of the given input rows of layer L."""
    import oracle
    import synth
    wl, lin = L.wl, L.lin
    if L.swiglu:
        return oracle.prepare_swiglu(L.prep_input_host(rows), lin.k, wl.n, wl.m, wl.fmt)
    g = synth.gamma(wl, lin) if lin.norm else None
    return oracle.prepare(L.x_host, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt, rows=rows)


def cpu_baseline(layers):
    """The oracle (C prep + float64 numpy product) on a bounded sample: the
    first CPU_ROWS input rows of every linear (MoE: against expert 0).  The
    prep runs on every usable core (rows split over threads that each call the
    single-threaded oracle on CPU_ROWS rows of their own; ctypes releases the
    interpreter lock during the call) and once on one thread; the product
    runs as float64 BLAS on the same number of threads."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores, _ = usable_cores()
    t_prep1 = t_prep_all = t_gemm = 0.0
    flops = 0.0
    b1 = b_all = 0
    for L in layers:
        wl, lin = L.wl, L.lin
        S = min(CPU_ROWS, L.prep_tokens)
        dw = oracle_weight(L, 0).deq(0)  # offline on both sides: not timed
        rows = np.arange(S)
        if L.swiglu:
            L._cpu_in = L.prep_input_host(np.arange(min(S * cores, L.prep_tokens)))
        t0 = time.perf_counter()
        p = oracle_prep_rows(L, rows)
        t1 = time.perf_counter()
        with threadpool_limits(limits=cores, user_api="blas"):
            t2 = time.perf_counter()
            _ = p.deq_backbone() @ dw.T + p.deq_residual() @ dw.T
            t3 = time.perf_counter()
        t_prep1 += t1 - t0
        t_gemm += t3 - t2
        flops += gemm_flops(S, lin.k, lin.nout, wl.n, wl.m)
        b1 += prep_bytes(S, lin.k, wl.fmt, L.swiglu)
        n_all = min(S * cores, L.prep_tokens)
        chunks = [c for c in np.array_split(np.arange(n_all), cores) if c.size]
        with ThreadPoolExecutor(len(chunks)) as ex:
            t4 = time.perf_counter()
            list(ex.map(lambda r: oracle_prep_rows(L, r), chunks))
            t_prep_all += time.perf_counter() - t4
        b_all += prep_bytes(n_all, lin.k, wl.fmt, L.swiglu)
        L._cpu_in = None
    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    prep_all_gbps = b_all / t_prep_all / 1e9
    t_prep_sample = b1 / (prep_all_gbps * 1e9)  # the sample's prep at the all-cores rate
    total = t_prep_sample + t_gemm
    return {
        "value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": f"first {CPU_ROWS} input rows of every linear (full weights); prep in the single-threaded C "
                  f"oracle on {len(chunks)} threads ({prep_all_gbps:.3f} GB/s; {b1 / t_prep1 / 1e9:.3f} GB/s on "
                  f"one thread), product in float64 numpy ({flops / t_gemm / 1e9:.2f} GFLOP/s on {cores} BLAS "
                  f"threads); value = sample product flops / (sample prep at the all-cores rate + product time)",
        "seconds": t_prep1 + t_prep_all + t_gemm, "prep_GBps_1thread": b1 / t_prep1 / 1e9,
        "prep_GBps_all_cores": prep_all_gbps, "prep_threads": len(chunks), "gemm_GFLOPs": flops / t_gemm / 1e9,
        "blas_threads_default": int(blas_threads), "host": host_info(),
    }


def oracle_prep_rows(L, rows):
    """oracle_prep for the CPU baseline: swiglu layers read their cached host rows."""
    import oracle
    if L.swiglu:
        wl = L.wl
        return oracle.prepare_swiglu(L._cpu_in[rows], L.lin.k, wl.n, wl.m, wl.fmt)
    return oracle_prep(L, rows)


def error_report(layers):
    """Relative Frobenius error of sampled output rows against an unquantized
    reference (the FP32 prepared activation x^ times the bf16 weight, in
    float64): SharQ on the GPU, SharQ in the oracle, plain FP4 round to
    nearest (N = M, no residual), the N = M ablation (residual kept, no
    mask), and SharQ's activation side alone (unquantized weight).  For a
    SiLU(gate)*up input, x^ is that product of the sampled rows; NVFP4 RTN
    and ablation rows then take the sample's own tensor scale."""
    import oracle
    import synth
    out = {}
    for L in layers:
        wl, lin = L.wl, L.lin
        S = min(ERROR_ROWS, L.rows)
        toks = L.sample_tokens[:S]
        exps = L.sample_experts[:S]
        if L.swiglu:
            sh = oracle.prepare_swiglu(L.prep_input_host(toks), lin.k, wl.n, wl.m, wl.fmt, trace=True)
            xh = sh.xhat
            rtn = oracle.prepare(xh, "f32", lin.k, oracle.NORM_NONE, None, None, 0.0, wl.m, wl.m, wl.fmt)
        else:
            x = L.x_host[toks]
            g = synth.gamma(wl, lin) if lin.norm else None
            xh = oracle.normalize(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps)
            sh = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.n, wl.m, wl.fmt)
            rtn = oracle.prepare(x, wl.dtype, lin.k, lin.norm, g, None, wl.eps, wl.m, wl.m, wl.fmt)
        xh = xh.astype(np.float64)
        xs = sh.deq_backbone() + sh.deq_residual()
        xa = rtn.deq_backbone() + rtn.deq_residual()
        ref = np.zeros((S, lin.nout))
        y = {k: np.zeros((S, lin.nout)) for k in ("sharq_oracle", "rtn", "nm_ablation", "activation_only")}
        for e in sorted(set(exps.tolist())):
            sel = np.nonzero(exps == e)[0]
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


def _replay_ms(torch, graph, reps=3):
    """Time of one replay of a captured graph: the median of `reps` replays
    after a warm one (HIP events on the current stream, which the replay is
    launched on)."""
    graph.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return sorted(ts)[len(ts) // 2]


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def phase_ms(torch, fn, launches):
    """Per-launch time of a phase: a graph holding `launches` calls fn(i),
    timed around one replay."""
    g = _capture(torch, lambda: [fn(i) for i in range(launches)])
    ms = _replay_ms(torch, g) / launches
    del g
    return ms


def swiglu_report(sq, torch, wl, layers):
    """The SiLU(gate)*up prep of the down projection (fused in the prep
    kernel, as in the layer step) against the unfused chain: torch SiLU*up to a
    bf16 tensor, then the bf16 prep."""
    down = next((L for L in layers if L.swiglu), None)
    if down is None:
        return None
    Ys = down.src.y                     # rotated copies, each larger than the Infinity Cache
    T, K = Ys[0].shape[0], down.lin.k
    out = sq.alloc_prepared(T, K, down.pfmt, Ys[0].device)
    it = [0]

    def nxt():
        it[0] += 1
        return Ys[it[0] % len(Ys)]

    fused = _event_ms(torch, lambda: sq.prepare_swiglu(nxt(), K, n=wl.n, m=wl.m, fmt=down.pfmt, out=out))
    act = torch.empty((T, K), dtype=torch.bfloat16, device=Ys[0].device)

    def unfused_chain():
        Y = nxt()
        act.copy_(torch.nn.functional.silu(Y[:, :K]) * Y[:, K:2 * K])
        sq.prepare(act, norm=0, n=wl.n, m=wl.m, fmt=down.pfmt, out=out)

    chain = _event_ms(torch, unfused_chain)
    return {"rows": T, "K": K, "fused_us": round(fused * 1e3, 2),
            "fused_GBps": round(prep_bytes(T, K, down.pfmt, True) / (fused * 1e-3) / 1e9, 1),
            "unfused_torch_silu_bf16_then_prep_us": round(chain * 1e3, 2),
            "speedup": round(chain / fused, 3),
            "timing": "eager launches, HIP events around 20 of them"}


def gemm_baselines(torch, synth, wl, layers, sharq_ms):
    """The same linears as plain bf16 GEMMs (torch.matmul, hipBLASLt) and as
    per-tensor-scaled FP8 e4m3 GEMMs (torch._scaled_mm), activation
    quantization not included; times next to SharQ's prep + product."""
    if wl.experts > 1:
        return None
    res = {}
    tot = {"bf16": 0.0, "fp8": 0.0}
    for L in layers:
        dev = L.y[0].device
        w = torch.from_numpy(np.ascontiguousarray(L.w_host[0]).view(np.int16)).view(torch.bfloat16).to(dev)
        if L.x is not None:
            x = L.x[0]
        else:  # SiLU(gate)*up of src's output as a bf16 activation
            Y = L.src.y[0]
            x = (torch.nn.functional.silu(Y[:, :L.lin.k]) * Y[:, L.lin.k:2 * L.lin.k]).to(torch.bfloat16)
        bf = _event_ms(torch, lambda: torch.matmul(x, w.t()))
        r = {"bf16_us": round(bf * 1e3, 2)}
        tot["bf16"] += bf
        try:
            f8 = torch.float8_e4m3fn
            xq, wq = x.to(f8), w.to(f8)
            one = torch.ones((), dtype=torch.float32, device=dev)
            fp8 = _event_ms(torch, lambda: torch._scaled_mm(xq, wq.t(), scale_a=one, scale_b=one,
                                                            out_dtype=torch.bfloat16))
            r["fp8_us"] = round(fp8 * 1e3, 2)
            if tot["fp8"] is not None:
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


def measured_traffic(name, epi=False):
    """HBM-side bytes per step of a kernel family from the committed counter
    summary under profiles/ (FETCH_SIZE / WRITE_SIZE scaled by a plain copy),
    or None when the kernel sources changed after the counters were taken or
    the counters come from the other layer-step mode (SwiGLU epilogue on or
    off)."""
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
    if t.get("swiglu_epilogue", False) != epi:
        return None
    return t if h.hexdigest() == t["source_sha256"] else None


def prep_copies(x_bytes):
    """Copies of a prep input that a prep-only timing graph rotates over:
    together more than twice the Infinity Cache (at most 48)."""
    return int(min(48, 2 * INFINITY_CACHE_BYTES // max(1, x_bytes) + 1))


def prep_format(wl, args):
    """The preparation's format: NVFP4 2:4 workloads whose K are whole 128-element
    tiles store the backbone compressed (unless --nv-backbone dense)."""
    if (wl.fmt == 1 and wl.n == 2 and wl.m == 4 and args.nv_backbone == "sp24"
            and all(lin.k % 128 == 0 for lin in wl.linears)):
        return FMT_NVFP4_SP24
    return wl.fmt


def swiglu_epilogue(args, wl, tokens):
    """The layer step prepares the down projection inside the gate_up
    product (MXFP4; "on": batches of more than 32 tokens, where its 128-row
    tiles beat the few-row products plus the separate prep -- measured on
    MI355X at 1, 8 and 64 tokens: 6% and 4% slower, 4% faster; "all": every
    batch)."""
    mode = getattr(args, "swiglu_epilogue", "on")
    return wl.fmt == 0 and (mode == "all" or (mode == "on" and tokens > 32))


def link_epilogues(layers, epi):
    if not epi:
        return
    for L in layers.values():
        if L.src is not None:
            L.src.epi_dst, L.epi_src = L, L.src


def build_layers(args, sq, torch, synth, dev):
    if args.rotate is None:
        args.rotate = 8 if args.workload.startswith("decode") else 3
    decode = args.workload.startswith("decode")
    if args.workload in ("llama", "qwen") or decode:
        wl = synth.WORKLOADS[3 if args.workload == "qwen" else (2 if decode else 1)]
        tokens = int(args.workload[len("decode"):]) if decode else wl.tokens
        pfmt = prep_format(wl, args)
        epi = swiglu_epilogue(args, wl, tokens)
        srcs = {lin.swiglu_of for lin in wl.linears if lin.swiglu_of}
        layers = {}
        for lin in wl.linears:
            pc = None if decode else prep_copies(tokens * lin.k * 2)
            layers[lin.name] = Layer(sq, torch, synth, wl, lin, tokens, args.rotate, dev,
                                     src=layers.get(lin.swiglu_of), prep_copies=pc, pfmt=pfmt,
                                     gate_up_order=epi and lin.name in srcs)
        link_epilogues(layers, epi)
        return wl, list(layers.values())
    if args.workload == "moe":
        wl = synth.WORKLOADS[4]
        route = synth.moe_routing(wl)
        rows = int(route.offsets[-1])
        gu_lin, down_lin = wl.linears
        # gate_up: prep the unique tokens, the product gathers each expert's rows;
        # down: prepared from gate_up's expert-sorted FP32 rows as SiLU(gate)*up
        epi = swiglu_epilogue(args, wl, wl.tokens)
        gu = Layer(sq, torch, synth, wl, gu_lin, wl.tokens, args.rotate, dev, route, gather=True,
                   prep_copies=prep_copies(wl.tokens * gu_lin.k * 2), gate_up_order=epi)
        down = Layer(sq, torch, synth, wl, down_lin, rows, args.rotate, dev, route, src=gu)
        link_epilogues({"gu": gu, "down": down}, epi)
        return wl, [gu, down]
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

    use_graph = args.graph == "on"
    decode = layers[0].prep_tokens <= 64

    # untimed runs of the whole step before any capture
    for i in range(2):
        for L in layers:
            L.run(sq, i)
    for L in layers:
        L.fill_outputs(sq, torch)
    torch.cuda.synchronize()

    # the W warmup steps and the K timed steps, each captured as one graph
    # (consecutive layer steps rotating over the buffer copies, as a model's
    # forward pass over its layers would be captured); captured here, before
    # the phase timings, so that no capture idles the GPU right before the
    # timed replay
    warm = steps_graph = None
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in layers:
                L.run(sq, 0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        if args.warmup > 0:
            warm = _capture(torch, lambda: [L.run(sq, s) for s in range(args.warmup) for L in layers])
        steps_graph = _capture(torch, lambda: [L.run(sq, s) for s in range(args.steps) for L in layers])
        torch.cuda.synchronize()

    # untimed steps for about 30 ms: a GPU that was idle runs its first
    # milliseconds at a lower clock (~10% slower layer steps, measured)
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < 0.03:
        for L in layers:
            L.run(sq, i)
        torch.cuda.synchronize()
        i += 1

    # ---- per-launch kernel times: graphs of one phase over rotated copies,
    # measured before the timed steps so that those too start on a GPU that
    # has been busy for a while
    # prep_ms: the prep kernels (the down projection's SiLU(gate)*up prep
    # timed on its own even when the layer step runs it in gate_up's
    # epilogue); step_prep_ms: the step's own prep launches
    prep_ms, gemm_ms, step_prep_ms = [], [], []
    for L in layers:
        n_prep = args.steps if decode else max(12, L.n_in)
        n_gemm = args.steps if decode else 12
        prep_ms.append(phase_ms(torch, lambda i, L=L: L.run_prep_kernel(sq, i), n_prep))
        step_prep_ms.append(0.0 if L.epi_src is not None else prep_ms[-1])
        gemm_ms.append(phase_ms(torch, lambda i, L=L: L.run_gemm(sq, i), n_gemm))

    # ---- W warmup steps, then exactly K timed steps
    if use_graph:
        if warm is not None:
            warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps_graph.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    else:
        for i in range(args.warmup):
            for L in layers:
                L.run(sq, i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            for L in layers:
                L.run(sq, s)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    flops = [gemm_flops(L.rows, L.lin.k, L.lin.nout, wl.n, wl.m) for L in layers]
    pbytes = [prep_bytes(L.prep_tokens, L.lin.k, L.pfmt, L.swiglu) for L in layers]
    wbytes = [weight_bytes(L.E, L.lin.nout, L.lin.k, wl.fmt) for L in layers]
    gemm_tflops = sum(flops) / (sum(gemm_ms) * 1e-3) / 1e12
    prep_gbps = sum(pbytes) / (sum(prep_ms) * 1e-3) / 1e9
    value = sum(flops) / (ms_step * 1e-3) / 1e12
    nv = wl.fmt != 0
    sp24 = layers[0].pfmt == FMT_NVFP4_SP24
    tokens = layers[0].prep_tokens
    plain = [i for i, L in enumerate(layers) if not L.swiglu]
    fused = [i for i, L in enumerate(layers) if L.swiglu]
    epi = any(L.epi_dst is not None for L in layers)

    def kind_gbps(ix):
        return None if not ix else round(sum(pbytes[i] for i in ix) / (sum(prep_ms[i] for i in ix) * 1e-3) / 1e9, 1)

    timing = (f"graphs of one phase over rotated copies (prep inputs over enough copies to exceed twice the "
              f"Infinity Cache; products over the step's {args.rotate} copies), HIP events around a replay (median "
              f"of three after a warm one), per launch = replay time / launches; measured before the timed steps")
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
        "dtype": ("fp4-e2m1 (nvfp4) -> f16 mfma (2:4 sparse backbone) -> fp32" if sp24 else
                  "fp4-e2m1 (nvfp4) -> f16 mfma -> fp32") if nv else "fp4-e2m1 (mxfp4) x fp4 -> fp32",
        "data": "synthetic (seeded; model-shaped activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": f"{wl.name}" + ("" if tokens == wl.tokens else f"_T{tokens}"),
                   "tokens": tokens, "linears": {L.lin.name: [L.lin.k, L.lin.nout] for L in layers},
                   "prep_input": {L.lin.name: ("SiLU(gate)*up of " + L.src.lin.name + " FP32 output")
                                  if L.swiglu else ("bf16, " + ("RMSNorm" if L.lin.norm == 1 else "no norm"))
                                  for L in layers},
                   "mask": f"{wl.n}:{wl.m}", "format": "NVFP4" if nv else "MXFP4",
                   "backbone": ("compressed 2:4 (kept codes + 2-bit positions), sparse f16 MFMA" if sp24 else
                                "zero-filled, dense MFMA"),
                   "rotated_copies": args.rotate,
                   "down_prep": ("in the gate_up product's epilogue (sharq_linear_swiglu)" if epi else
                                 "its own kernel on gate_up's FP32 output") if fused else None,
                   "launch": "the K timed steps as one HIP graph" if use_graph else "eager launches"},
        "prep_GBps": round(prep_gbps, 1),
        "prep_frac_hbm": round(prep_gbps / HBM_PEAK_GBPS, 4),
        "prep_GBps_bf16_input": kind_gbps(plain),
        "prep_GBps_swiglu_input": kind_gbps(fused),
        "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_peak": round(gemm_tflops / MXFP4_PEAK_TFLOPS, 4),
        "per_linear": {L.lin.name: {"rows": L.rows, "prep_us": round(prep_ms[i] * 1e3, 2),
                                    "prep_in_step_us": round(step_prep_ms[i] * 1e3, 2),
                                    "gemm_us": round(gemm_ms[i] * 1e3, 2),
                                    "prep_bytes": pbytes[i],
                                    "prep_GBps": round(pbytes[i] / (prep_ms[i] * 1e-3) / 1e9, 1),
                                    "gemm_TFLOPs": round(flops[i] / (gemm_ms[i] * 1e-3) / 1e12, 1),
                                    "weight_stream_GBps": round(wbytes[i] / (gemm_ms[i] * 1e-3) / 1e9, 1)}
                       for i, L in enumerate(layers)},
        "roofline": {"bound": "hbm" if decode else "mfma", "achieved": round(gemm_tflops, 1),
                     "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_tflops / MXFP4_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "kernel": ("k_dual_gemm<NVFP4_SP24> (dual-path product: 2:4 sparse f16 MFMA backbone, "
                                "dense f16 MFMA residual)" if sp24 else
                                "k_dual_gemm<NVFP4> (dual-path product, f16 MFMA)") if nv
                     else "k_dual_gemm<MXFP4> (dual-path product)",
                     "per_launch": "algorithmic 2*rows*Nout*K*(1+N/M) flops / launch time, summed over the linears"
                                   + ("; the gate_up launch also prepares the down projection's input in its "
                                      "epilogue (sharq_linear_swiglu)" if epi else ""),
                     "timing": timing},
        "roofline_prep": {"bound": "hbm", "achieved": round(prep_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(prep_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                          "per_launch": "algorithmic bytes (input read once, codes, scales and mask written) / "
                                        "launch time, summed over the linears' prep kernels"
                                        + ("; the down projection's SiLU(gate)*up prep kernel is timed on gate_up's "
                                           "FP32 output, while the layer step prepares that input in the gate_up "
                                           "product's epilogue instead" if epi else ""),
                          "timing": timing},
    }
    if decode:
        wstream = sum(wbytes) / (sum(gemm_ms) * 1e-3) / 1e9
        result["roofline"].update({"achieved": round(wstream, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(wstream / HBM_PEAK_GBPS, 4),
                                   "per_launch": "FP4 weight payload bytes / launch time (the weight stream), "
                                                 "summed over the linears",
                                   "gemm_TFLOPs": round(gemm_tflops, 1)})
    if nv:
        result["roofline"]["frac_of_f16_peak"] = round(gemm_tflops / F16_PEAK_TFLOPS, 4)
    for key, fname in (("roofline", f"k_dual_gemm_{wl.name}.traffic.json"),
                       ("roofline_prep", f"k_prep_{wl.name}.traffic.json")):
        t = measured_traffic(fname, epi) if tokens == wl.tokens else None
        if t is not None:
            result[key]["traffic"] = t["bytes_per_step"]
            result[key]["traffic_unit"] = "bytes per step (all launches of the kernel in one step)"
            result[key]["algorithmic_bytes_per_step"] = t["algorithmic_bytes_per_step"]
    if not decode:
        result["roofline"]["mfma_ceiling_random_fp4_TFLOPs"] = MFMA_RANDOM_FP4_TFLOPS
    if not args.no_extras:
        # products with BF16 output (the FP32 accumulator rounded to nearest even)
        g16 = {}
        for L in layers:
            L.y16 = [torch.empty((L.rows, L.lin.nout), dtype=torch.bfloat16, device=dev) for _ in range(L.rotate)]
            g16[L.lin.name] = phase_ms(torch, lambda i, L=L: L.run_gemm(sq, i, bf16=True),
                                       args.steps if decode else 12)
            L.y16 = None
        result["bf16_output"] = {
            "gemm_us": {k: round(v * 1e3, 2) for k, v in g16.items()},
            "gemm_TFLOPs": round(sum(flops) / (sum(g16.values()) * 1e-3) / 1e12, 1),
            "note": "same products, Y stored as BF16; FP32 Y is the parity contract and the headline"}
        result["swiglu_prep"] = swiglu_report(sq, torch, wl, layers)
        result["gemm_baselines"] = gemm_baselines(torch, synth, wl, layers, sum(step_prep_ms) + sum(gemm_ms))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers)
        result["error_report"] = error_report(layers)
    if args.workload == "llama" and not args.no_extras and not args.no_other_workloads:
        torch.cuda.synchronize()
        result["other_workloads"] = other_workloads(args)
    print(json.dumps(result), flush=True)


OTHER_WORKLOADS = ("decode1", "decode8", "decode64", "qwen", "moe")


def other_workloads(args):
    """The other workloads, each a child run of this script after the timed
    region of the default one (own process, own buffers): the step and
    roofline figures of its line.  A child that fails is reported with its
    exit status; the default workload's figures do not depend on these."""
    import subprocess
    keep = ("ms_per_step", "value", "unit", "dtype", "prep_GBps", "prep_frac_hbm", "gemm_TFLOPs",
            "gemm_frac_peak")
    out = {}
    for w in OTHER_WORKLOADS:
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", w, "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--no-extras", "--no-cpu-baseline"]
        try:
            r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
        except (subprocess.TimeoutExpired, OSError) as e:
            out[w] = {"status": "not run to the end", "error": str(e)[-400:]}
            continue
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            out[w] = {"status": r.returncode, "stderr_tail": r.stderr[-400:]}
            continue
        d = json.loads(lines[-1])
        res = {k: d[k] for k in keep if k in d}
        res["workload"] = d["config"]["workload"]
        res["per_linear_us"] = {k: {"prep": v["prep_in_step_us"], "product": v["gemm_us"]}
                                for k, v in d["per_linear"].items()}
        rf = d["roofline"]
        res["roofline"] = {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                               "frac_of_f16_peak") if k in rf}
        res["roofline_prep_frac"] = d["roofline_prep"]["frac"]
        out[w] = res
    return out


if __name__ == "__main__":
    main()
