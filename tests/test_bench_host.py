"""Host-side checks of bench.py that need no GPU: the single-GPU refusal of
--gpus N > 1, and the algorithmic work and byte counts its roofline uses
(2*T*Nout*K*(1 + N/M) flops for the dual product; read X once and write
codes, scales and mask once for the prep; the FP4 weight payload)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_dual_product_flops_count_backbone_and_residual():
    # 2:4: the backbone carries half the multiply-adds of a dense product
    assert bench.gemm_flops(2048, 4096, 28672, 2, 4) == 2 * 2048 * 28672 * 4096 * 1.5
    assert bench.gemm_flops(1, 128, 64, 4, 4) == 2 * 64 * 128 * 2.0   # N = M: two dense products


def test_prep_and_weight_bytes():
    T, K = 2048, 4096
    # bf16 read, two code arrays (K/2 each), two scale arrays (K/32 MX, K/16 NV), bit mask K/8
    assert bench.prep_bytes(T, K, 0) == T * (2 * K + K + 2 * K // 32 + K // 8)
    assert bench.prep_bytes(T, K, 1) == T * (2 * K + K + 2 * K // 16 + K // 8)
    assert bench.weight_bytes(1, 28672, 4096, 0) == 28672 * 4096 * (0.5 + 1 / 32)
    assert bench.weight_bytes(128, 1536, 2048, 1) == 128 * 1536 * 2048 * (0.5 + 1 / 16)


def test_compressed_backbone_prep_bytes_and_format_choice():
    import types
    import synth
    T, K = 4096, 3584
    # backbone: K/4 kept code bytes + K/8 position bytes; residual K/2; NVFP4 scales; mask
    assert bench.prep_bytes(T, K, bench.FMT_NVFP4_SP24) == T * (2 * K + K // 2 + 3 * K // 8 + 2 * K // 16 + K // 8)
    sp, dense = types.SimpleNamespace(nv_backbone="sp24"), types.SimpleNamespace(nv_backbone="dense")
    assert bench.prep_format(synth.WORKLOADS[3], sp) == bench.FMT_NVFP4_SP24
    assert bench.prep_format(synth.WORKLOADS[3], dense) == synth.FMT_NVFP4
    for cid in (1, 2, 4):   # MXFP4 workloads keep the zero-filled backbone
        assert bench.prep_format(synth.WORKLOADS[cid], sp) == synth.FMT_MXFP4


def test_swiglu_prep_reads_gate_and_up_as_fp32():
    # the down projection's prep reads 2K float32 values per row instead of K bf16
    T, K = 2048, 14336
    assert bench.prep_bytes(T, K, 0, swiglu=True) == T * (8 * K + K + 2 * K // 32 + K // 8)


def test_prep_timing_rotation_exceeds_the_infinity_cache():
    x_bytes = 2048 * 4096 * 2
    n = bench.prep_copies(x_bytes)
    assert n * x_bytes > 2 * bench.INFINITY_CACHE_BYTES and n <= 48
    assert bench.prep_copies(1) == 48


def test_layer_workloads_have_four_linears_with_fused_down():
    import synth
    for cid in (1, 2, 3):
        names = [lin.name for lin in synth.WORKLOADS[cid].linears]
        assert names == ["qkv", "o_proj", "gate_up", "down"]
        lins = {lin.name: lin for lin in synth.WORKLOADS[cid].linears}
        assert lins["down"].swiglu_of == "gate_up" and lins["gate_up"].nout == 2 * lins["down"].k
        assert lins["o_proj"].k == lins["o_proj"].nout == lins["qkv"].k and lins["o_proj"].norm == 0
    moe = {lin.name: lin for lin in synth.WORKLOADS[4].linears}
    assert moe["expert_down"].swiglu_of == "expert_gate_up"
    assert moe["expert_gate_up"].nout == 2 * moe["expert_down"].k


def test_other_workloads_parses_child_lines_and_reports_failures(monkeypatch):
    """The default line's other_workloads: each child's JSON line is reduced
    to its step and roofline figures; a child that fails, times out or
    cannot start is reported with its status, and the others still run."""
    import json
    import types

    line = {"ms_per_step": 1.5, "value": 10.0, "unit": "TFLOP/s", "dtype": "x", "prep_GBps": 1.0,
            "prep_frac_hbm": 0.1, "gemm_TFLOPs": 2.0, "gemm_frac_peak": 0.2,
            "config": {"workload": "wl"},
            "per_linear": {"qkv": {"prep_in_step_us": 3.0, "gemm_us": 4.0}},
            "roofline": {"bound": "mfma", "achieved": 2.0, "peak": 10.0, "unit": "TFLOP/s", "frac": 0.2,
                         "traffic": None},
            "roofline_prep": {"frac": 0.1}}
    calls = []

    def fake_run(cmd, **kw):
        w = cmd[cmd.index("--workload") + 1]
        calls.append(w)
        assert "--no-extras" in cmd and "--no-cpu-baseline" in cmd
        if w == "qwen":
            return types.SimpleNamespace(returncode=1, stdout="", stderr="boom")
        if w == "moe":
            raise subprocess.TimeoutExpired(cmd, kw.get("timeout"))
        return types.SimpleNamespace(returncode=0, stdout="log line\n" + json.dumps(line) + "\n", stderr="")

    monkeypatch.setattr(subprocess, "run", fake_run)
    out = bench.other_workloads(types.SimpleNamespace(steps=3, warmup=1))
    assert calls == list(bench.OTHER_WORKLOADS)
    assert out["decode1"]["ms_per_step"] == 1.5 and out["decode1"]["workload"] == "wl"
    assert out["decode1"]["per_linear_us"] == {"qkv": {"prep": 3.0, "product": 4.0}}
    assert out["decode1"]["roofline"]["frac"] == 0.2 and out["decode1"]["roofline_prep_frac"] == 0.1
    assert out["qwen"]["status"] == 1 and "boom" in out["qwen"]["stderr_tail"]
    assert out["moe"]["status"] == "not run to the end"
