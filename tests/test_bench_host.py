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
