"""The gfx950 2:4 sparse f16 matrix instruction (v_smfmac_f32_32x32x32_f16)
on the GPU against a host model of its operand layout, and the rate of the
sparse instruction next to the dense f16 one.  Evidence for the sparse-MFMA
decision: the sparse instruction multiplies exactly (f16 products, FP32
sums) with a 2-bit position per kept value and no block-scale operand; the
SharQ NVFP4 backbone (E2M1 code times E4M3 scale, exact in f16) could feed
it, the block-scaled MXFP4 one could not (SharQ: Bridging Activation
Sparsity and FP4 Quantization for LLM Inference, Abstract: a sparse FP4
product on the backbone).

Host model of the instruction (D = A * B, A 32x32 with two kept values in
every group of four consecutive K positions, B 32x32, D 32x32):
  A, lane l: row l % 32, eight halves v = 0..7, the kept values of K
     positions 16h .. 16h + 15 (h = l / 32), value v in group v // 2 at
     position p = bits 2v, 2v+1 of the selected 16-bit half of the index
     word (abid 0: bits 0-15, abid 1: bits 16-31): K = 16h + 4(v // 2) + p;
  B, lane l: column l % 32, halves 0..7 at K = 8h + k, halves 8..15 at
     K = 16 + 8h + (k - 8);
  D, lane l, register r: row 8(r // 4) + 4h + r % 4, column l % 32.
Operands are small integers, so every product and sum is exact and the
comparison is bit for bit."""
import ctypes
import os

import numpy as np
import pytest

from smfmac_model import lanes_to_matrix as _lanes, model as _model

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "hwprobe", "libsmfmac_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (python tests/hwprobe/build.py)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_smfmac.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    lib.probe_smfmac.restype = ctypes.c_int
    lib.probe_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    lib.probe_rate.restype = ctypes.c_int
    return lib


def test_host_model_reduces_to_a_dense_product_when_indices_list_every_position():
    """Pin of the model itself: two instructions whose kept positions are
    {0, 1} and {2, 3} of every group together multiply the dense rows."""
    rng = np.random.default_rng(5)
    Adense = rng.integers(-4, 5, (32, 32)).astype(np.float64)
    B = rng.integers(-4, 5, (64, 16)).astype(np.float64)
    assert not _model(np.zeros((64, 8)), B, np.zeros(64, np.int64)).any()
    total = np.zeros((32, 32))
    for pos, word in (((0, 1), 0b0100_0100_0100_0100), ((2, 3), 0b1110_1110_1110_1110)):
        A = np.zeros((64, 8))
        for l in range(64):
            h = l // 32
            for v in range(8):
                A[l, v] = Adense[l % 32, 16 * h + 4 * (v // 2) + pos[v % 2]]
        total += _model(A, B, np.full(64, word))
    Bfull = np.zeros((32, 32))
    for l in range(64):
        h = l // 32
        for k in range(16):
            Bfull[8 * h + k if k < 8 else 16 + 8 * h + (k - 8), l % 32] = B[l, k]
    assert np.array_equal(total, Adense @ Bfull)


@pytest.mark.gpu
@pytest.mark.parametrize("abid", [0, 1])
def test_sparse_f16_instruction_matches_the_host_model(abid):
    import torch
    lib = _probe()
    rng = np.random.default_rng(11 + abid)
    A = rng.integers(-4, 5, (64, 8)).astype(np.float16)
    B = rng.integers(-4, 5, (64, 16)).astype(np.float16)
    idx = rng.integers(0, 2**32, 64, dtype=np.uint64).astype(np.uint32)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(A).to(dev)
    b = torch.from_numpy(B).to(dev)
    i = torch.from_numpy(idx.view(np.int32)).to(dev)
    d = torch.zeros(64, 16, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.probe_smfmac(a.data_ptr(), b.data_ptr(), i.data_ptr(), d.data_ptr(), abid, stream) == 0
    torch.cuda.synchronize()
    got = _lanes(d.cpu().numpy().astype(np.float64))
    half = (idx >> 16) if abid else (idx & 0xFFFF)
    want = _model(A.astype(np.float64), B.astype(np.float64), half)
    assert np.array_equal(got, want)


@pytest.mark.gpu
def test_sparse_and_dense_f16_instruction_rates():
    """Dense-equivalent rate of the sparse instruction (32x32x32 per
    instruction) against the dense one (32x32x16), same loop shape; printed
    for the record.  The sparse one covers twice the K per instruction, so a
    ratio near 2 means it issues at about the dense instruction's rate."""
    import torch
    lib = _probe()
    dev = torch.device("cuda:0")
    a = torch.ones(64, 8, dtype=torch.float16, device=dev)
    b = torch.ones(64, 16, dtype=torch.float16, device=dev)
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rates = {}
    for sparse, k in ((1, 32), (0, 16)):
        best = 0.0
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert lib.probe_rate(sparse, a.data_ptr(), b.data_ptr(), out.data_ptr(), blocks, iters,
                                  ctypes.c_void_p(stream.cuda_stream)) == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            flops = blocks * 4 * iters * 4 * 2 * 32 * 32 * k
            best = max(best, flops / (ms * 1e-3) / 1e12)
        rates["sparse" if sparse else "dense"] = best
    ratio = rates["sparse"] / rates["dense"]
    print(f"f16 32x32: sparse {rates['sparse']:.0f} dense-equivalent TFLOP/s, dense {rates['dense']:.0f} "
          f"TFLOP/s, ratio {ratio:.2f}")
    assert np.isfinite(out[:256].cpu().numpy()).all()
    assert ratio > 1.0  # the sparse instruction covers more K per unit time than the dense one
