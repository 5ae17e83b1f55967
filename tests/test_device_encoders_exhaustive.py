"""The library's device encoders against the oracle on every float32 input
of their domain: the E2M1 conversion (the gfx950 FP32 -> FP4 conversion
instruction with scale 1, followed by the canonical-zero fix; oracle:
nearest E2M1 value, ties to the even code, saturating at 6, zero magnitude
as code 0x0) on all 2^32 bit patterns (NaN inputs lie outside the method's
domain and are only counted), and the E4M3 block-scale encoder and MX
shared exponent on every non-negative finite float32."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "hwprobe", "libencoder_probe.so")
CHUNK = 1 << 26


@pytest.mark.gpu
def test_device_e2m1_matches_oracle_on_every_float32():
    import torch
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (python tests/hwprobe/build.py)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_e2m1.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_e2m1.restype = ctypes.c_int
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    low = np.arange(CHUNK, dtype=np.uint32)
    bad, nan_diff, nans = 0, 0, 0
    examples = []
    for c in range((1 << 32) // CHUNK):
        base = c * CHUNK
        rc = lib.probe_e2m1(base, CHUNK, ctypes.c_void_p(out.data_ptr()), stream)
        assert rc == 0, rc
        got = out.cpu().numpy()
        pats = low + np.uint32(base)
        u = pats.view(np.float32)
        want = oracle.e2m1_encode_array(u)
        diff = got != want
        isnan = np.isnan(u)
        nans += int(isnan.sum())
        nan_diff += int((diff & isnan).sum())
        d = np.flatnonzero(diff & ~isnan)
        bad += d.size
        examples += [(hex(int(pats[i])), int(got[i]), int(want[i])) for i in d[:3]]
        if c % 16 == 15:
            print(f"e2m1 exhaustive: {(c + 1) * CHUNK:#x} patterns, {bad} mismatches", flush=True)
    print(f"e2m1 exhaustive: NaN patterns {nans}, of which {nan_diff} coded differently", file=sys.stderr)
    assert bad == 0, examples[:10]


@pytest.mark.gpu
def test_device_scale_encoders_match_oracle_on_every_nonnegative_float32():
    """The NVFP4 block-scale encoder (nearest E4M3, ties to even, saturating
    at 448) and the MX shared exponent (floor(log2 amax) - 2, clamped at
    -127, zero giving -127) against the oracle on every non-negative finite
    float32, subnormals included (their domain: block maxima and their
    quotients)."""
    import torch
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (python tests/hwprobe/build.py)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_scales.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_scales.restype = ctypes.c_int
    e4 = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    e8 = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    end = 0x7F800000                     # +inf: the first non-finite pattern
    low = np.arange(CHUNK, dtype=np.uint32)
    bad4, bad8, examples = 0, 0, []
    for base in range(0, end, CHUNK):
        n = min(CHUNK, end - base)
        rc = lib.probe_scales(base, n, ctypes.c_void_p(e4.data_ptr()), ctypes.c_void_p(e8.data_ptr()), stream)
        assert rc == 0, rc
        got4, got8 = e4[:n].cpu().numpy(), e8[:n].cpu().numpy()
        pats = low[:n] + np.uint32(base)
        u = pats.view(np.float32)
        w4 = oracle.e4m3_encode_array(u)
        w8 = (oracle.mx_exponent_array(u) + 127).astype(np.uint8)
        d4, d8 = np.flatnonzero(got4 != w4), np.flatnonzero(got8 != w8)
        bad4 += d4.size
        bad8 += d8.size
        examples += [("e4m3", hex(int(pats[i])), int(got4[i]), int(w4[i])) for i in d4[:3]]
        examples += [("e8m0", hex(int(pats[i])), int(got8[i]), int(w8[i])) for i in d8[:3]]
        if (base // CHUNK) % 8 == 7:
            print(f"scale encoders: {base + n:#x} patterns, {bad4} + {bad8} mismatches", flush=True)
    assert bad4 == 0 and bad8 == 0, examples[:10]
