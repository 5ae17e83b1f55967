"""The library's device E2M1 conversion (the gfx950 FP32 -> FP4 conversion
instruction with scale 1, followed by the canonical-zero fix) against the
oracle's encoder (nearest E2M1 value, ties to the even code, saturating at
6, zero magnitude as code 0x0) on every one of the 2^32 float32 bit
patterns.  NaN inputs lie outside the method's domain and are only counted."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "hwprobe", "libe2m1_probe.so")
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
