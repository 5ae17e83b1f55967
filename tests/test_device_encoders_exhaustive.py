"""The library's device encoders against the oracle on every float32 input
of their domain: the E2M1 conversion (the gfx950 FP32 -> FP4 conversion
instruction with scale 1, followed by the canonical-zero fix; oracle:
nearest E2M1 value, ties to the even code, saturating at 6, zero magnitude
as code 0x0) on all 2^32 bit patterns (NaN inputs lie outside the method's
domain and are only counted), the E4M3 block-scale encoder and MX
shared exponent on every non-negative finite float32, the device SiLU on
all 2^32 patterns, and the NVFP4 element quotient against float division on
quotients next to the float midpoints."""
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


@pytest.mark.gpu
def test_device_silu_matches_oracle_on_every_float32():
    """SiLU(g) = g / (1 + e^-g) of the library's device code against the
    oracle on all 2^32 float32 patterns g: the function the SwiGLU epilogue
    and the SiLU(gate)*up prep call (silu_times_n, which takes a shorter
    instruction sequence when a wave's values all lie in [-80, 80]), and that
    short sequence itself on every g of the range (the hardware reciprocal
    and one remainder correction in place of the division routine: exact for
    these divisors only, which this test is what shows).  Equal bit patterns are required, NaN results only have to be
    NaN on both sides (their payloads are not part of the definition)."""
    import concurrent.futures as cf
    import torch
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (python tests/hwprobe/build.py)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_silu.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_silu.restype = ctypes.c_int
    outs = [torch.empty(CHUNK, dtype=torch.float32, device="cuda") for _ in range(2)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    low = np.arange(CHUNK, dtype=np.uint32)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    bad, examples = [0, 0], []
    with cf.ThreadPoolExecutor(workers) as ex:
        for c in range((1 << 32) // CHUNK):
            base = c * CHUNK
            for mode in (0, 1):
                rc = lib.probe_silu(base, CHUNK, mode, ctypes.c_void_p(outs[mode].data_ptr()), stream)
                assert rc == 0, rc
            g = (low + np.uint32(base)).view(np.float32)
            want = np.concatenate(list(ex.map(oracle.silu32_array, np.array_split(g, workers))))
            wnan = np.isnan(want)
            for mode in (0, 1):
                got = outs[mode].cpu().numpy()
                ok = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & wnan)
                d = np.flatnonzero(~ok)
                bad[mode] += d.size
                examples += [(mode, hex(int(g.view(np.uint32)[i])), float(got[i]), float(want[i])) for i in d[:3]]
            if c % 16 == 15:
                print(f"silu exhaustive: {(c + 1) * CHUNK:#x} patterns, mismatches {bad}", flush=True)
    assert bad == [0, 0], examples[:10]


def _near_midpoint_pairs(rng, n):
    """Float pairs (x, d), d > 0, whose quotients lie as close as floats allow
    to the midpoints between adjacent floats (x = fl32(mid * d) and its two
    neighbours), divisors across the subnormal and normal range."""
    xs, ds = [], []
    for lo, hi in ((-149, -126), (-126, 0), (0, 127)):
        d = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(lo, hi, n)).astype(np.float32)
        d = d[(d > 0) & np.isfinite(d)]
        q = (rng.uniform(1, 2, d.size) * 2.0 ** rng.integers(-12, 10, d.size)).astype(np.float32)
        mid = (q.astype(np.float64) + np.nextafter(q, np.float32(np.inf)).astype(np.float64)) / 2
        with np.errstate(over="ignore"):
            x = (mid * d.astype(np.float64)).astype(np.float32)
        for xx in (x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))):
            keep = np.isfinite(xx)
            xs.append(np.where(rng.random(xx.size) < 0.5, xx, -xx)[keep])
            ds.append(d[keep])
    return np.concatenate(xs), np.concatenate(ds)


@pytest.mark.gpu
def test_device_nvfp4_quotient_matches_float_division():
    """The NVFP4 element quotient as the prep kernels form it,
    float(double(x) * r) with r the hardware double reciprocal of the
    positive float divisor refined by two Newton steps, against IEEE float
    division (numpy's, correctly rounded: the definition) on quotients next to
    the float midpoints, where a reciprocal off by more than the argument
    allows would show, and on random pairs with positive finite divisors and
    quotients in the normal range or zero."""
    import torch
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (python tests/hwprobe/build.py)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_quotient.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.probe_quotient.restype = ctypes.c_int
    rng = np.random.default_rng(7)
    x0, d0 = _near_midpoint_pairs(rng, 1_000_000)
    bits = rng.integers(0, 2 ** 32, size=(2, 4_000_000), dtype=np.uint64).astype(np.uint32)
    x1, d1 = bits[0].view(np.float32), np.abs(bits[1].view(np.float32))
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        q64 = np.abs(x1.astype(np.float64) / d1.astype(np.float64))
    # quotients below the normal float range are left out: on the subnormal
    # grid an exact tie can part from a reciprocal-based product, but every
    # such quotient lies far below the smallest E2M1 step (0.25) and
    # quantizes to zero either way
    ok = np.isfinite(x1) & np.isfinite(d1) & (d1 > 0) & ((q64 == 0) | (q64 >= 2.0 ** -126))
    x = np.concatenate([x0, x1[ok]]).astype(np.float32)
    d = np.concatenate([d0, d1[ok]]).astype(np.float32)
    assert x.size > 9_000_000
    xt, dt = torch.from_numpy(x).cuda(), torch.from_numpy(d).cuda()
    qt = torch.empty_like(xt)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.probe_quotient(ctypes.c_void_p(xt.data_ptr()), ctypes.c_void_p(dt.data_ptr()), x.size,
                            ctypes.c_void_p(qt.data_ptr()), stream)
    assert rc == 0, rc
    got = qt.cpu().numpy()
    with np.errstate(over="ignore", under="ignore"):
        want = np.divide(x, d, dtype=np.float32)
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, [(float(x[i]), float(d[i]), float(got[i]), float(want[i])) for i in bad[:5]]
