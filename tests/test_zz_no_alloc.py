"""The allocation-free preparation entry point (sharq_prepare_noalloc),
called through the C ABI, against sharq_prepare on the same inputs: every
prepared byte and the NVFP4 tensor scale must be identical.  Two calls in a
row, the second with fewer rows (its scratch array keeps the first call's
per-row statistics, which the second must not read)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from parity_util import dev16, prepared_to_host

pytestmark = pytest.mark.gpu

CASES = [  # (T, K, norm): the second call is smaller
    ((300, 1024, 1), (37, 512, 2)),
    ((2100, 4096, 1), (5, 4096, 0)),
]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("fmt", [0, 1], ids=["mxfp4", "nvfp4"])
@pytest.mark.parametrize("calls", CASES, ids=["small", "prefill"])
def test_noalloc_matches_prepare(fmt, calls):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparsity_prep_amd as sq
    L = sq.lib()
    for i, (T, K, norm) in enumerate(calls):
        tag = 900 + 10 * i + fmt
        x = dev16(synth.small_case(K, T, "bf16", outliers=3, dist="t" if fmt else "normal", tag=tag), "bf16")
        g = dev16(synth.small_gamma(K, "bf16", tag=tag), "bf16") if norm else None
        b = dev16(synth.small_gamma(K, "bf16", tag=tag + 1), "bf16") if norm == 2 else None
        ref = sq.prepare(x, norm=norm, gamma=g, beta=b, eps=1e-5, n=2, m=4, fmt=fmt)
        out = sq.alloc_prepared(T, K, fmt, x.device)
        for t in (out.b_codes, out.b_scales, out.r_codes, out.r_scales, out.mask):
            t.fill_(0x5A)
        if out.global_scale is not None:
            out.global_scale.fill_(-1.0)
        st = L.sharq_prepare_noalloc(_ptr(x), 1, T, K, x.stride(0), norm, _ptr(g), _ptr(b), 1e-5, 2, 4, fmt,
                                     _ptr(out.mask), _ptr(out.b_codes), _ptr(out.b_scales), _ptr(out.r_codes),
                                     _ptr(out.r_scales), _ptr(out.global_scale),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, L.sharq_status_string(st)
        torch.cuda.synchronize()
        got, want = prepared_to_host(out), prepared_to_host(ref)
        for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales", "G"):
            assert np.array_equal(got[key], want[key]), (i, T, K, key)
