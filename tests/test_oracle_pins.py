"""Pins for the CPU oracle: checks against what the formats, the pages and the
mathematics fix, each written differently from the oracle's own code path
(brute force, closed forms, invariants, hand-worked examples).

The pages (SharQ abstract) print no numbers for the operator, so the pins
come from: the OCP MX v1.0 element and scale definitions (E2M1 grid, E8M0
shared exponent floor(log2 amax) - 2), the E4M3 definition used by NVFP4,
the N:M selection definition, hand-worked rows under tests/golden/, and
algebraic invariants of the decomposition (masked-out residual equals the
normalized input, N = M reduces to plain round-to-nearest quantization,
zero in gives zero out, sign and power-of-two equivariance).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from golden_io import load as load_golden

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# ---------------------------------------------------------------- helpers (independent)

def nearest_grid_code(a: np.ndarray) -> np.ndarray:
    """Brute-force nearest E2M1 magnitude for a >= 0 (float64), ties to the even code.
    Magnitudes beyond 7 are clipped first (their nearest point is 6 either way)
    so that float64 distances stay exact."""
    d = np.abs(np.minimum(a, 7.0)[..., None] - GRID)
    m = d.min(-1, keepdims=True)
    cand = d == m
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(-1, keepdims=True), even, cand)
    return pick.argmax(-1)


def signed_code(v: np.ndarray, mag: np.ndarray) -> np.ndarray:
    neg = np.signbit(v) & (mag != 0)
    return (mag | (neg * 8)).astype(np.uint8)


def e4m3_table():
    """All non-negative finite E4M3 values by code, from the format definition
    (1 sign, 4 exponent bits with bias 7, 3 fraction bits, subnormals at
    exponent field 0, the all-ones pattern is NaN)."""
    vals = {}
    for code in range(0x7F):
        e, f = code >> 3, code & 7
        vals[code] = (f / 8.0) * 2.0 ** -6 if e == 0 else (1 + f / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = e4m3_table()
E4M3_CODES = np.array(sorted(E4M3))
E4M3_VALS = np.array([E4M3[c] for c in E4M3_CODES])


def e4m3_bruteforce(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 by exhaustive search, ties to the even code, values
    above the largest finite value saturate to it."""
    d = np.abs(np.minimum(x.astype(np.float64), 1000.0)[..., None] - E4M3_VALS)
    m = d.min(-1, keepdims=True)
    cand = d == m
    even = cand & (E4M3_CODES % 2 == 0)
    pick = np.where(even.any(-1, keepdims=True), even, cand)
    return E4M3_CODES[pick.argmax(-1)].astype(np.uint8)


def floor_log2(a: float) -> int:
    m, e = math.frexp(a)  # a = m * 2^e, 0.5 <= m < 1
    return e - 1


def textbook_mx(v: np.ndarray):
    """Plain OCP MX quantization of rows of float32 v: returns (codes, scale bytes, deq)."""
    rows, K = v.shape
    blk = v.reshape(rows, K // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(-1)
    _, ex = np.frexp(amax)
    E = np.clip(ex - 1 - 2, -127, 127)
    E = np.where(amax == 0, -127, E)
    u = blk / np.exp2(E)[..., None]
    mag = nearest_grid_code(np.abs(u))
    codes = signed_code(blk, mag).reshape(rows, K)
    deq = (np.where(np.signbit(blk) & (mag != 0), -1, 1) * GRID[mag] * np.exp2(E)[..., None])
    return codes, (E + 127).astype(np.uint8), deq.reshape(rows, K)


def textbook_nv(v: np.ndarray, G: float):
    """Plain NVFP4 quantization of rows of float32 v with tensor scale G."""
    rows, K = v.shape
    blk = v.reshape(rows, K // 16, 16).astype(np.float32)
    amax = np.abs(blk).max(-1)
    G32 = np.float32(G)
    t = (amax / (np.float32(6.0) * G32)).astype(np.float32)
    s = e4m3_bruteforce(t)
    sval = np.array([E4M3[int(c)] for c in s.reshape(-1)], np.float32).reshape(s.shape)
    D = (sval * G32).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(D[..., None] > 0, blk / D[..., None], 0).astype(np.float32)
    mag = nearest_grid_code(np.abs(u).astype(np.float64))
    codes = signed_code(blk, mag)
    mag_val = (GRID[mag].astype(np.float32) * D[..., None]).astype(np.float32)
    deq = np.where(codes & 8, -mag_val, mag_val).astype(np.float32)
    return codes.reshape(rows, K), s, deq.reshape(rows, K)


def unpack(p):
    return oracle.unpack_codes(p)


# ---------------------------------------------------------------- element formats

def test_e2m1_decode_is_the_ocp_grid():
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert abs(v) == GRID[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_e2m1_encode_matches_bruteforce():
    # every bf16 magnitude below 16, both signs
    bf = np.arange(0, 0x4180, dtype=np.uint32) << np.uint32(16)
    vals = [bf.view(np.float32), -bf.view(np.float32)]
    # +-4 ulps around every grid point and midpoint
    pts = np.array([0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 8], np.float32)
    for p in pts:
        b = p.view(np.uint32).astype(np.int64)
        vals.append(np.arange(b - 4, b + 5).astype(np.uint32).view(np.float32))
    rng = np.random.default_rng(1)
    vals.append(rng.uniform(-9, 9, 200_000).astype(np.float32))
    vals.append(synth.uniform_bits_f32(200_000, seed=2))
    u = np.concatenate(vals).astype(np.float32)
    got = oracle.e2m1_encode_array(u)
    want = signed_code(u, nearest_grid_code(np.abs(u.astype(np.float64))))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (u[bad[:5]], got[bad[:5]], want[bad[:5]])
    # ties go to the even code; negative zero and tiny negatives are canonical +0
    assert oracle.e2m1_encode(0.25) == 0 and oracle.e2m1_encode(0.75) == 2
    assert oracle.e2m1_encode(2.5) == 4 and oracle.e2m1_encode(5.0) == 6
    assert oracle.e2m1_encode(-0.0) == 0 and oracle.e2m1_encode(-0.2) == 0
    assert oracle.e2m1_encode(100.0) == 7 and oracle.e2m1_encode(-100.0) == 15


def test_mx_exponent_is_floor_log2_minus_2():
    assert oracle.mx_exponent(0.0) == -127
    for k in range(-149, 128):
        p = np.float32(2.0 ** k)
        for v in (p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(np.inf))):
            if not np.isfinite(v) or v == 0:
                continue
            want = min(max(floor_log2(float(v)) - 2, -127), 127)
            assert oracle.mx_exponent(float(v)) == want, (k, v)


def test_e4m3_decode_table():
    for code, val in E4M3.items():
        assert oracle.e4m3_decode(code) == val
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert np.all(np.diff(E4M3_VALS) > 0)


def test_e4m3_encode_matches_bruteforce():
    rng = np.random.default_rng(3)
    vals = [rng.uniform(0, 500, 100_000), np.exp2(rng.uniform(-12, 9.5, 100_000))]
    mids = (E4M3_VALS[1:] + E4M3_VALS[:-1]) / 2
    for mdp in mids.astype(np.float32):
        b = mdp.view(np.uint32).astype(np.int64)
        vals.append(np.arange(b - 2, b + 3).astype(np.uint32).view(np.float32))
    vals.append(np.array([0, 448, 449, 464, 480, 1e30, 2.0 ** -10, 2.0 ** -11], np.float32))
    x = np.concatenate([np.asarray(v, np.float32) for v in vals])
    got = oracle.e4m3_encode_array(x)
    want = e4m3_bruteforce(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


# ---------------------------------------------------------------- N:M selection

def brute_force_keep(v, n):
    """The unique size-n subset whose every kept element dominates every
    dropped one (larger magnitude, or equal magnitude and lower index)."""
    m = len(v)
    a = [abs(float(x)) for x in v]
    found = []
    for sub in itertools.combinations(range(m), n):
        dropped = [j for j in range(m) if j not in sub]
        if all(a[i] > a[j] or (a[i] == a[j] and i < j) for i in sub for j in dropped):
            found.append(sub)
    assert len(found) == 1
    keep = np.zeros(m, np.uint8)
    keep[list(found[0])] = 1
    return keep


def test_selection_matches_bruteforce_exhaustive_ties():
    for mags in itertools.product(range(4), repeat=4):
        for signs in itertools.product((1.0, -1.0), repeat=4):
            v = [s * m for s, m in zip(signs, mags)]
            for n in range(5):
                assert np.array_equal(oracle.select_group(v, n), brute_force_keep(v, n)), (v, n)


def test_selection_m8_random():
    rng = np.random.default_rng(4)
    for _ in range(300):
        v = rng.integers(-3, 4, 8).astype(np.float32) * np.float32(0.5)
        for n in range(9):
            assert np.array_equal(oracle.select_group(v, n), brute_force_keep(v, n))


# ---------------------------------------------------------------- hand-worked rows

@pytest.mark.parametrize("name", ["worked_mxfp4_2of4.txt", "worked_nvfp4_2of4.txt"])
def test_golden_worked_rows(name):
    g = load_golden(name)
    p = oracle.prepare(g["x"], g["dtype"], g["K"], g["norm"], None, None, g["eps"],
                       g["N"], g["M"], g["fmt"])
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
        assert np.array_equal(getattr(p, key), g[key]), (key, getattr(p, key), g[key])
    assert p.G == g["gscale"]


def test_residual_is_against_quantized_backbone():
    """A residual taken against the unquantized sparse values would be zero at
    the kept positions of the worked row; SharQ's is not."""
    g = load_golden("worked_mxfp4_2of4.txt")
    p = oracle.prepare(g["x"], g["dtype"], g["K"], 0, None, None, 0.0, 2, 4, 0, trace=True)
    keep = oracle.unpack_mask(p.mask)[0]
    assert np.any(p.resid[0][keep] != 0)
    assert np.array_equal(p.resid[0], (p.xhat[0] - p.deqb[0]).astype(np.float32))


# ---------------------------------------------------------------- decomposition invariants

def _case(K=256, T=12, dtype="bf16", dist="normal", tag=0, outliers=4):
    x = synth.small_case(K, T, dtype, seed=0, outliers=outliers, dist=dist, tag=tag)
    g = synth.small_gamma(K, dtype, tag=tag)
    return x, g


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("nm", [(2, 4), (1, 4), (4, 8), (1, 2), (3, 4), (8, 16)])
def test_invariants(fmt, nm):
    n, m = nm
    K = 256
    x, g = _case(K, tag=n * 100 + m)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5, n, m, fmt, trace=True)
    keep = oracle.unpack_mask(p.mask)
    # exactly N survivors per group of M
    assert np.all(keep.reshape(keep.shape[0], -1, m).sum(-1) == n)
    # masked-out residual is the normalized input, bit for bit
    assert np.array_equal(p.resid.view(np.uint32)[~keep], p.xhat.view(np.uint32)[~keep])
    # backbone values are the normalized values at kept positions, +0 elsewhere
    # (checked through its quantization: backbone scale equals plain RTN scale of xhat)
    if fmt == 0:
        _, sc_rtn, _ = textbook_mx(p.xhat)
        assert np.array_equal(p.b_scales, sc_rtn)
        # residual reconstruction bound: |xhat - deq_b - deq_r| <= 2 * 2^E_r
        dr = p.deq_residual()
        err = np.abs(p.xhat.astype(np.float64) - p.deqb.astype(np.float64) - dr)
        Er = p.r_scales.astype(np.float64) - 127
        bound = 2.0 * np.exp2(np.repeat(Er, 32, axis=1))
        assert np.all(err <= bound)
        # kept elements: |R| <= 2 * 2^E_backbone
        Eb = np.repeat(p.b_scales.astype(np.float64) - 127, 32, axis=1)
        assert np.all(np.abs(p.resid[keep]) <= 2.0 * np.exp2(Eb[keep]))
    # dequantized backbone is zero wherever the mask dropped the element
    assert np.all(p.deq_backbone()[~keep] == 0)


def test_n_equals_m_is_plain_mx_rtn():
    K = 512
    x, g = _case(K, tag=7)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5, 4, 4, 0, trace=True)
    assert np.all(oracle.unpack_mask(p.mask))
    codes, sc, deq = textbook_mx(p.xhat)
    assert np.array_equal(unpack(p.b_codes), codes)
    assert np.array_equal(p.b_scales, sc)
    assert np.array_equal(p.deq_backbone(), deq)
    rc, rs, _ = textbook_mx((p.xhat - deq).astype(np.float32))
    assert np.array_equal(unpack(p.r_codes), rc)
    assert np.array_equal(p.r_scales, rs)


def test_n_equals_m_is_plain_nvfp4():
    K = 256
    x, g = _case(K, dist="t", tag=8)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-6, 4, 4, 1, trace=True)
    G = float(np.float32(np.abs(p.xhat).max()) / np.float32(2688.0))
    assert p.G == np.float32(G)
    codes, s, deq = textbook_nv(p.xhat, p.G)
    assert np.array_equal(unpack(p.b_codes), codes)
    assert np.array_equal(p.b_scales, s)
    assert np.array_equal(p.deqb, deq)
    rc, rs, _ = textbook_nv((p.xhat - deq).astype(np.float32), p.G)
    assert np.array_equal(unpack(p.r_codes), rc)
    assert np.array_equal(p.r_scales, rs)


@pytest.mark.parametrize("fmt", [0, 1])
def test_zero_input_gives_zero(fmt):
    K = 128
    x = np.zeros((4, K), np.uint16)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, synth.small_gamma(K), None, 1e-5, 2, 4, fmt)
    assert not p.b_codes.any() and not p.r_codes.any()
    if fmt == 0:
        assert not p.b_scales.any() and not p.r_scales.any()
    w = oracle.quantize_weight(synth.small_weight(8, K), "bf16", fmt)
    assert np.all(oracle.linear(p, w) == 0)


def test_power_of_two_and_sign_equivariance():
    K = 256
    x, _ = _case(K, tag=9)
    xf = synth.bits_to_f32(x, "bf16")
    p0 = oracle.prepare(x, "bf16", K, oracle.NORM_NONE, None, None, 0.0, 2, 4, 0)
    for j in (-5, 3):
        xj = synth.to_bits(xf * np.float32(2.0 ** j), "bf16")
        pj = oracle.prepare(xj, "bf16", K, oracle.NORM_NONE, None, None, 0.0, 2, 4, 0)
        assert np.array_equal(pj.mask, p0.mask)
        assert np.array_equal(pj.b_codes, p0.b_codes) and np.array_equal(pj.r_codes, p0.r_codes)
        assert np.array_equal(pj.b_scales.astype(int), p0.b_scales.astype(int) + j)
        assert np.array_equal(pj.r_scales.astype(int), p0.r_scales.astype(int) + j)
    xn = synth.to_bits(-xf, "bf16")
    pn = oracle.prepare(xn, "bf16", K, oracle.NORM_NONE, None, None, 0.0, 2, 4, 0)
    assert np.array_equal(pn.mask, p0.mask)
    assert np.array_equal(pn.b_scales, p0.b_scales) and np.array_equal(pn.r_scales, p0.r_scales)
    for a, b in ((pn.b_codes, p0.b_codes), (pn.r_codes, p0.r_codes)):
        ca, cb = unpack(a), unpack(b)
        assert np.array_equal(ca & 7, cb & 7)
        nz = (cb & 7) != 0
        assert np.array_equal((ca ^ cb)[nz], np.full(nz.sum(), 8, np.uint8))


# ---------------------------------------------------------------- norms

def test_rmsnorm_close_to_textbook():
    K = 384
    x, g = _case(K, tag=10)
    xh = oracle.normalize(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5)
    xf = synth.bits_to_f32(x, "bf16").astype(np.float64)
    gf = synth.bits_to_f32(g, "bf16").astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(1, keepdims=True) + np.float64(np.float32(1e-5))) * gf
    assert np.max(np.abs(xh - ref) / np.maximum(np.abs(ref), 1e-30)) < 3 * 2.0 ** -24


def test_layernorm_close_to_textbook():
    K = 256
    x, g = _case(K, tag=11)
    b = synth.small_gamma(K, tag=12)
    xh = oracle.normalize(x, "bf16", K, oracle.NORM_LAYER, g, b, 1e-5)
    xf = synth.bits_to_f32(x, "bf16").astype(np.float64)
    gf = synth.bits_to_f32(g, "bf16").astype(np.float64)
    bf = synth.bits_to_f32(b, "bf16").astype(np.float64)
    mu = xf.mean(1, keepdims=True)
    ref = (xf - mu) / np.sqrt(((xf - mu) ** 2).mean(1, keepdims=True) + np.float64(np.float32(1e-5))) * gf + bf
    assert np.max(np.abs(xh - ref)) < 1e-5 * np.max(np.abs(ref))


def test_fp16_decode_exact():
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    xh = oracle.normalize(h.reshape(1, -1)[:, :31744], "f16", 31744, oracle.NORM_NONE, None, None, 0)
    assert np.array_equal(xh[0], h[:31744].view(np.float16).astype(np.float32))


# ---------------------------------------------------------------- layer product

def _tiny_prod(prep, wq):
    """Triple loop over explicitly decoded nibbles (no oracle dequant)."""
    def decode_rows(codes, scales, K, G, fmt):
        B = 32 if fmt == 0 else 16
        out = np.zeros((codes.shape[0], K))
        for r in range(codes.shape[0]):
            for k in range(K):
                byte = int(codes[r, k // 2])
                c = (byte >> 4) if k % 2 else (byte & 15)
                v = GRID[c & 7] * (-1 if c & 8 else 1)
                s = int(scales[r, k // B])
                out[r, k] = v * (2.0 ** (s - 127) if fmt == 0 else E4M3[s] * G)
        return out
    K = prep.K
    a = decode_rows(prep.b_codes, prep.b_scales, K, prep.G, prep.fmt)
    r = decode_rows(prep.r_codes, prep.r_scales, K, prep.G, prep.fmt)
    w = decode_rows(wq.codes[0], wq.scales[0], K, float(wq.gscale[0]), wq.fmt)
    y = np.zeros((a.shape[0], w.shape[0]))
    for t in range(a.shape[0]):
        for n in range(w.shape[0]):
            s = 0.0
            for k in range(K):
                s += a[t, k] * w[n, k] + r[t, k] * w[n, k]
            y[t, n] = s
    return y


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_matches_triple_loop(fmt):
    K, T, NO = 64, 3, 5
    x, g = _case(K, T=T, tag=13)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5, 2, 4, fmt)
    wq = oracle.quantize_weight(synth.small_weight(NO, K, tag=13), "bf16", fmt)
    y = oracle.linear(p, wq)
    ref = _tiny_prod(p, wq)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_linear_permutation_weight_returns_reconstruction():
    """W with a single 1 per row picks one column of deq(backbone)+deq(residual)."""
    K = 128
    x, g = _case(K, T=6, tag=14)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5, 2, 4, 0)
    perm = np.random.default_rng(5).permutation(K)
    w = np.zeros((K, K), np.float32)
    w[np.arange(K), perm] = 1.0
    wq = oracle.quantize_weight(synth.to_bits(w, "bf16"), "bf16", 0)
    assert np.array_equal(oracle.dequant(wq.codes[0], wq.scales[0], K, 0), w.astype(np.float64))
    y = oracle.linear(p, wq)
    rec = p.deq_backbone() + p.deq_residual()
    assert np.array_equal(y, rec[:, perm])


@pytest.mark.parametrize("fmt", [0, 1])
def test_weight_quantization_is_plain_rtn(fmt):
    K, NO = 256, 16
    wb = synth.small_weight(NO, K, tag=15)
    wq = oracle.quantize_weight(wb, "bf16", fmt)
    wf = synth.bits_to_f32(wb[0], "bf16")
    if fmt == 0:
        codes, sc, _ = textbook_mx(wf)
    else:
        G = float(np.float32(np.abs(wf).max()) / np.float32(2688.0))
        assert wq.gscale[0] == np.float32(G)
        codes, sc, _ = textbook_nv(wf, float(wq.gscale[0]))
    assert np.array_equal(unpack(wq.codes[0]), codes)
    assert np.array_equal(wq.scales[0], sc)


def test_grouped_linear_matches_per_expert():
    K, NO, E = 64, 8, 3
    x, g = _case(K, T=10, tag=16)
    p = oracle.prepare(x, "bf16", K, oracle.NORM_RMS, g, None, 1e-5, 2, 4, 0)
    wq = oracle.quantize_weight(synth.small_weight(NO, K, experts=E, tag=16), "bf16", 0)
    offsets = np.array([0, 4, 4, 9], np.int32)
    ridx = np.array([3, 1, 0, 9, 2, 2, 5, 6, 7], np.int32)
    y = oracle.linear_grouped(p, wq, offsets, ridx)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            sub = oracle.Prepared(1, K, 0)
            for key in ("b_codes", "b_scales", "r_codes", "r_scales"):
                getattr(sub, key)[:] = getattr(p, key)[ridx[r]]
            sub.gscale[:] = p.gscale
            assert np.array_equal(y[r], oracle.linear(sub, wq, expert=e)[0])


# ---------------------------------------------------------------- SiLU(gate) * up
# The down projection's input is SiLU(gate) * up; its fused preparation is
# defined with a float exponential built from fixed IEEE steps (so the GPU and
# the oracle can reproduce it bit for bit).  Pins: the mathematics of exp and
# SiLU within a few ulp, and the column convention of the gate/up rows.

def _ulp(v: float) -> float:
    return float(np.spacing(np.float32(abs(v)))) if v != 0 else float(np.finfo(np.float32).smallest_subnormal)


def test_exp32_against_the_exponential():
    ys = np.concatenate([np.linspace(-87.0, 88.0, 20001, dtype=np.float32),
                         np.array([0.0, 1e-30, -1e-30, 0.5, -0.5, 1.0, -1.0, 20.0, -20.0], np.float32)])
    for y in ys:
        got, ref = oracle.exp32(float(y)), math.exp(float(y))
        assert abs(got - ref) <= 4 * _ulp(ref), (float(y), got, ref)
    assert oracle.exp32(0.0) == 1.0
    assert oracle.exp32(-87.5) == 0.0 and math.isinf(oracle.exp32(88.5))


def test_silu32_against_its_definition():
    for g in np.linspace(-40.0, 40.0, 8001, dtype=np.float32):
        got, ref = oracle.silu32(float(g)), float(g) / (1.0 + math.exp(-float(g)))
        assert abs(got - ref) <= 4 * _ulp(ref) + 1e-37, (float(g), got, ref)
    assert oracle.silu32(0.0) == 0.0
    assert oracle.silu32(100.0) == 100.0                       # e^-100 is below the range: exactly g
    assert oracle.silu32(-100.0) == 0.0 and math.copysign(1.0, oracle.silu32(-100.0)) < 0  # g / inf = -0


@pytest.mark.parametrize("fmt", [oracle.FMT_MXFP4, oracle.FMT_NVFP4])
def test_prepare_swiglu_is_prepare_of_the_product(fmt):
    rng = np.random.default_rng(5 + fmt)
    T, K, ld = 6, 256, 2 * 256 + 32
    gu = (rng.standard_normal((T, ld)) * 3.0).astype(np.float32)
    gu[:, 7] *= 20.0
    x = np.empty((T, K), np.float32)
    for t in range(T):
        for k in range(K):
            x[t, k] = np.float32(oracle.silu32(float(gu[t, k]))) * gu[t, K + k]
    a = oracle.prepare_swiglu(gu, K, 2, 4, fmt, trace=True)
    b = oracle.prepare(x, "f32", K, oracle.NORM_NONE, None, None, 0.0, 2, 4, fmt)
    assert np.array_equal(a.xhat.view(np.uint32), x.view(np.uint32))
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales", "gscale"):
        assert np.array_equal(getattr(a, key), getattr(b, key)), key


def test_prepare_swiglu_column_convention():
    """gate = 100 gives SiLU = 100 exactly, gate = 0 gives 0: the activation
    is 100*up and 0*up; swapping gate and up would change both."""
    K = 64
    up = np.linspace(-3.0, 3.0, K, dtype=np.float32)
    gu = np.zeros((2, 2 * K), np.float32)
    gu[0, :K] = 100.0
    gu[0, K:] = up
    gu[1, K:] = up
    a = oracle.prepare_swiglu(gu, K, 2, 4, oracle.FMT_MXFP4, trace=True)
    assert np.array_equal(a.xhat[0], np.float32(100.0) * up)
    assert np.array_equal(a.xhat[1].view(np.uint32), (np.float32(0.0) * up).view(np.uint32))


# ---------------------------------------------------------------- sampled-row entry points
# The full-size GPU checks compare sampled rows: a sample of weight rows
# quantized with the weight's own tensor scale (quantize_rows), and a subset
# of activation rows (prepare / prepare_swiglu with rows=...), where the NVFP4
# tensor scale must still come from every row of the tensor.

@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_rows_is_plain_rtn(fmt):
    K, NO = 512, 24
    wb = synth.small_weight(NO, K, tag=61)[0]
    wf = synth.bits_to_f32(wb, "bf16")
    rows = np.array([17, 0, 5, 5, 23, 11])
    G = 1.0
    if fmt == 1:
        G = float(np.float32(np.abs(wf).max()) / np.float32(2688.0))  # the whole weight's scale
    c, s = oracle.quantize_rows(wb[rows], "bf16", fmt, G)
    if fmt == 0:
        codes, sc, _ = textbook_mx(wf[rows])
    else:
        codes, sc, _ = textbook_nv(wf[rows], G)
    assert np.array_equal(unpack(c), codes)
    assert np.array_equal(s, sc)
    # and the same bytes as those rows of the whole-weight payload
    wq = oracle.quantize_weight(wb, "bf16", fmt)
    assert np.float32(G) == wq.gscale[0]
    assert np.array_equal(c, wq.codes[0][rows])
    assert np.array_equal(s, wq.scales[0][rows])


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("norm", [oracle.NORM_RMS, oracle.NORM_LAYER, oracle.NORM_NONE])
def test_prepare_row_subset(fmt, norm):
    K, T = 256, 40
    x, g = _case(K, T=T, dist="t" if fmt else "normal", tag=62 + norm)
    beta = synth.small_gamma(K, "bf16", tag=70) if norm == oracle.NORM_LAYER else None
    gam = g if norm != oracle.NORM_NONE else None
    xf = synth.bits_to_f32(x, "bf16")
    hot = int(np.argmax(np.abs(xf).max(1)))
    # out of order, repeated, and without the row that holds the largest value
    rows = np.array([t for t in (39, 3, 3, 0, 21, 38, 7) if t != hot])
    full = oracle.prepare(x, "bf16", K, norm, gam, beta, 1e-5, 2, 4, fmt, trace=True)
    sub = oracle.prepare(x, "bf16", K, norm, gam, beta, 1e-5, 2, 4, fmt, rows=rows, trace=True)
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales", "xhat", "deqb", "resid"):
        assert np.array_equal(getattr(sub, key), getattr(full, key)[rows]), key
    assert sub.G == full.G
    if fmt == 1:
        # NVFP4: the tensor scale is the whole tensor's amax / 2688 (textbook),
        # not the subset's, and the subset's codes follow the textbook quantizer
        G = float(np.float32(np.abs(full.xhat).max()) / np.float32(2688.0))
        assert sub.G == np.float32(G)
        assert np.abs(sub.xhat).max() < np.abs(full.xhat).max()
        S = np.where(oracle.unpack_mask(sub.mask), sub.xhat, np.float32(0)).astype(np.float32)
        codes, s, _ = textbook_nv(S, sub.G)
        assert np.array_equal(unpack(sub.b_codes), codes)
        assert np.array_equal(sub.b_scales, s)
    else:
        # MXFP4 has no tensor-level coupling: each row alone gives the same bytes
        for i, t in enumerate(rows):
            one = oracle.prepare(x[t:t + 1], "bf16", K, norm, gam, beta, 1e-5, 2, 4, fmt)
            for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
                assert np.array_equal(getattr(one, key)[0], getattr(sub, key)[i]), (key, t)


@pytest.mark.parametrize("fmt", [0, 1])
def test_prepare_swiglu_row_subset(fmt):
    K, T = 128, 24
    gu = synth.small_gate_up(K, T, tag=63 + fmt)
    rows = np.array([23, 1, 1, 12])
    full = oracle.prepare_swiglu(gu, K, 2, 4, fmt, trace=True)
    sub = oracle.prepare_swiglu(gu, K, 2, 4, fmt, rows=rows, trace=True)
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales", "xhat"):
        assert np.array_equal(getattr(sub, key), getattr(full, key)[rows]), key
    assert sub.G == full.G
    if fmt == 1:
        assert full.G == np.float32(np.float32(np.abs(full.xhat).max()) / np.float32(2688.0))


# ---------------------------------------------------------------- compressed 2:4 backbone (NVFP4_SP24)

def _sp24_case(T, K, seed):
    x = synth.small_case(K, T, "bf16", outliers=3, mult=40.0, tag=seed)
    g = synth.small_gamma(K, "bf16", tag=seed + 1)
    return oracle.prepare(x, "bf16", K, 1, g, None, 1e-5, 2, 4, oracle.FMT_NVFP4)


def test_sp24_pack_round_trip():
    """Unpacking the compressed backbone gives back the dense backbone codes
    and the mask, and its scales are a permutation of each tile's eight."""
    p = _sp24_case(7, 384, 21)
    rec, sc = oracle.sp24_pack(p)
    assert rec.shape == (7, 3, 48) and sc.shape == p.b_scales.shape
    codes, mask = oracle.sp24_unpack(rec, 384)
    assert np.array_equal(codes, p.b_codes) and np.array_equal(mask, p.mask)
    assert np.array_equal(np.sort(sc.reshape(7, 3, 8), -1), np.sort(p.b_scales.reshape(7, 3, 8), -1))


def test_sp24_pack_feeds_the_sparse_instruction():
    """The compressed backbone, read the way the product reads it (in
    sub-step p, lane half h takes chunk (p, h, u) with index half u; the
    weight lane of half h' takes elements 32(2h' + p) + 16u + [0, 16) of its
    row), and multiplied by the host model of the 2:4 sparse f16 instruction,
    gives the dense product of the backbone codes over the tile's 128
    elements; each (p, u) covers elements 32p + 16u + [0, 16) and
    64 + 32p + 16u + [0, 16)."""
    from smfmac_model import model
    p = _sp24_case(32, 128, 33)
    rec, _ = oracle.sp24_pack(p)
    grid = np.array([oracle.e2m1_decode(c) for c in range(16)])
    bb = grid[oracle.unpack_codes(p.b_codes)]           # [32, 128] backbone code values
    rng = np.random.default_rng(4)
    w = rng.integers(-3, 4, (32, 128)).astype(np.float64)  # 32 weight rows of one tile
    total = np.zeros((32, 32))
    for pp in (0, 1):
        for u in (0, 1):
            A = np.zeros((64, 8))
            idx = np.zeros(64, np.int64)
            Bl = np.zeros((64, 16))
            for l in range(64):
                row, h = l % 32, l // 32
                c = 4 * pp + 2 * h + u
                for v in range(8):
                    A[l, v] = grid[(rec[row, 0, 4 * c + v // 2] >> (4 * (v % 2))) & 0xF]
                word = int.from_bytes(bytes(rec[row, 0, 32 + 4 * (2 * pp + h):36 + 4 * (2 * pp + h)]), "little")
                idx[l] = (word >> (16 * u)) & 0xFFFF
                Bl[l] = w[l % 32, 32 * (2 * h + pp) + 16 * u + np.arange(16)]
            D = model(A, Bl, idx)
            cols = np.concatenate([32 * pp + 16 * u + np.arange(16), 64 + 32 * pp + 16 * u + np.arange(16)])
            assert np.array_equal(D, bb[:, cols] @ w[:, cols].T), (pp, u)
            total += D
    assert np.array_equal(total, bb @ w.T)


def test_sp24_pack_needs_a_2of4_mask():
    x = synth.small_case(128, 3, "bf16", outliers=1, mult=10.0, tag=2)
    g = synth.small_gamma(128, "bf16", tag=2)
    p = oracle.prepare(x, "bf16", 128, 1, g, None, 1e-5, 1, 4, oracle.FMT_NVFP4)
    with pytest.raises(ValueError):
        oracle.sp24_pack(p)
