"""Host model of gfx950's 2:4 sparse f16 matrix instruction
v_smfmac_f32_32x32x32_f16 (D = A * B, 32x32 output), shared by the
instruction probe and the pins of the compressed backbone layout.

  A, lane l: row l % 32, eight values v = 0..7, the kept values of K
     positions 16h .. 16h + 15 (h = l / 32): value v lies in group v // 2 at
     position p = bits 2v, 2v+1 of the 16-bit index half (abid 0: bits 0-15 of
     the index word, abid 1: bits 16-31), i.e. at K = 16h + 4(v // 2) + p;
  B, lane l: column l % 32, halves 0..7 at K = 8h + k, halves 8..15 at
     K = 16 + 8h + (k - 8);
  D, lane l, register r: row 8(r // 4) + 4h + r % 4, column l % 32."""
import numpy as np


def model(A, B, idx16):
    """D [32, 32] from A [64 lanes, 8], B [64 lanes, 16], idx16 [64] (the
    selected 16-bit index half of each lane)."""
    Ad = np.zeros((32, 32))
    for l in range(64):
        h = l // 32
        for v in range(8):
            p = (int(idx16[l]) >> (2 * v)) & 3
            Ad[l % 32, 16 * h + 4 * (v // 2) + p] += A[l, v]
    Bd = np.zeros((32, 32))
    for l in range(64):
        h = l // 32
        for k in range(16):
            K = 8 * h + k if k < 8 else 16 + 8 * h + (k - 8)
            Bd[K, l % 32] = B[l, k]
    return Ad @ Bd


def lanes_to_matrix(D):
    """D [32, 32] from the per-lane accumulators D [64 lanes, 16]."""
    M = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            M[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = D[l, r]
    return M
