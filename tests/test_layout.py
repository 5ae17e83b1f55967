"""K-tiled FP4 operand layout: the host views against the layout's own
definition (element k of row r, tile t = floor(k/128) of width w_t, sits at
byte t*rows*(128/P) + r*(w_t/P) + (k mod 128)/P, P = 2 for codes, the block
size for scales), written out element by element."""
import numpy as np
import pytest

from sparsity_prep_amd.layout import ktile_to_rows, rows_to_ktile

CASES = [(1, 128, 2), (3, 256, 2), (5, 384, 32), (7, 96, 2), (4, 2080, 2), (6, 2080, 32),
         (2, 48, 16), (9, 2064, 16), (1, 64, 2), (33, 800, 32), (4, 5152, 16)]


def byte_index(r, k, rows, K, per):
    t = k // 128
    w = min(128, K - 128 * t)
    return t * rows * (128 // per) + r * (w // per) + (k % 128) // per


@pytest.mark.parametrize("rows,K,per", CASES)
def test_ktile_matches_definition(rows, K, per):
    rng = np.random.default_rng(rows * 10007 + K + per)
    a = rng.integers(0, 256, size=(rows, K // per), dtype=np.uint8)
    flat = rows_to_ktile(a, K, per)
    assert flat.shape == (rows * K // per,)
    seen = np.zeros(flat.size, bool)
    for r in range(rows):
        for j in range(K // per):
            i = byte_index(r, j * per, rows, K, per)
            assert flat[i] == a[r, j]
            seen[i] = True
    assert seen.all()  # a permutation: every byte written exactly once
    assert np.array_equal(ktile_to_rows(flat, rows, K, per), a)


def test_ktile_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        ktile_to_rows(np.zeros(10, np.uint8), 3, 128, 2)
    with pytest.raises(ValueError):
        rows_to_ktile(np.zeros((3, 10), np.uint8), 128, 2)
