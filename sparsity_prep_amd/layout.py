"""Host-side views of the K-tiled FP4 operand layout (pure byte permutation).

Every code and scale array the library writes or reads is K-tiled: K is cut
into tiles of 128 elements (the last one narrower when K is not a multiple
of 128) and tile t holds all rows back to back, each row carrying the tile's
bytes -- w/2 code bytes or w/B scale bytes for a tile of width w.  These
helpers convert such an array to and from the plain row-major [rows, K/per]
form (per = 2 for codes, the block size B for scales), e.g. to inspect
prepared tensors or to compare them with a row-major reference.  They run on
the host with NumPy and play no part in the GPU path.
"""
import numpy as np

TILE_K = 128


def ktile_to_rows(buf, rows: int, K: int, per: int) -> np.ndarray:
    """K-tiled bytes (rows*K/per of them) -> row-major uint8 [rows, K/per]."""
    flat = np.asarray(buf, dtype=np.uint8).reshape(-1)
    if K % per or flat.size != rows * (K // per):
        raise ValueError("buffer size does not match rows x K / per")
    full, tb = K // TILE_K, TILE_K // per
    out = np.empty((rows, K // per), np.uint8)
    head = full * rows * tb
    if full:
        out[:, :full * tb] = flat[:head].reshape(full, rows, tb).transpose(1, 0, 2).reshape(rows, full * tb)
    if K - full * TILE_K:
        out[:, full * tb:] = flat[head:].reshape(rows, (K - full * TILE_K) // per)
    return out


def rows_to_ktile(arr, K: int, per: int) -> np.ndarray:
    """Row-major uint8 [rows, K/per] -> K-tiled bytes (flat)."""
    a = np.asarray(arr, dtype=np.uint8)
    rows = a.shape[0]
    if a.shape != (rows, K // per):
        raise ValueError("array shape does not match K / per")
    full, tb = K // TILE_K, TILE_K // per
    parts = []
    if full:
        parts.append(a[:, :full * tb].reshape(rows, full, tb).transpose(1, 0, 2).reshape(-1))
    if K - full * TILE_K:
        parts.append(a[:, full * tb:].reshape(-1))
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)
