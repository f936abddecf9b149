"""Bitmap-compressed unstructured sparsity (the Coruscant sparse format) and its product.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU baseline.

Source
------
"Coruscant: Co-Designing GPU Kernel and Sparse Tensor Core ..." (the page is a
Chinese summary), Sec. 3.1 and Fig. 7: the matrix is cut into tiles of 64
elements; each tile is stored as its non-zero values plus a 64-bit bitmap of
where they sit, and a tile-offset array points at the first non-zero of each
tile. Sec. 3.2 (other optimisations): each tile's non-zeros are padded to a
multiple of 8 so that one 128-bit load serves them. Sec. 3.1 gives the
resulting sizes: 56.25 % of the dense fp16 matrix at 50 % sparsity and
36.25 % at 70 % (values + bitmaps).

Readings where the pages are silent
-----------------------------------
* Tile orientation: a tile is 64 consecutive positions along K in one row
  (the page's tiles run down a column, to suit its shared-memory banks; the
  content -- bitmap + packed values + offsets -- is the same). K % 64 == 0.
* "Non-zero" means any value whose magnitude bits are not all zero: +0 and -0
  are both zeros and are not stored (so -0 decodes as +0).
* Values are packed in ascending position order; the padding values are +0.
* tile_offsets holds R*(K/64) + 1 uint32 entries: the exclusive prefix sum of
  the padded counts in row-major tile order, then the total.
"""
from __future__ import annotations

import numpy as np

TILE = 64


def _nonzero(a16: np.ndarray) -> np.ndarray:
    return (np.asarray(a16, dtype=np.float16).view(np.uint16) & 0x7FFF) != 0


def encode_bitmap(A: np.ndarray):
    """A float16 R x K (K % 64 == 0) -> (bitmaps uint64 R x K/64, tile_offsets uint32
    R*K/64 + 1, values float16 [tile_offsets[-1]])."""
    A = np.asarray(A, dtype=np.float16)
    R, K = A.shape
    T = K // TILE
    tiles = A.reshape(R * T, TILE)
    nz = _nonzero(tiles)
    weights = np.left_shift(np.uint64(1), np.arange(TILE, dtype=np.uint64))
    bitmaps = (nz.astype(np.uint64) * weights[None, :]).sum(axis=1, dtype=np.uint64)
    counts = nz.sum(axis=1)
    padded = (counts + 7) // 8 * 8
    offsets = np.zeros(R * T + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    values = np.zeros(int(offsets[-1]), dtype=np.float16)
    for t in range(R * T):
        kept = tiles[t][nz[t]]
        values[offsets[t]:offsets[t] + kept.size] = kept
    return bitmaps.reshape(R, T), offsets.astype(np.uint32), values


def decode_bitmap(bitmaps: np.ndarray, tile_offsets: np.ndarray, values: np.ndarray, K: int) -> np.ndarray:
    """Dense float16 R x K: position i of tile t holds the next stored value if bit i is set."""
    bitmaps = np.asarray(bitmaps, dtype=np.uint64)
    R = bitmaps.shape[0]
    T = K // TILE
    out = np.zeros((R * T, TILE), dtype=np.float16)
    flat = bitmaps.reshape(-1)
    offs = np.asarray(tile_offsets, dtype=np.int64)
    for t in range(R * T):
        bits = (flat[t] >> np.arange(TILE, dtype=np.uint64)) & np.uint64(1)
        pos = np.nonzero(bits)[0]
        out[t, pos] = values[offs[t]:offs[t] + pos.size]
    return out.reshape(R, K)


def spmm_bitmap(bitmaps, tile_offsets, values, B: np.ndarray) -> np.ndarray:
    """Y = decode(A) @ B in float64."""
    B = np.asarray(B)
    A_hat = decode_bitmap(bitmaps, tile_offsets, values, B.shape[0])
    return A_hat.astype(np.float64) @ B.astype(np.float64)


def format_bytes(bitmaps, tile_offsets, values, with_offsets: bool = True) -> int:
    """Bytes of the compressed arrays (values fp16 + 8-byte bitmaps [+ 4-byte offsets])."""
    n = np.asarray(values).size * 2 + np.asarray(bitmaps).size * 8
    if with_offsets:
        n += np.asarray(tile_offsets).size * 4
    return int(n)
