"""V:N:M (here V:2:M) pruning, the three-array format, decompression and the product.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU baseline.

Sources
-------
"VENOM: A vectorized N:M format ...", Sec. 3 (The V:N:M format) and Fig. 2:
split the dense matrix into V x M blocks; in each block keep the four most
significant columns (vector-wise pruning); then, in each row of the four kept
columns, keep the two most meaningful weights (2:4 pruning). Density is 2/M.
Fig. 3 and the text after it: the format is three arrays -- the non-zero
values (R x K/M*2), the 2-bit m-indices (one per value, naming one of the four
*selected* columns, not an original column) and column-loc (R/V x K/M x 4),
saying which four of the M columns of each block survived; column-loc entries
are printed in ascending order within each block. Fig. 4: the product gathers,
per block of V rows, the K/M*4 selected rows of the dense B and runs 2:4 on
them.

Readings where the pages are silent
-----------------------------------
* "Most significant column" = largest L2 norm over the block's V rows. Ranking
  by the sum of squares gives the same order without a square root. The sum
  is taken in float64, sequentially over the block's rows in ascending order
  (each fp16 square is exact in float64; the fixed order makes the score, and
  so the selection, reproducible bit for bit by any implementation that sums
  in that order).
* Ties between columns: the lower column index wins. Ties inside the 2:4
  step follow the 2:4 oracle (lower position wins, magnitude key on the
  float16 bits).
* m-index packing follows the 2:4 metadata: code = p0 | p1 << 2 over the
  positions p0 < p1 in 0..3 of the selected columns, two group codes per
  byte, low nibble first. column-loc is one uint8 per entry (M <= 256).
* Non-finite inputs are outside the method's domain here; their result is
  unspecified.
"""
from __future__ import annotations

import numpy as np

from .nm import magnitude_key, select_top_n, _pack_codes, _unpack_codes


def column_scores(A: np.ndarray, V: int, M: int) -> np.ndarray:
    """score[b, g, c] = sum over the V rows r of block b (ascending) of A[r, g*M + c]^2, float64."""
    A = np.asarray(A, dtype=np.float16)
    R, K = A.shape
    blocks = A.reshape(R // V, V, K // M, M).astype(np.float64)
    score = np.zeros((R // V, K // M, M), dtype=np.float64)
    for r in range(V):                      # sequential, ascending row order
        score = score + blocks[:, r] * blocks[:, r]
    return score


def prune_encode_vnm(A: np.ndarray, V: int, M: int):
    """V:2:M prune along K and compress.

    A: float16 R x K with R % V == 0, K % M == 0, (K/M) even, 4 <= M <= 256.
    Returns (values float16 R x 2K/M, midx uint8 R x K/(2M), colloc uint8 R/V x K/M x 4).
    """
    A = np.ascontiguousarray(A, dtype=np.float16)
    R, K = A.shape
    if R % V or K % M or (K // M) % 2 or not (4 <= M <= 256):
        raise ValueError("unsupported V:N:M shape")
    G = K // M
    # Stage 1 (vector-wise): four columns of largest score per V x M block, ascending.
    col_keep = select_top_n(column_scores(A, V, M), 4)           # (R/V, G, M)
    colloc = np.nonzero(col_keep.reshape(-1, M))[1].reshape(R // V, G, 4)
    # Stage 2 (2:4): per row, the two of the four selected values with the largest magnitude.
    blocks = A.reshape(R // V, V, G, M)
    gathered = np.take_along_axis(blocks, np.broadcast_to(colloc[:, None], (R // V, V, G, 4)), axis=3)
    keep = select_top_n(magnitude_key(gathered), 2)               # (R/V, V, G, 4)
    pos = np.nonzero(keep.reshape(-1, 4))[1].reshape(R // V, V, G, 2)
    values = np.take_along_axis(gathered, pos, axis=3).reshape(R, 2 * G)
    codes = (pos[..., 0] | (pos[..., 1] << 2)).reshape(R, G)
    return values, _pack_codes(codes), colloc.astype(np.uint8)


def decode_vnm(values: np.ndarray, midx: np.ndarray, colloc: np.ndarray, V: int, M: int,
               K: int) -> np.ndarray:
    """A_hat[r, g*M + colloc[r // V, g, p]] = value for each stored (value, position p)."""
    values = np.asarray(values, dtype=np.float16)
    R = values.shape[0]
    G = K // M
    codes = _unpack_codes(midx)[:, :G].astype(np.int64)
    pos = np.stack([codes & 3, (codes >> 2) & 3], axis=-1)        # R x G x 2
    cl = np.repeat(np.asarray(colloc, dtype=np.int64), V, axis=0)  # R x G x 4
    cols = np.take_along_axis(cl, pos, axis=2) + (np.arange(G) * M)[None, :, None]
    out = np.zeros((R, K), dtype=np.float16)
    out[np.arange(R)[:, None, None], cols] = values.reshape(R, G, 2)
    return out


def spmm_vnm(values, midx, colloc, V: int, M: int, B: np.ndarray) -> np.ndarray:
    """Y = decode_vnm(...) @ B in float64."""
    B = np.asarray(B)
    A_hat = decode_vnm(values, midx, colloc, V, M, B.shape[0])
    return A_hat.astype(np.float64) @ B.astype(np.float64)
