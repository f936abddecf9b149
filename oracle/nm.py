"""2:4 magnitude pruning, the compressed format, decompression and the product.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU baseline.

Sources
-------
"2:4 sparsity on sparse tensor cores", section "The definition": in every
group of four consecutive weights along a row, at most two survive, chosen by
magnitude. Section "Recipe and accuracy": prune the two smallest-magnitude
weights of every group of four. Section "The compressed format": an R x C
matrix is stored as R x C/2 surviving values, pushed to the left, plus one
2-bit tag per value naming its slot (00..11) in the group. Section "How the
tensor core uses it": the tags select which K/2 of the K elements of each
dense B column are multiplied. Worked example: slot 1 of the second group is
column 4 + 1 = 5.

"Dynamic N:M ... attention", Sec. 4.2 and Fig. 6(b): the six legal 4-bit
group codes of 2:4 on 16-bit data are 0xe 0xd 0x9 0xc 0x8 0x4, and four
consecutive codes are concatenated into one 16-bit word.

Readings where the pages are silent
-----------------------------------
* Magnitude key: kappa(a) = bits(a) & 0x7FFF of the float16 value. For finite
  values this orders exactly as |a| (and +0, -0 tie); NaN ranks above +-Inf,
  which ranks above every finite value.
* Ties: within a group, rank(i) = #{j : k_j > k_i} + #{j < i : k_j = k_i};
  the slots of rank < n survive, so on equal magnitude the lower slot wins
  (consistent with "survivors are pushed to the left").
* Slot order and bit order: survivors are stored in ascending slot order;
  the group code is s0 | s1 << 2 (this yields exactly the six codes of
  Fig. 6(b)); group g occupies bits [4(g mod 4), 4(g mod 4)+3] of 16-bit word
  g // 4, stored little-endian, so byte b of a metadata row holds group 2b in
  its low nibble and group 2b+1 in its high nibble.
* Values are bit copies: -0, subnormals and NaN payloads are preserved.
"""
from __future__ import annotations

import numpy as np

# Fig. 6(b) of the attention page: the six 4-bit codes a 2:4 group can carry.
NM_LEGAL_CODES = frozenset({0x4, 0x8, 0x9, 0xC, 0xD, 0xE})


def magnitude_key(a16: np.ndarray) -> np.ndarray:
    """Integer magnitude key of float16 values (sign bit cleared)."""
    a16 = np.ascontiguousarray(a16, dtype=np.float16)
    return (a16.view(np.uint16) & np.uint16(0x7FFF)).astype(np.int32)


def select_top_n(keys: np.ndarray, n: int) -> np.ndarray:
    """Boolean keep-mask along the last axis: the n largest keys, ties to the lower index.

    rank(i) = #{j: key_j > key_i} + #{j < i: key_j == key_i}; keep rank < n.
    """
    m = keys.shape[-1]
    ki = keys[..., :, None]      # element i
    kj = keys[..., None, :]      # element j
    lower = np.tril(np.ones((m, m), dtype=bool), k=-1)  # lower[i, j] = j < i
    rank = (kj > ki).sum(-1) + ((kj == ki) & lower).sum(-1)
    return rank < n


def _pack_codes(codes: np.ndarray) -> np.ndarray:
    """4-bit group codes (R x G, G even) -> bytes (R x G/2): group 2b low nibble, 2b+1 high."""
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _unpack_codes(meta: np.ndarray) -> np.ndarray:
    """bytes (R x G/2) -> 4-bit group codes (R x G)."""
    meta = np.asarray(meta, dtype=np.uint8)
    out = np.empty((meta.shape[0], meta.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = meta & 0x0F
    out[:, 1::2] = meta >> 4
    return out


def prune_encode_nm(A: np.ndarray):
    """2:4 prune along K and compress.

    A: float16 R x K, K a multiple of 8 (whole metadata bytes).
    Returns (values float16 R x K/2, meta uint8 R x K/8).
    """
    A = np.ascontiguousarray(A, dtype=np.float16)
    R, K = A.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    G = K // 4
    groups = A.reshape(R, G, 4)
    keep = select_top_n(magnitude_key(groups), 2)            # R x G x 4, two True per group
    slots = np.nonzero(keep.reshape(-1, 4))[1].reshape(R, G, 2)   # ascending per group
    s0, s1 = slots[..., 0], slots[..., 1]
    values = np.take_along_axis(groups, slots, axis=2).reshape(R, 2 * G)
    codes = s0 | (s1 << 2)
    return values, _pack_codes(codes)


def decode_nm(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Rebuild the dense float16 R x K matrix: A_hat[r, 4g + slot] = value, zero elsewhere."""
    values = np.asarray(values, dtype=np.float16)
    R = values.shape[0]
    G = K // 4
    codes = _unpack_codes(meta)[:, :G].astype(np.int64)
    s0 = codes & 3
    s1 = (codes >> 2) & 3
    out = np.zeros((R, G, 4), dtype=np.float16)
    rows = np.arange(R)[:, None]
    grp = np.arange(G)[None, :]
    v = values.reshape(R, G, 2)
    out[rows, grp, s0] = v[..., 0]
    out[rows, grp, s1] = v[..., 1]
    return out.reshape(R, K)


def spmm_nm(values: np.ndarray, meta: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Y = decode(values, meta) @ B in float64 (every fp16 -> fp64 conversion is exact)."""
    B = np.asarray(B)
    A_hat = decode_nm(values, meta, B.shape[0])
    return A_hat.astype(np.float64) @ B.astype(np.float64)
