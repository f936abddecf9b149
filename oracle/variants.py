"""The DFSS data-type variants: bf16 scores with 2:4, fp32 scores with 1:2.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU baseline.

Sources
-------
"Dynamic N:M fine-grained structured sparse attention mechanism on GPUs"
(PPoPP'23; the page is a machine translation into Chinese):
* Sec. 1 and Fig. 1-3: the mechanism is evaluated at 1:2 and 2:4; the
  pruning step keeps one of every two scores (1:2) or two of every four
  (2:4) by magnitude.
* Sec. 4.2 (pruning epilogue): every consecutive 8 bytes of scores are
  pruned by half; the sparse tensor core's own shapes fix the pairing of
  data type and pattern -- 32-bit (tf32) data is 1:2, 16-bit data (f16 and
  bf16) is 2:4. Fig. 6(b) gives the 4-bit codes, and for 32-bit data only
  0x4 (the first 4-byte element of the 8 bytes) and 0xe (the second) occur.
* Sec. 4.3: four 4-bit codes form one 16-bit metadata word.

Readings where the pages are silent
-----------------------------------
* bf16 rounding: every bf16 result is one round-to-nearest-even of the exact
  (float64) value onto the bf16 grid: 8 significant bits, exponent range of
  float32 (gradual underflow below 2**-126, overflow to infinity).
* bf16 2:4 selection is the 2:4 rule on the 16-bit words: the magnitude key
  bits & 0x7FFF orders finite bf16 values exactly as their magnitudes (sign
  and magnitude layout, like fp16), ties go to the lower slot. The values
  are bit copies.
* 1:2 on fp32: in each pair of consecutive fp32 scores the one with the
  larger magnitude is kept (key bits & 0x7FFFFFFF); on a tie the first. The
  metadata is the 2:4 metadata of the same bytes seen as 16-bit halves: the
  kept element is the halves (0, 1) -> code 0x4, or (2, 3) -> code 0xe; one
  code per pair, two codes per byte, low nibble first, so a row of K fp32
  scores has K/4 metadata bytes and K/2 values.
* fp32 scores are round-to-nearest-even of the float64 product (this
  hardware has no tf32 matrix unit; its fp32 products carry the full fp32
  inputs, so the exact product is the reference).
* The softmax and the product with V take the kept scores at their stored
  positions, as in the fp16 pipeline; float64 throughout.
"""
from __future__ import annotations

import numpy as np

from .nm import select_top_n, _pack_codes, _unpack_codes

# ---------------------------------------------------------------------------------------
# bf16 as 16-bit containers (numpy has no bf16 type)

BF16_MAX = float.fromhex("0x1.fep127")


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of a float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, one round-to-nearest-even onto the bf16 grid.

    The grid spacing around |x| is 2**(max(e, -126) - 7), e = floor(log2 |x|); x is
    divided by that power of two (exact), rounded half to even (np.rint), and scaled
    back (exact). Values beyond the largest finite bf16 after rounding become infinity.
    """
    x0 = np.asarray(x, dtype=np.float64)
    x = np.atleast_1d(x0)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    fin = np.isfinite(x) & (ax > 0)
    e = np.full(x.shape, -126, dtype=np.int64)
    e[fin] = np.maximum(np.floor(np.log2(ax[fin])).astype(np.int64), -126)
    # floor(log2) of a float64 can be off by one next to a power of two; fix it exactly
    lo = fin & (ax < np.ldexp(1.0, e)) & (e > -126)
    e[lo] -= 1
    hi = fin & (ax >= np.ldexp(1.0, e + 1))
    e[hi] += 1
    ulp_exp = e - 7
    q = np.rint(np.ldexp(x, -ulp_exp))           # exact scaling, then ties to even
    out[:] = np.ldexp(q, ulp_exp)
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    out[np.abs(out) > BF16_MAX] = np.copysign(np.inf, x[np.abs(out) > BF16_MAX])
    zero = x == 0
    out[zero] = x[zero]                           # keeps the sign of zero
    # the float64 value is now a bf16 value: its float32 form is exact, take the top half
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits.reshape(x0.shape)


# ---------------------------------------------------------------------------------------
# bf16, 2:4

def prune_encode_nm_bf16(bits: np.ndarray):
    """2:4 prune of a bf16 R x K matrix (uint16 bits) along K.

    Returns (values uint16 R x K/2, meta uint8 R x K/8). Same rule, slot order and
    metadata layout as the fp16 format.
    """
    A = np.ascontiguousarray(bits, dtype=np.uint16)
    R, K = A.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    G = K // 4
    groups = A.reshape(R, G, 4)
    keys = (groups & np.uint16(0x7FFF)).astype(np.int32)
    keep = select_top_n(keys, 2)
    slots = np.nonzero(keep.reshape(-1, 4))[1].reshape(R, G, 2)
    values = np.take_along_axis(groups, slots, axis=2).reshape(R, 2 * G)
    codes = slots[..., 0] | (slots[..., 1] << 2)
    return values, _pack_codes(codes)


def decode_nm_bf16(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Dense R x K float64 matrix of a bf16 2:4 operand: A[r, 4g + slot] = value."""
    v = bf16_to_f64(values)
    R = v.shape[0]
    G = K // 4
    codes = _unpack_codes(meta)[:, :G].astype(np.int64)
    out = np.zeros((R, G, 4), dtype=np.float64)
    rr = np.arange(R)[:, None]
    gg = np.arange(G)[None, :]
    vv = v.reshape(R, G, 2)
    out[rr, gg, codes & 3] = vv[..., 0]
    out[rr, gg, (codes >> 2) & 3] = vv[..., 1]
    return out.reshape(R, K)


def spmm_nm_bf16(values: np.ndarray, meta: np.ndarray, B_bits: np.ndarray) -> np.ndarray:
    """Y = decode(values, meta) @ B in float64; B is bf16 bits K x C."""
    B = bf16_to_f64(B_bits)
    return decode_nm_bf16(values, meta, B.shape[0]) @ B


def scores_bf16(Q_bits: np.ndarray, K_bits: np.ndarray, scale: float) -> np.ndarray:
    """S[b] = bf16_RNE(float64(Q[b]) @ float64(K[b])^T * scale) as uint16 bits."""
    Q = bf16_to_f64(Q_bits)
    Km = bf16_to_f64(K_bits)
    return f64_to_bf16(np.matmul(Q, np.swapaxes(Km, -1, -2)) * float(scale))


def sddmm_prune_nm_bf16(Q_bits, K_bits, scale: float):
    """bf16 scores pruned 2:4 along the key axis.

    Returns (values uint16 [b, Lq, Lk/2], meta uint8 [b, Lq, Lk/8], S uint16 [b, Lq, Lk]).
    """
    S = scores_bf16(Q_bits, K_bits, scale)
    b, lq, lk = S.shape
    values, meta = prune_encode_nm_bf16(S.reshape(b * lq, lk))
    return values.reshape(b, lq, lk // 2), meta.reshape(b, lq, lk // 8), S


# ---------------------------------------------------------------------------------------
# fp32, 1:2

CODE_FIRST = 0x4    # halves 0 and 1: the first fp32 element of the pair
CODE_SECOND = 0xE   # halves 2 and 3: the second


def prune_encode_1of2(A32: np.ndarray):
    """1:2 prune of an fp32 R x K matrix along K (K a multiple of 4).

    Returns (values float32 R x K/2, meta uint8 R x K/4).
    """
    A = np.ascontiguousarray(A32, dtype=np.float32)
    R, K = A.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4 (whole metadata bytes)")
    pairs = A.reshape(R, K // 2, 2)
    keys = (pairs.view(np.uint32) & np.uint32(0x7FFFFFFF)).astype(np.int64)
    keep = select_top_n(keys, 1)                         # R x K/2 x 2, one True per pair
    second = keep[..., 1]
    values = np.where(second, pairs[..., 1], pairs[..., 0]).astype(np.float32)
    codes = np.where(second, CODE_SECOND, CODE_FIRST).astype(np.uint8)
    return values, _pack_codes(codes)


def decode_1of2(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Dense R x K float64 matrix of a 1:2 fp32 operand: the kept element of pair p sits at
    2p (code 0x4) or 2p + 1 (code 0xe)."""
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    R = v.shape[0]
    P = K // 2
    codes = _unpack_codes(meta)[:, :P]
    if not np.isin(codes, (CODE_FIRST, CODE_SECOND)).all():
        raise ValueError("a 1:2 code is neither 0x4 nor 0xe")
    out = np.zeros((R, P, 2), dtype=np.float64)
    second = (codes == CODE_SECOND).astype(np.int64)
    out[np.arange(R)[:, None], np.arange(P)[None, :], second] = v
    return out.reshape(R, K)


def spmm_1of2(values: np.ndarray, meta: np.ndarray, B32: np.ndarray) -> np.ndarray:
    """Y = decode(values, meta) @ B in float64; B fp32 K x C."""
    B = np.asarray(B32, dtype=np.float32).astype(np.float64)
    return decode_1of2(values, meta, B.shape[0]) @ B


def scores_f32(Q32, K32, scale: float) -> np.ndarray:
    """S[b] = fp32_RNE(float64(Q[b]) @ float64(K[b])^T * scale)."""
    Q = np.asarray(Q32, dtype=np.float32).astype(np.float64)
    Km = np.asarray(K32, dtype=np.float32).astype(np.float64)
    return (np.matmul(Q, np.swapaxes(Km, -1, -2)) * float(scale)).astype(np.float32)


def sddmm_prune_1of2(Q32, K32, scale: float):
    """fp32 scores pruned 1:2 along the key axis.

    Returns (values float32 [b, Lq, Lk/2], meta uint8 [b, Lq, Lk/4], S float32 [b, Lq, Lk]).
    """
    S = scores_f32(Q32, K32, scale)
    b, lq, lk = S.shape
    values, meta = prune_encode_1of2(S.reshape(b * lq, lk))
    return values.reshape(b, lq, lk // 2), meta.reshape(b, lq, lk // 4), S


# ---------------------------------------------------------------------------------------
# softmax over kept entries and the product with V, given the GPU's own pattern

def softmax_rows(kept: np.ndarray) -> np.ndarray:
    """p = exp(v - max) / sum(exp(v - max)) over the last axis, float64."""
    v = np.asarray(kept, dtype=np.float64)
    e = np.exp(v - v.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_bf16_from_pattern(S_bits: np.ndarray, meta: np.ndarray, V_bits: np.ndarray):
    """Scores S (bf16 bits [b, Lq, Lk]) and a 2:4 pattern -> (P [b, Lq, Lk/2], O [b, Lq, d]),
    float64: softmax over the kept scores, then decode(P) @ V."""
    b, lq, lk = S_bits.shape
    P = np.empty((b, lq, lk // 2))
    O = np.empty((b, lq, V_bits.shape[-1]))
    for i in range(b):
        S = bf16_to_f64(S_bits[i])
        codes = _unpack_codes(meta[i].reshape(lq, lk // 8))[:, : lk // 4].astype(np.int64)
        kept = np.stack([np.take_along_axis(S.reshape(lq, lk // 4, 4), (codes & 3)[..., None], 2)[..., 0],
                         np.take_along_axis(S.reshape(lq, lk // 4, 4), ((codes >> 2) & 3)[..., None], 2)[..., 0]],
                        axis=-1).reshape(lq, lk // 2)
        p = softmax_rows(kept)
        dense = np.zeros((lq, lk // 4, 4))
        rr = np.arange(lq)[:, None]
        gg = np.arange(lk // 4)[None, :]
        pp = p.reshape(lq, lk // 4, 2)
        dense[rr, gg, codes & 3] = pp[..., 0]
        dense[rr, gg, (codes >> 2) & 3] = pp[..., 1]
        P[i] = p
        O[i] = dense.reshape(lq, lk) @ bf16_to_f64(V_bits[i])
    return P, O


def attention_1of2_from_pattern(S32: np.ndarray, meta: np.ndarray, V32: np.ndarray):
    """Scores S (fp32 [b, Lq, Lk]) and a 1:2 pattern -> (P [b, Lq, Lk/2], O [b, Lq, d]),
    float64."""
    b, lq, lk = S32.shape
    P = np.empty((b, lq, lk // 2))
    O = np.empty((b, lq, V32.shape[-1]))
    for i in range(b):
        S = np.asarray(S32[i], dtype=np.float32).astype(np.float64).reshape(lq, lk // 2, 2)
        codes = _unpack_codes(meta[i].reshape(lq, lk // 4))[:, : lk // 2]
        second = (codes == CODE_SECOND).astype(np.int64)
        kept = np.take_along_axis(S, second[..., None], 2)[..., 0]
        p = softmax_rows(kept)
        dense = np.zeros((lq, lk // 2, 2))
        dense[np.arange(lq)[:, None], np.arange(lk // 2)[None, :], second] = p
        P[i] = p
        O[i] = dense.reshape(lq, lk) @ np.asarray(V32[i], dtype=np.float32).astype(np.float64)
    return P, O
