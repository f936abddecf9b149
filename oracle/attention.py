"""Dynamic 2:4 attention: SDDMM with a pruning epilogue, softmax over kept entries, SpMM.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU baseline.

Sources
-------
"Dynamic N:M fine-grained structured sparse attention mechanism on GPUs"
(PPoPP'23; the page is a machine translation into Chinese):
* Sec. 3.2 and Listing 1: the attention score matrix Q K^T is produced by an
  SDDMM kernel that prunes it to N:M by magnitude and compresses it (values +
  metadata) in one pass; softmax then runs on each row's kept entries only
  (softmax is monotonic, so keeping the largest entries keeps each row's
  maximum); the probabilities multiply V through an N:M SpMM. The scores are
  scaled by 1/sqrt(d) before the softmax, as in ordinary attention.
* Sec. 4.2 / 4.3: for 16-bit data the epilogue keeps the 2 larger of each 4
  adjacent 2-byte entries, i.e. pruning acts on the 16-bit scores.

Readings where the pages are silent
-----------------------------------
* S = fp16_RNE(Q K^T * scale), with the product in float64 and one rounding to
  float16; the 2:4 rule of the weight oracle (magnitude key on the float16
  bits, lower slot wins ties) is then applied along the key axis.
* "Softmax only on each row's non-zeros": dropped logits count as -inf, i.e.
  they contribute nothing to the row's max and sum.
"""
from __future__ import annotations

import numpy as np

from .nm import prune_encode_nm, _unpack_codes


def scores_f16(Q: np.ndarray, Kmat: np.ndarray, scale: float) -> np.ndarray:
    """S[b] = fp16_RNE(float64(Q[b]) @ float64(K[b])^T * scale), shape [batch, Lq, Lk]."""
    Q = np.asarray(Q, dtype=np.float16).astype(np.float64)
    Kmat = np.asarray(Kmat, dtype=np.float16).astype(np.float64)
    S = np.matmul(Q, np.swapaxes(Kmat, -1, -2)) * float(scale)
    return S.astype(np.float16)


def sddmm_prune_nm(Q: np.ndarray, Kmat: np.ndarray, scale: float):
    """Scores pruned 2:4 along the key axis.

    Returns (values float16 [batch, Lq, Lk/2], meta uint8 [batch, Lq, Lk/8],
    S float16 [batch, Lq, Lk] -- the scores before pruning).
    """
    S = scores_f16(Q, Kmat, scale)
    b, lq, lk = S.shape
    values, meta = prune_encode_nm(S.reshape(b * lq, lk))
    return values.reshape(b, lq, lk // 2), meta.reshape(b, lq, lk // 8), S


def softmax_nm_rows(values: np.ndarray) -> np.ndarray:
    """Row softmax over the stored (kept) values only, float64.

    values: [..., kept_per_row]. p = exp(v - max) / sum(exp(v - max)) per row.
    """
    v = np.asarray(values).astype(np.float64)
    mx = v.max(axis=-1, keepdims=True)
    e = np.exp(v - mx)
    return e / e.sum(axis=-1, keepdims=True)


def gather_kept(S: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """Entries of a dense [rows, L] matrix at the positions a 2:4 metadata array names,
    in stored order: out[r, 2g + j] = S[r, 4g + slot_j]."""
    S = np.asarray(S)
    rows, L = S.shape
    codes = _unpack_codes(meta)[:, : L // 4].astype(np.int64)
    slots = np.stack([codes & 3, (codes >> 2) & 3], axis=-1)       # rows x G x 2
    return np.take_along_axis(S.reshape(rows, L // 4, 4), slots, axis=2).reshape(rows, L // 2)


def attention_from_pattern(S: np.ndarray, meta: np.ndarray, Vmat: np.ndarray):
    """Given scores S [batch, Lq, Lk] and a 2:4 pattern, return (P [batch, Lq, Lk/2] float64,
    O [batch, Lq, d] float64): softmax over the kept scores, then P (decoded) @ V."""
    b, lq, lk = S.shape
    kept = gather_kept(S.reshape(b * lq, lk), meta.reshape(b * lq, lk // 8))
    P = softmax_nm_rows(kept)
    O = np.empty((b, lq, Vmat.shape[-1]), dtype=np.float64)
    codes_meta = meta.reshape(b, lq, lk // 8)
    for i in range(b):
        # scatter the float64 probabilities back to their key columns: P_hat[q, 4g + slot] = p
        codes = _unpack_codes(codes_meta[i])[:, : lk // 4].astype(np.int64)
        dense = np.zeros((lq, lk // 4, 4), dtype=np.float64)
        pv = P.reshape(b, lq, lk // 4, 2)[i]
        rr = np.arange(lq)[:, None]
        gg = np.arange(lk // 4)[None, :]
        dense[rr, gg, codes & 3] = pv[..., 0]
        dense[rr, gg, (codes >> 2) & 3] = pv[..., 1]
        O[i] = dense.reshape(lq, lk) @ np.asarray(Vmat[i], dtype=np.float64)
    return P.reshape(b, lq, lk // 2), O


def attention_nm(Q, Kmat, Vmat, scale: float):
    """The whole dynamic 2:4 attention: returns (values, meta, S, P, O)."""
    values, meta, S = sddmm_prune_nm(Q, Kmat, scale)
    P, O = attention_from_pattern(S, meta, np.asarray(Vmat, dtype=np.float16))
    return values, meta, S, P, O


def full_attention(S: np.ndarray, Vmat: np.ndarray, mask=None) -> np.ndarray:
    """Textbook dense attention on given scores: softmax(S [-inf where mask is False]) @ V, float64."""
    S = np.asarray(S, dtype=np.float64)
    if mask is not None:
        S = np.where(mask, S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    E = np.exp(S)
    return np.matmul(E / E.sum(axis=-1, keepdims=True), np.asarray(Vmat, dtype=np.float64))
