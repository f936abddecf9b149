"""Pins of the dynamic 2:4 attention oracle (CPU only)."""
import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
from oracle.attention import gather_kept, attention_from_pattern, scores_f16
import workloads


def _qkv(seed, b=2, lq=32, lk=64, d=16):
    rng = np.random.default_rng(seed)
    return (workloads.normal_f16(rng, (b, lq, d)), workloads.normal_f16(rng, (b, lk, d)),
            workloads.normal_f16(rng, (b, lk, d)))


def test_identity_keys_give_scaled_queries():
    # Lk = d and K = I: S = Q / 8 exactly (a power-of-two scale), so the SDDMM output is
    # the 2:4 encoding of Q / 8
    Q, _, _ = _qkv(0, lk=16, d=16)
    eye = np.broadcast_to(np.eye(16, dtype=np.float16), (2, 16, 16))
    values, meta, S = oracle.sddmm_prune_nm(Q, eye, 0.125)
    assert np.array_equal(S.view(np.uint16), (Q.astype(np.float64) / 8).astype(np.float16).view(np.uint16))
    v2, m2 = oracle.prune_encode_nm((Q.astype(np.float64) / 8).astype(np.float16).reshape(-1, 16))
    assert np.array_equal(values.reshape(-1, 8).view(np.uint16), v2.view(np.uint16))
    assert np.array_equal(meta.reshape(-1, 2), m2)


def test_scores_match_library_matmul():
    Q, K, _ = _qkv(1)
    S = scores_f16(Q, K, 0.125)
    ref = np.einsum("bqd,bkd->bqk", Q.astype(np.float32), K.astype(np.float32)) * 0.125
    assert np.allclose(S.astype(np.float64), ref, rtol=2e-3, atol=2e-3)
    assert S.dtype == np.float16


def test_softmax_rows_sum_to_one_and_match_scipy():
    vals = workloads.small_matrix(2, (10, 32)) * np.float16(3)
    P = oracle.softmax_nm_rows(vals)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-14)
    assert np.allclose(P, scipy_softmax(vals.astype(np.float64), axis=-1), rtol=1e-13, atol=0)


def test_softmax_constant_row_and_permutation():
    L = 64
    const = np.full((3, L // 2), 1.5, dtype=np.float16)
    assert np.allclose(oracle.softmax_nm_rows(const), 2.0 / L)
    vals = workloads.small_matrix(3, (4, 32))
    perm = np.random.default_rng(0).permutation(32)
    assert np.allclose(oracle.softmax_nm_rows(vals)[:, perm], oracle.softmax_nm_rows(vals[:, perm]))


def test_kept_entries_contain_row_max():
    # keeping the local largest of each group keeps each row's maximum (softmax is monotonic)
    Q, K, _ = _qkv(4)
    values, meta, S = oracle.sddmm_prune_nm(Q, K, 0.125)
    # the kept set holds the largest |s|; the row maximum of s is kept unless a larger -s exists
    mags = np.abs(S.astype(np.float64))
    assert np.all(np.abs(values.astype(np.float64)).max(-1) == mags.max(-1))


def test_compressed_route_equals_dense_masked_softmax():
    Q, K, V = _qkv(5)
    values, meta, S, P, O = oracle.attention_nm(Q, K, V, 0.125)
    b, lq, lk = S.shape
    dense_vals = oracle.decode_nm(values.reshape(b * lq, lk // 2), meta.reshape(b * lq, lk // 8), lk)
    # mask from the encoding's positions (a kept value may be 0.0, so use the codes, not != 0)
    mask = np.zeros((b * lq, lk // 4, 4), dtype=bool)
    codes = oracle.nm._unpack_codes(meta.reshape(b * lq, lk // 8))
    rr = np.arange(b * lq)[:, None]
    gg = np.arange(lk // 4)[None, :]
    mask[rr, gg, codes & 3] = True
    mask[rr, gg, codes >> 2] = True
    mask = mask.reshape(b, lq, lk)
    assert np.array_equal(np.where(mask, S, 0).view(np.uint16) & 0x7FFF,
                          dense_vals.reshape(b, lq, lk).view(np.uint16) & 0x7FFF)
    ref = oracle.full_attention(S, V, mask=mask)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)
    # P sums to one per row and equals the kept softmax
    assert np.allclose(P.sum(-1), 1.0)


def test_nothing_dropped_is_textbook_attention():
    # N = M: keep every entry; the kept-row softmax then P @ V is ordinary attention,
    # checked against scipy's softmax and numpy's matmul
    Q, K, V = _qkv(6)
    S = scores_f16(Q, K, 0.125)
    P = oracle.softmax_nm_rows(S)
    O = np.matmul(P, V.astype(np.float64))
    ref = np.matmul(scipy_softmax(S.astype(np.float64), axis=-1), V.astype(np.float64))
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_gather_kept_uses_the_metadata():
    S = np.arange(16, dtype=np.float16).reshape(1, 16)
    meta = np.array([[0x8 | (0xD << 4), 0x4 | (0xE << 4)]], dtype=np.uint8)
    # groups: (0,2), (1,3), (0,1), (2,3) -> columns 0,2, 5,7, 8,9, 14,15
    assert gather_kept(S, meta).tolist() == [[0, 2, 5, 7, 8, 9, 14, 15]]
