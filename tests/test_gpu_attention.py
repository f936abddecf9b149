"""GPU parity of dynamic 2:4 attention: SDDMM-prune, softmax over kept entries, P.V.

The GPU accumulates Q K^T in fp32, the oracle in float64, so a score can differ by one
fp16 ulp at a rounding boundary and a near-tie can then flip. Parity is layered:
(i) structural invariants; (ii) bit-exact self-consistency: the oracle's 2:4 rule applied
to the GPU's own pre-prune scores reproduces the GPU's values and metadata; (iii) the
GPU's scores against the oracle's within the fp16 bars; (iv) every GPU selection is valid
for the oracle's scores up to that tolerance; and the exact special case K = I."""
import numpy as np
import pytest

import oracle
from oracle.nm import _unpack_codes
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _qkv(seed, b, lq, lk, d):
    rng = np.random.default_rng(seed)
    return (workloads.normal_f16(rng, (b, lq, d)), workloads.normal_f16(rng, (b, lk, d)),
            workloads.normal_f16(rng, (b, lk, d)))


def _layered_sddmm_checks(Q, K, scale, values, meta, S_gpu, what):
    b, lq, lk = S_gpu.shape
    # (i) invariants
    codes = _unpack_codes(meta.reshape(-1, lk // 8))
    assert set(np.unique(codes).tolist()) <= set(oracle.NM_LEGAL_CODES), what
    # (ii) self-consistency, bit exact
    sv, sm = oracle.prune_encode_nm(S_gpu.reshape(-1, lk))
    assert_bits_equal(values.reshape(-1, lk // 2), sv, what + " values vs 2:4(S_gpu)")
    assert_bits_equal(meta.reshape(-1, lk // 8), sm, what + " meta vs 2:4(S_gpu)")
    # (iii) scores against the float64 oracle
    S_ref = oracle.attention.scores_f16(Q, K, scale)
    exact = (Q.astype(np.float64) @ np.swapaxes(K.astype(np.float64), -1, -2)) * scale
    assert_fp16_close(S_gpu, exact, what + " scores")
    # (iv) selection validity with respect to the oracle's scores
    tau = 1e-2 * (1 + np.abs(exact))
    mags = np.abs(exact).reshape(-1, lk // 4, 4)
    t4 = tau.reshape(-1, lk // 4, 4)
    keep = np.zeros(mags.shape, dtype=bool)
    rr = np.arange(mags.shape[0])[:, None]
    gg = np.arange(lk // 4)[None, :]
    keep[rr, gg, codes & 3] = True
    keep[rr, gg, codes >> 2] = True
    kept_min = np.where(keep, mags + t4, np.inf).min(-1)
    drop_max = np.where(~keep, mags - t4, -np.inf).max(-1)
    assert np.all(kept_min >= drop_max), what + " invalid selection"
    om = oracle.prune_encode_nm(S_ref.reshape(-1, lk))[1]
    differ = np.count_nonzero(_unpack_codes(om) != codes)
    assert differ <= max(2, codes.size // 1000), f"{what}: {differ} groups differ from the oracle"
    return differ


@pytest.mark.parametrize("b,lq,lk,d", [(1, 32, 32, 64), (2, 100, 64, 64), (3, 257, 96, 16),
                                       (2, 64, 128, 32), (1, 40, 64, 128), (2, 512, 512, 64)])
def test_sddmm_prune_layered(b, lq, lk, d):
    snm = _snm()
    Q, K, _ = _qkv(b * 1000 + lq + lk + d, b, lq, lk, d)
    scale = 1.0 / np.sqrt(d)
    v, m, S = snm.sddmm_prune_nm(to_dev(Q), to_dev(K), scale, return_dense=True)
    _layered_sddmm_checks(Q, K, scale, to_host(v), to_host(m), to_host(S), f"{b}x{lq}x{lk}x{d}")


def test_sddmm_identity_keys_exact():
    # Lk = d, K = I: S = Q / 8 exactly, so the output is the 2:4 encoding of Q / 8
    snm = _snm()
    Q = workloads.small_matrix(3, (2, 48, 64))
    eye = np.ascontiguousarray(np.broadcast_to(np.eye(64, dtype=np.float16), (2, 64, 64)))
    v, m = snm.sddmm_prune_nm(to_dev(Q), to_dev(eye), 0.125)
    ov, om, _ = oracle.sddmm_prune_nm(Q, eye, 0.125)
    assert_bits_equal(to_host(v), ov, "values")
    assert_bits_equal(to_host(m), om, "meta")


@pytest.mark.parametrize("rows,kept", [(7, 2048), (5, 104), (3, 4096), (2, 5000), (64, 32)])
def test_softmax_rows(rows, kept):
    snm = _snm()
    x = (workloads.small_matrix(rows + kept, (rows, kept)).astype(np.float64) * 3).astype(np.float16)
    t = to_dev(x)
    snm.softmax_nm_rows(t)
    got = to_host(t)
    ref = oracle.softmax_nm_rows(x)
    assert_fp16_close(got, ref, f"softmax {rows}x{kept}")
    assert np.allclose(got.astype(np.float64).sum(-1), 1.0, atol=2e-3 + kept * 5e-7)


def test_softmax_constant_row():
    snm = _snm()
    t = to_dev(np.full((4, 2048), 1.5, dtype=np.float16))
    snm.softmax_nm_rows(t)
    assert np.all(to_host(t) == np.float16(1.0 / 2048))


@pytest.mark.parametrize("b,L,d", [(2, 128, 64), (1, 512, 64), (3, 96, 32)])
def test_attention_end_to_end(b, L, d):
    snm = _snm()
    Q, K, V = _qkv(77 + L, b, L, L, d)
    scale = 1.0 / np.sqrt(d)
    O = snm.attention_nm(to_dev(Q), to_dev(K), to_dev(V), scale)
    # downstream parity is judged on the GPU's own pattern (a flipped near-tie may swap a +x
    # for a -x logit), with the oracle's float64 softmax and product
    v, m, S = snm.sddmm_prune_nm(to_dev(Q), to_dev(K), scale, return_dense=True)
    S_ref = oracle.attention.scores_f16(Q, K, scale)
    P_ref, O_ref = oracle.attention.attention_from_pattern(S_ref, to_host(m), V)
    assert_fp16_close(to_host(O), O_ref, f"attention {b}x{L}x{d}")
    snm.softmax_nm_rows(v)
    assert_fp16_close(to_host(v), P_ref, "P")


def test_attention_workload_sampled_heads():
    # batch 4 x 16 heads, seq 4096, head_dim 64, through the full pipeline; the oracle checks
    # two (batch, head) slices in full and 64 sampled query rows of every other slice
    snm = _snm()
    w = workloads.WORKLOADS["attention_2_4"]
    Q, K, V = workloads.attention_qkv(w)
    scale = 0.125
    dQ, dK, dV = to_dev(Q), to_dev(K), to_dev(V)
    vals, meta = snm.sddmm_prune_nm(dQ, dK, scale)
    meta_h = to_host(meta)
    snm.softmax_nm_rows(vals)
    O = to_host(snm.spmm_nm(vals, meta, dV))
    P = vals
    rng = np.random.default_rng(5)
    for h in range(Q.shape[0]):
        qrows = np.arange(4096) if h in (0, 37) else np.sort(rng.choice(4096, 64, replace=False))
        S_ref = oracle.attention.scores_f16(Q[h:h + 1, qrows], K[h:h + 1], scale)
        P_ref, O_ref = oracle.attention.attention_from_pattern(S_ref, meta_h[h:h + 1, qrows], V[h:h + 1])
        assert_fp16_close(O[h:h + 1, qrows], O_ref, f"O head {h}")
        if h in (0, 37):
            assert_fp16_close(to_host(P[h:h + 1]), P_ref, f"P head {h}")
