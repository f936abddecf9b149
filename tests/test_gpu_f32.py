"""GPU parity of 1:2 dynamic attention on fp32 scores (SDDMM-prune, softmax, product).

Tolerances follow from fp32 arithmetic (unit roundoff u = 2**-24) and the classical bound
gamma_n = n u / (1 - n u) of an n-term sum accumulated in fp32:
* scores: |S - S_ref| <= gamma_{d+2} scale sum|q||k| + 2.02 u |S_exact|;
* softmax: each probability's relative error <= gamma_kept (the row sum) + 1e-5 (exp2 and
  the scaling by log2 e for |v - max| < 30);
* the product (a dense fp32 matrix-core product over all K positions, zeros included):
  |Y - Y_ref| <= 1.01 gamma_K (|A| |B|); with the GPU's probabilities or the softmax inside,
  (3 gamma_K + 2e-5) (P_ref |V|) + 1.01 u |O_ref|.
Each bound is checked per element, with a relative Frobenius error of at most 1e-4. Parity
of the pruning is layered as for 16-bit data: the oracle's 1:2 rule applied to the GPU's own
scores reproduces its values and metadata bit for bit, the scores are within their bound,
and each kept element is a valid choice for the oracle's scores within that bound; inputs
with exact fp32 products give bit-exact results.
"""
import numpy as np
import pytest

import oracle
from oracle import variants as ov
from oracle.nm import _unpack_codes
import workloads
from _parity import to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def gamma(n):
    return n * U / (1 - n * U)


def assert_within(got, ref, bound, what, frob=1e-4):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the bound; worst excess "
                           f"{(err - bound).max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}")
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / (nr if nr > 0 else 1.0)
    assert rel <= frob, f"{what}: relative Frobenius error {rel:.3e} > {frob}"


def assert_bits(got, ref, what):
    g, r = np.ascontiguousarray(got), np.ascontiguousarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gv = g.view(np.uint32) if g.dtype == np.float32 else g
    rv = r.view(np.uint32) if r.dtype == np.float32 else r
    mism = gv != rv
    assert not mism.any(), f"{what}: {mism.sum()} of {mism.size} differ, first at {np.argwhere(mism)[0]}"


def _qkv(seed, b, lq, lk, d):
    rng = np.random.default_rng(seed)
    return (workloads.normal_f32(rng, (b, lq, d)), workloads.normal_f32(rng, (b, lk, d)),
            workloads.normal_f32(rng, (b, lk, d)))


def _score_bound(Q, K, scale):
    q, k = Q.astype(np.float64), K.astype(np.float64)
    exact = (q @ np.swapaxes(k, -1, -2)) * scale
    e = gamma(q.shape[-1] + 2) * (np.abs(q) @ np.swapaxes(np.abs(k), -1, -2)) * abs(scale)
    return e + 2.02 * U * np.abs(exact) + 1e-37, exact


def _selection_valid(exact, tau, meta, what):
    rows = exact.reshape(-1, exact.shape[-1])
    lk = rows.shape[-1]
    codes = _unpack_codes(meta.reshape(-1, lk // 4))[:, : lk // 2]
    assert set(np.unique(codes).tolist()) <= {0x4, 0xE}, what
    second = codes == 0xE
    mags = np.abs(rows).reshape(-1, lk // 2, 2)
    t2 = tau.reshape(-1, lk // 2, 2)
    kept = np.where(second, mags[..., 1] + t2[..., 1], mags[..., 0] + t2[..., 0])
    dropped = np.where(second, mags[..., 0] - t2[..., 0], mags[..., 1] - t2[..., 1])
    assert np.all(kept >= dropped), what + " invalid selection"


@pytest.mark.parametrize("b,lq,lk,d", [(1, 32, 32, 64), (2, 100, 64, 64), (3, 257, 96, 16),
                                       (2, 64, 128, 32), (1, 40, 64, 128), (2, 300, 544, 64)])
def test_sddmm_1of2_layered(b, lq, lk, d):
    snm = _snm()
    Q, K, _ = _qkv(b * 1000 + lq + lk + d, b, lq, lk, d)
    scale = 1.0 / np.sqrt(d)
    v, m, S, rmax = snm.sddmm_prune_1of2_f32(to_dev(Q), to_dev(K), scale, return_dense=True,
                                             return_rowmax=True)
    v, m, S, rmax = to_host(v), to_host(m), to_host(S), to_host(rmax)
    what = f"1:2 {b}x{lq}x{lk}x{d}"
    sv, sm = ov.prune_encode_1of2(S.reshape(-1, lk))
    assert_bits(v.reshape(-1, lk // 2), sv, what + " values vs 1:2(S_gpu)")
    assert_bits(m.reshape(-1, lk // 4), sm, what + " meta vs 1:2(S_gpu)")
    tau, exact = _score_bound(Q, K, scale)
    assert_within(S, exact, tau, what + " scores", frob=1e-5)
    _selection_valid(exact, tau, m, what)
    assert_bits(rmax, v.max(-1), "row_max")
    v2, m2 = snm.sddmm_prune_1of2_f32(to_dev(Q), to_dev(K), scale)
    assert_bits(to_host(v2), v, "values without S")
    assert_bits(to_host(m2), m, "meta without S")


def test_sddmm_1of2_exact_integer_scores():
    # integer Q, K: every fp32 product and partial sum is exact, so the GPU's S, values and
    # metadata equal the oracle's bit for bit (ties between equal magnitudes included)
    snm = _snm()
    rng = np.random.default_rng(31)
    Q = rng.integers(-8, 9, size=(2, 64, 64)).astype(np.float32)
    K = rng.integers(-8, 9, size=(2, 160, 64)).astype(np.float32)
    v, m, S = snm.sddmm_prune_1of2_f32(to_dev(Q), to_dev(K), 0.25, return_dense=True)
    ovals, ometa, oS = ov.sddmm_prune_1of2(Q, K, 0.25)
    assert_bits(to_host(S), oS, "S")
    assert_bits(to_host(v), ovals, "values")
    assert_bits(to_host(m), ometa, "meta")
    assert np.count_nonzero(np.abs(oS[..., 0::2]) == np.abs(oS[..., 1::2])) > 10   # ties occur


def test_sddmm_1of2_identity_keys_exact():
    snm = _snm()
    rng = np.random.default_rng(32)
    Q = workloads.normal_f32(rng, (2, 48, 64))
    eye = np.ascontiguousarray(np.broadcast_to(np.eye(64, dtype=np.float32), (2, 64, 64)))
    v, m = snm.sddmm_prune_1of2_f32(to_dev(Q), to_dev(eye), 0.125)
    ovals, ometa, _ = ov.sddmm_prune_1of2(Q, eye, 0.125)
    assert_bits(to_host(v), ovals, "values")
    assert_bits(to_host(m), ometa, "meta")


@pytest.mark.parametrize("rows,kept", [(7, 2048), (5, 104), (3, 4096), (2, 5000), (64, 32), (3, 37)])
def test_softmax_f32(rows, kept):
    snm = _snm()
    x = workloads.normal_f32(np.random.default_rng(rows + kept), (rows, kept), 3.0)
    t = to_dev(x)
    snm.softmax_nm_rows_f32(t)
    ref = ov.softmax_rows(x)
    assert_within(to_host(t), ref, (gamma(kept) + 1e-5) * ref + 1e-37, f"softmax {rows}x{kept}")


def test_softmax_f32_constant_row():
    snm = _snm()
    t = to_dev(np.full((4, 2048), 1.5, dtype=np.float32))
    snm.softmax_nm_rows_f32(t)
    assert np.all(to_host(t) == np.float32(1.0 / 2048))


def _spmm_problem(seed, b, R, K, C):
    rng = np.random.default_rng(seed)
    A = workloads.normal_f32(rng, (b, R, K))
    B = workloads.normal_f32(rng, (b, K, C))
    values, meta = ov.prune_encode_1of2(A.reshape(b * R, K))
    return values.reshape(b, R, K // 2), meta.reshape(b, R, K // 4), B


@pytest.mark.parametrize("b,R,K,C", [
    (1, 32, 32, 64), (2, 100, 64, 64), (1, 130, 96, 72), (1, 257, 64, 8), (3, 64, 160, 4),
    (1, 40, 256, 128), (1, 200, 512, 100), (2, 129, 2048, 64), (1, 300, 256, 260)])
def test_spmm_1of2_vs_oracle(b, R, K, C):
    snm = _snm()
    values, meta, B = _spmm_problem(R * 7 + K + C, b, R, K, C)
    Y = to_host(snm.spmm_1of2_f32(to_dev(values), to_dev(meta), to_dev(B)))
    for i in range(b):
        Ad = ov.decode_1of2(values[i], meta[i], K)
        ref = Ad @ B[i].astype(np.float64)
        bound = 1.01 * gamma(K) * (np.abs(Ad) @ np.abs(B[i].astype(np.float64))) + 1e-37
        assert_within(Y[i], ref, bound, f"spmm 1:2 {b}x{R}x{K}x{C} [{i}]")


def test_spmm_1of2_identity_exact_2d_and_empty():
    import torch
    snm = _snm()
    values, meta, _ = _spmm_problem(41, 1, 96, 128, 8)
    Y = to_host(snm.spmm_1of2_f32(to_dev(values[0]), to_dev(meta[0]), to_dev(np.eye(128, dtype=np.float32))))
    assert_bits(Y, ov.decode_1of2(values[0], meta[0], 128).astype(np.float32), "identity")
    out = torch.full((1, 40, 64), 7.0, dtype=torch.float32, device="cuda")
    snm.spmm_1of2_f32(torch.empty((1, 40, 0), device="cuda"), torch.empty((1, 40, 0), dtype=torch.uint8, device="cuda"),
                      torch.empty((1, 0, 64), device="cuda"), out=out)
    assert np.all(to_host(out) == 0)


def test_spmm_1of2_softmax_constant_rows():
    # equal kept scores 0.5 (a power of two, so 0.5 log2(e) is exact in fp32 and the exponent
    # is exactly 0): every exponential is 1 and each row sum is K/2 = 128 (a power of two), so
    # each output is the exact mean of the kept rows of B
    snm = _snm()
    R, K, C = 64, 256, 64
    values = np.full((1, R, K // 2), 0.5, dtype=np.float32)
    codes = np.where(np.arange(K // 2) % 3 == 0, 0xE, 0x4)[None, :].repeat(R, 0)
    meta = oracle.nm._pack_codes(codes).reshape(1, R, K // 4)
    B = (np.round(workloads.normal_f32(np.random.default_rng(5), (1, K, C)) * 64) / 64).astype(np.float32)
    rmax = np.full((1, R), 0.5, dtype=np.float32)
    Y = to_host(snm.spmm_1of2_f32(to_dev(values), to_dev(meta), to_dev(B), row_max=to_dev(rmax)))
    kept = 2 * np.arange(K // 2) + (codes[0] == 0xE)
    mean = B[0][kept].astype(np.float64).mean(0)
    assert_bits(Y[0], np.broadcast_to(mean.astype(np.float32), (R, C)), "constant rows")


def _decode_p(p, meta, lk):
    codes = _unpack_codes(meta)[:, : lk // 2]
    out = np.zeros((p.shape[0], lk // 2, 2))
    out[np.arange(p.shape[0])[:, None], np.arange(lk // 2)[None, :], (codes == 0xE).astype(np.int64)] = p
    return out.reshape(p.shape[0], lk)


@pytest.mark.parametrize("b,lq,lk,d", [(2, 128, 128, 64), (1, 512, 512, 64), (3, 96, 96, 32),
                                       (2, 160, 256, 128), (2, 100, 256, 64)])
def test_attention_1of2_end_to_end(b, lq, lk, d):
    # downstream reference: the oracle's float64 softmax over the GPU's own scores and its
    # product with V (the score stage is checked above)
    snm = _snm()
    Q, K, V = _qkv(91 + lq + lk + d, b, lq, lk, d)
    scale = 1.0 / np.sqrt(d)
    dQ, dK, dV = to_dev(Q), to_dev(K), to_dev(V)
    O = to_host(snm.attention_1of2_f32(dQ, dK, dV, scale))
    Of = to_host(snm.attention_1of2_fused_f32(dQ, dK, dV, scale))
    v, m, S = snm.sddmm_prune_1of2_f32(dQ, dK, scale, return_dense=True)
    S, m = to_host(S), to_host(m)
    P_ref, O_ref = ov.attention_1of2_from_pattern(S, m, V)
    PV = np.stack([_decode_p(P_ref[i], m[i], lk) @ np.abs(V[i].astype(np.float64)) for i in range(b)])
    bound = (3 * gamma(lk) + 2e-5) * PV + 1.01 * U * np.abs(O_ref) + 1e-30
    assert_within(O, O_ref, bound, f"attention 1:2 {b}x{lq}x{lk}x{d}")
    assert_within(Of, O_ref, bound, "fused")
    snm.softmax_nm_rows_f32(v)
    assert_within(to_host(v), P_ref, (gamma(lk // 2) + 1e-5) * P_ref + 1e-37, "P")


def test_attention_1of2_workload_sampled_heads():
    # batch 4 x 16 heads, seq 4096, head_dim 64 in fp32 through both pipelines in the launch
    # configuration the benchmark times; on 32 sampled query rows of every slice: the kept
    # scores against the oracle's, the validity of the pattern, P and O
    import torch
    snm = _snm()
    w = workloads.WORKLOADS["attention_2_4"]
    Q, K, V = workloads.attention_qkv_typed(w, "f32")
    scale = 0.125
    dQ, dK, dV = to_dev(Q), to_dev(K), to_dev(V)
    vals, meta, rmax = snm.sddmm_prune_1of2_f32(dQ, dK, scale, return_rowmax=True)
    Of = snm.spmm_1of2_f32(vals, meta, dV, row_max=rmax)
    scores = vals.clone()
    snm.softmax_nm_rows_f32(vals)
    O = snm.spmm_1of2_f32(vals, meta, dV)
    rng = np.random.default_rng(8)
    L = 4096
    for h in range(Q.shape[0]):
        rows = np.sort(rng.choice(L, 32, replace=False))
        ri = torch.from_numpy(rows).cuda()
        sc, mh, ph = to_host(scores[h, ri]), to_host(meta[h, ri]), to_host(vals[h, ri])
        tau, exact = _score_bound(Q[h, rows], K[h], scale)
        _selection_valid(exact, tau, mh, f"head {h}")
        second = (_unpack_codes(mh)[:, : L // 2] == 0xE).astype(np.int64)
        kept_exact = np.take_along_axis(exact.reshape(32, L // 2, 2), second[..., None], 2)[..., 0]
        kept_tau = np.take_along_axis(tau.reshape(32, L // 2, 2), second[..., None], 2)[..., 0]
        assert_within(sc, kept_exact, kept_tau, f"kept scores head {h}", frob=1e-5)
        P_ref = ov.softmax_rows(sc)
        O_ref = _decode_p(P_ref, mh, L) @ V[h].astype(np.float64)
        PV = _decode_p(P_ref, mh, L) @ np.abs(V[h].astype(np.float64))
        bound = (3 * gamma(L) + 2e-5) * PV + 1.01 * U * np.abs(O_ref) + 1e-30
        assert_within(ph, P_ref, (gamma(L // 2) + 1e-5) * P_ref + 1e-37, f"P head {h}")
        assert_within(to_host(O[h, ri]), O_ref, bound, f"O head {h}")
        assert_within(to_host(Of[h, ri]), O_ref, bound, f"fused O head {h}")
