"""GPU parity of the bf16 variant of dynamic 2:4 attention and of the bf16 2:4 product.

Tolerances are derived from bf16's unit roundoff u = 2**-8 (one RNE rounding moves a
value by at most u times its magnitude) and the fp32 arithmetic of the kernels:
* a product Y = A B accumulated in fp32 and rounded once: |Y - Y_ref| <= gamma_K (|A| |B|)
  + u |Y_ref| (gamma_K = K 2**-24 / (1 - K 2**-24), the classical bound for a K-term sum);
* scores S = bf16(fp32(Q K^T) * scale): |S - S_ref| <= (1 + u) e + 2u |S_exact| with e the
  fp32 accumulation bound, since both sides round a value at most e apart;
* softmax: each probability is rounded once (u) after fp32 arithmetic whose error is far
  below u (exp2 and the scaling by log2 e: < 1e-5 relative for |v - max| < 30);
* P V with the GPU's bf16 probabilities: |O - O_ref| <= 1.01 u (P_ref |V| + |O_ref|); with
  the softmax inside the product (probabilities rounded before the normalising sum):
  2.02 u P_ref |V| + 1.01 u |O_ref|.
Every bound is checked per element, plus a relative Frobenius error of at most 2u.
Scores are pruned by the GPU from its own S, which can differ from the oracle's by one
bf16 ulp; as for fp16, parity is layered: bit-exact self-consistency, S within the bound,
every selection valid for the oracle's S within that bound, and exact special cases.
"""
import numpy as np
import pytest

import oracle
from oracle import variants as ov
from oracle.nm import _unpack_codes
import workloads
from _parity import to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -8
U32 = 2.0 ** -24


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    import torch
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gamma(k):
    return k * U32 / (1 - k * U32)


def assert_within(got, ref, bound, what):
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
    assert rel <= 2 * U, f"{what}: relative Frobenius error {rel:.3e} > {2 * U:.3e}"


def assert_bits(got, ref, what):
    g, r = np.ascontiguousarray(got), np.ascontiguousarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    mism = g != r
    assert not mism.any(), f"{what}: {mism.sum()} of {mism.size} differ, first at {np.argwhere(mism)[0]}"


def _qkv(seed, b, lq, lk, d):
    rng = np.random.default_rng(seed)
    return (workloads.normal_bf16(rng, (b, lq, d)), workloads.normal_bf16(rng, (b, lk, d)),
            workloads.normal_bf16(rng, (b, lk, d)))


def _score_bound(Q, K, scale):
    """Elementwise bound of |S_gpu - S_ref| and the exact scores (float64)."""
    q, k = ov.bf16_to_f64(Q), ov.bf16_to_f64(K)
    exact = (q @ np.swapaxes(k, -1, -2)) * scale
    e = gamma(q.shape[-1]) * (np.abs(q) @ np.swapaxes(np.abs(k), -1, -2)) * scale
    return (1 + U) * e + 2 * U * np.abs(exact) * (1 + U) + 1e-30, exact


def _layered_checks(Q, K, scale, values, meta, S_gpu, what):
    b, lq, lk = S_gpu.shape
    codes = _unpack_codes(meta.reshape(-1, lk // 8))
    assert set(np.unique(codes).tolist()) <= set(oracle.NM_LEGAL_CODES), what
    sv, sm = ov.prune_encode_nm_bf16(S_gpu.reshape(-1, lk))
    assert_bits(values.reshape(-1, lk // 2), sv, what + " values vs 2:4(S_gpu)")
    assert_bits(meta.reshape(-1, lk // 8), sm, what + " meta vs 2:4(S_gpu)")
    tau, exact = _score_bound(Q, K, scale)
    assert_within(ov.bf16_to_f64(S_gpu), exact, tau, what + " scores")
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


@pytest.mark.parametrize("b,lq,lk,d", [(1, 32, 32, 64), (2, 100, 64, 64), (3, 257, 96, 16),
                                       (2, 64, 128, 32), (1, 40, 64, 128), (2, 512, 512, 64)])
def test_sddmm_bf16_layered(b, lq, lk, d):
    snm = _snm()
    Q, K, _ = _qkv(b * 1000 + lq + lk + d, b, lq, lk, d)
    scale = 1.0 / np.sqrt(d)
    v, m, S, rmax = snm.sddmm_prune_nm_bf16(dev_bf16(Q), dev_bf16(K), scale, return_dense=True,
                                            return_rowmax=True)
    v, m, S, rmax = host_bits(v), to_host(m), host_bits(S), to_host(rmax)
    _layered_checks(Q, K, scale, v, m, S, f"bf16 {b}x{lq}x{lk}x{d}")
    assert_bits(rmax, ov.bf16_to_f64(v).max(-1).astype(np.float32), "row_max")
    v2, m2 = snm.sddmm_prune_nm_bf16(dev_bf16(Q), dev_bf16(K), scale)   # no optional outputs
    assert_bits(host_bits(v2), v, "values without S")
    assert_bits(to_host(m2), m, "meta without S")


def test_sddmm_bf16_exact_integer_scores():
    # integer Q, K: every fp32 dot product is exact, so S is one RNE rounding of an exact
    # value on both sides (pins the GPU's fp32 -> bf16 conversion, ties included)
    snm = _snm()
    rng = np.random.default_rng(21)
    Qi = rng.integers(-8, 9, size=(2, 64, 64)).astype(np.float64)
    Ki = rng.integers(-8, 9, size=(2, 128, 64)).astype(np.float64)
    Q, K = ov.f64_to_bf16(Qi), ov.f64_to_bf16(Ki)
    v, m, S = snm.sddmm_prune_nm_bf16(dev_bf16(Q), dev_bf16(K), 1.0, return_dense=True)
    ovals, ometa, oS = ov.sddmm_prune_nm_bf16(Q, K, 1.0)
    assert_bits(host_bits(S), oS, "S")
    assert_bits(host_bits(v), ovals, "values")
    assert_bits(to_host(m), ometa, "meta")
    # many scores need rounding (|S| > 256 has more than 8 significant bits)
    assert np.count_nonzero(np.abs(np.einsum("bqd,bkd->bqk", Qi, Ki)) > 256) > 1000


def test_sddmm_bf16_identity_keys_exact():
    snm = _snm()
    rng = np.random.default_rng(22)
    Q = workloads.normal_bf16(rng, (2, 48, 64))
    eye = np.ascontiguousarray(np.broadcast_to(ov.f64_to_bf16(np.eye(64)), (2, 64, 64)))
    v, m = snm.sddmm_prune_nm_bf16(dev_bf16(Q), dev_bf16(eye), 0.125)
    ovals, ometa, _ = ov.sddmm_prune_nm_bf16(Q, eye, 0.125)
    assert_bits(host_bits(v), ovals, "values")
    assert_bits(to_host(m), ometa, "meta")


@pytest.mark.parametrize("rows,kept", [(7, 2048), (5, 104), (3, 4096), (2, 5000), (64, 32), (3, 37)])
def test_softmax_bf16(rows, kept):
    snm = _snm()
    x = workloads.normal_bf16(np.random.default_rng(rows + kept), (rows, kept), 3.0)
    t = dev_bf16(x)
    snm.softmax_nm_rows_bf16(t)
    got = ov.bf16_to_f64(host_bits(t))
    ref = ov.softmax_rows(ov.bf16_to_f64(x))
    assert_within(got, ref, (1.01 * U + 1e-5) * ref + 1e-38, f"softmax {rows}x{kept}")


def test_softmax_bf16_constant_row():
    snm = _snm()
    t = dev_bf16(np.full((4, 2048), ov.f64_to_bf16(1.5), dtype=np.uint16))
    snm.softmax_nm_rows_bf16(t)
    assert np.all(host_bits(t) == ov.f64_to_bf16(1.0 / 2048))


def _decode_p(p, meta, lk):
    """float64 probabilities [rows, lk/2] placed at their 2:4 positions -> [rows, lk]."""
    codes = _unpack_codes(meta)[:, : lk // 4].astype(np.int64)
    rows = p.shape[0]
    out = np.zeros((rows, lk // 4, 4))
    rr = np.arange(rows)[:, None]
    gg = np.arange(lk // 4)[None, :]
    pp = p.reshape(rows, lk // 4, 2)
    out[rr, gg, codes & 3] = pp[..., 0]
    out[rr, gg, codes >> 2] = pp[..., 1]
    return out.reshape(rows, lk)


def _spmm_problem(seed, b, R, K, C, sigma=1.0):
    rng = np.random.default_rng(seed)
    A = workloads.normal_bf16(rng, (b, R, K), sigma)
    B = workloads.normal_bf16(rng, (b, K, C))
    values, meta = ov.prune_encode_nm_bf16(A.reshape(b * R, K))
    return values.reshape(b, R, K // 2), meta.reshape(b, R, K // 8), B


def _spmm_bound(values, meta, B):
    b, R, half = values.shape
    K = 2 * half
    refs, bounds = [], []
    for i in range(b):
        Ad = ov.decode_nm_bf16(values[i], meta[i], K)
        Bd = ov.bf16_to_f64(B[i])
        ref = Ad @ Bd
        refs.append(ref)
        bounds.append(1.01 * (gamma(K) * (np.abs(Ad) @ np.abs(Bd)) + U * np.abs(ref)) + 1e-38)
    return np.stack(refs), np.stack(bounds)


@pytest.mark.parametrize("b,R,K,C", [
    (1, 32, 32, 64), (2, 100, 64, 64), (1, 130, 48, 72), (1, 257, 80, 8), (3, 64, 80, 24),
    (1, 40, 256, 128), (1, 200, 512, 136), (2, 129, 2048, 64), (1, 300, 256, 264), (1, 64, 4096, 32),
    (1, 520, 256, 512)])
def test_spmm_bf16_vs_oracle(b, R, K, C):
    snm = _snm()
    values, meta, B = _spmm_problem(R * 7 + K + C, b, R, K, C)
    Y = snm.spmm_nm_bf16(dev_bf16(values), dev(meta), dev_bf16(B))
    ref, bound = _spmm_bound(values, meta, B)
    assert_within(ov.bf16_to_f64(host_bits(Y)), ref, bound, f"spmm bf16 {b}x{R}x{K}x{C}")


def test_spmm_bf16_identity_exact_and_2d():
    # B = I: every output is one product with 1, so Y is the decoded operand, bit for bit
    snm = _snm()
    values, meta, _ = _spmm_problem(31, 1, 96, 128, 8)
    eye = ov.f64_to_bf16(np.eye(128))
    Y = snm.spmm_nm_bf16(dev_bf16(values[0]), dev(meta[0]), dev_bf16(eye))
    dense = ov.decode_nm_bf16(values[0], meta[0], 128)
    assert_bits(host_bits(Y), ov.f64_to_bf16(dense), "identity")


def test_spmm_bf16_empty_reduction_writes_zeros():
    import torch
    snm = _snm()
    values = torch.empty((1, 40, 0), dtype=torch.bfloat16, device="cuda")
    meta = torch.empty((1, 40, 0), dtype=torch.uint8, device="cuda")
    B = torch.empty((1, 0, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 40, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    snm.spmm_nm_bf16(values, meta, B, out=out)
    assert np.all(host_bits(out) == 0)


@pytest.mark.parametrize("b,lq,lk,d", [(2, 128, 128, 64), (1, 512, 512, 64), (3, 96, 96, 32),
                                       (2, 160, 256, 128), (2, 100, 256, 64)])
def test_attention_bf16_end_to_end(b, lq, lk, d):
    # the downstream reference takes the GPU's own scores (the score stage is checked above):
    # the oracle's float64 softmax over them and its product with V
    snm = _snm()
    Q, K, V = _qkv(91 + lq + lk + d, b, lq, lk, d)
    scale = 1.0 / np.sqrt(d)
    dQ, dK, dV = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    O = ov.bf16_to_f64(host_bits(snm.attention_nm_bf16(dQ, dK, dV, scale)))
    Of = ov.bf16_to_f64(host_bits(snm.attention_nm_fused_bf16(dQ, dK, dV, scale)))
    v, m, S = snm.sddmm_prune_nm_bf16(dQ, dK, scale, return_dense=True)
    S, m = host_bits(S), to_host(m)
    P_ref, O_ref = ov.attention_bf16_from_pattern(S, m, V)
    Vd = np.abs(ov.bf16_to_f64(V))
    PV = np.stack([_decode_p(P_ref[i], m[i], lk) for i in range(b)]) @ Vd
    assert_within(O, O_ref, 1.01 * U * (PV + np.abs(O_ref)) + 1e-6, f"attention bf16 {b}x{lq}x{lk}x{d}")
    assert_within(Of, O_ref, 2.02 * U * PV + 1.01 * U * np.abs(O_ref) + 1e-6, "fused")
    snm.softmax_nm_rows_bf16(v)
    P = ov.bf16_to_f64(host_bits(v))
    assert_within(P, P_ref, (1.01 * U + 1e-5) * P_ref + 1e-38, "P")


def test_attention_bf16_workload_sampled_heads():
    # batch 4 x 16 heads, seq 4096, head_dim 64 in bf16, in the launch configuration the
    # benchmark times (unfused and fused); scores and the pattern of 64 sampled query rows
    # of every slice are checked, and O on those rows
    snm = _snm()
    w = workloads.WORKLOADS["attention_2_4"]
    Q, K, V = workloads.attention_qkv_typed(w, "bf16")
    scale = 0.125
    dQ, dK, dV = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    vals, meta, S, rmax = snm.sddmm_prune_nm_bf16(dQ, dK, scale, return_dense=True, return_rowmax=True)
    Of = ov.bf16_to_f64(host_bits(snm.spmm_nm_softmax_bf16(vals, meta, rmax, dV)))
    snm.softmax_nm_rows_bf16(vals)
    O = ov.bf16_to_f64(host_bits(snm.spmm_nm_bf16(vals, meta, dV)))
    S, meta_h, vals_h = host_bits(S), to_host(meta), host_bits(vals)
    rng = np.random.default_rng(7)
    for h in range(Q.shape[0]):
        rows = np.sort(rng.choice(4096, 64, replace=False))
        Sh, mh = S[h:h + 1, rows], meta_h[h:h + 1, rows]
        tau, exact = _score_bound(Q[h:h + 1, rows], K[h:h + 1], scale)
        assert_within(ov.bf16_to_f64(Sh), exact, tau, f"S head {h}")
        sv, sm = ov.prune_encode_nm_bf16(Sh[0])
        assert_bits(mh[0], sm, f"meta head {h}")
        P_ref, O_ref = ov.attention_bf16_from_pattern(Sh, mh, V[h:h + 1])
        PV = _decode_p(P_ref[0], mh[0], 4096) @ np.abs(ov.bf16_to_f64(V[h]))
        assert_within(O[h, rows], O_ref[0], 1.01 * U * (PV + np.abs(O_ref[0])) + 1e-6, f"O head {h}")
        assert_within(Of[h, rows], O_ref[0], 2.02 * U * PV + 1.01 * U * np.abs(O_ref[0]) + 1e-6, f"fused O head {h}")
        assert_within(ov.bf16_to_f64(vals_h[h, rows]), P_ref[0], (1.01 * U + 1e-5) * P_ref[0] + 1e-38, f"P head {h}")
