"""GPU parity over the general V:N:M sweep (VENOM, Sec. 4 ablations, Fig. 9 and Fig. 10):
every (V, M) of the sweep, V in {32, 64, 128} and M in {5, 7, 8, 10, 20, 40, 100}.

Small cases compare the encoder bit for bit and the product element by element with the
oracle, on both product paths (wide outputs through the LDS-ring kernel, narrow outputs
through the general kernel). Full-size cases use the sweep's own shapes and compare the
encoding of whole V-blocks and sampled output rows."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _a_padded_lda(A):
    """A device view of A whose leading dimension is rounded up to a multiple of 8 (the
    encoder's alignment rule): odd M gives K = 4M * k that need not be one."""
    import torch
    R, K = A.shape
    lda = -(-K // 8) * 8
    buf = torch.zeros((R, lda), dtype=torch.float16, device="cuda")
    buf[:, :K] = to_dev(A)
    return buf[:, :K]


@pytest.mark.parametrize("V", workloads.SWEEP_V)
@pytest.mark.parametrize("M", workloads.SWEEP_M)
def test_sweep_pattern_small(V, M):
    snm = _snm()
    R = 2 * V + V          # three V-blocks
    K = workloads.pad_k(6 * 4 * M + 1, M)    # several groups of 4M, a ragged last stage
    seed = 5000 + V * 1000 + M
    A = workloads.small_matrix(seed, (R, K), 0.02)
    v, mi, cl = snm.prune_encode_vnm(_a_padded_lda(A), V, M)
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    assert_bits_equal(to_host(cl), ocl, f"V{V} M{M} colloc")
    assert_bits_equal(to_host(mi), omi, f"V{V} M{M} midx")
    assert_bits_equal(to_host(v), ov, f"V{V} M{M} values")
    for C in (264, 24):
        B = workloads.small_matrix(seed + C, (K, C))
        Y = snm.spmm_vnm(v, mi, cl, to_dev(B), V, M)
        assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"V{V} M{M} C{C}")


@pytest.mark.parametrize("V,M", [(32, 8), (32, 40), (64, 10), (128, 7)])
def test_sweep_pattern_identity_exact(V, M):
    # B = I: every output is one product, so the kernel must reproduce the decode exactly
    snm = _snm()
    K = workloads.pad_k(512, M)
    A = workloads.small_matrix(V + M, (2 * V, K))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K).astype(np.float64)
    C = 136
    B = np.eye(K, dtype=np.float16)[:, :C].copy()
    Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    assert np.array_equal(to_host(Y).astype(np.float64), dense[:, :C])


@pytest.mark.parametrize("family,V,M", [("fig10", 32, 7), ("fig10", 64, 20), ("fig10", 128, 100),
                                        ("fig9", 128, 10)])
def test_sweep_full_size(family, V, M):
    # the sweep's own shapes (fig9 at its largest K): the whole encoding bit for bit, and
    # 96 sampled output rows (every column) against the oracle's product
    snm = _snm()
    pts = [p for p in workloads.vnm_sweep() if p[0] == family and p[4] == V and p[5] == M]
    _, R, K, C, _, _ = pts[-1]
    rng = np.random.default_rng(7000 + V + M)
    A = workloads.normal_f16(rng, (R, K), 0.02)
    B = workloads.normal_f16(rng, (K, C), 1.0)
    v, mi, cl = snm.prune_encode_vnm(_a_padded_lda(A), V, M)
    Y = to_host(snm.spmm_vnm(v, mi, cl, to_dev(B), V, M))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    assert_bits_equal(to_host(cl), ocl, "colloc")
    assert_bits_equal(to_host(mi), omi, "midx")
    assert_bits_equal(to_host(v), ov, "values")
    rows = np.unique(np.concatenate([np.sort(rng.choice(R, 96, replace=False)), [0, V - 1, V, R - 1]]))
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K)[rows].astype(np.float64)
    assert_fp16_close(Y[rows], dense @ B.astype(np.float64), f"{family} {R}x{K}x{C} V{V} M{M} sampled rows")


def test_sweep_gpt3_layer_m8():
    # The larger problem the pages repeat the ablation on (36864 x 12288 x 4096, V = 128,
    # 2:8; column-loc of a V-block is 6144 bytes, the largest any test stages): the whole
    # encoding bit for bit (compared 32 V-blocks at a time), then 96 sampled output rows
    # and the first/last rows of V-blocks (every column) against the oracle's product, on
    # both storages (canonical and row-group interleaved).
    snm = _snm()
    (_, R, K, C, V, M), = [p for p in workloads.vnm_sweep() if p[0] == "gpt3" and p[5] == 8]
    rng = np.random.default_rng(7777)
    A = workloads.normal_f16(rng, (R, K), 0.02)
    B = workloads.normal_f16(rng, (K, C), 1.0)
    Ad, Bd = to_dev(A), to_dev(B)
    v, mi, cl = snm.prune_encode_vnm(Ad, V, M)
    Y = to_host(snm.spmm_vnm(v, mi, cl, Bd, V, M))
    vt, mit, clt = snm.prune_encode_vnm_tiled(Ad, V, M)
    Yt = to_host(snm.spmm_vnm_tiled(vt, mit, clt, Bd, V, M))
    del Ad
    v, mi, cl = to_host(v), to_host(mi), to_host(cl)
    assert_bits_equal(to_host(clt), cl, "colloc of the interleaved encode")
    step = 32 * V
    for r0 in range(0, R, step):
        ov, omi, ocl = oracle.prune_encode_vnm(A[r0:r0 + step], V, M)
        assert_bits_equal(cl[r0 // V:(r0 + step) // V], ocl, f"colloc rows {r0}+")
        assert_bits_equal(mi[r0:r0 + step], omi, f"midx rows {r0}+")
        assert_bits_equal(v[r0:r0 + step], ov, f"values rows {r0}+")
    rows = np.unique(np.concatenate([np.sort(rng.choice(R, 96, replace=False)), [0, V - 1, V, R - V, R - 1]]))
    dense = oracle.decode_vnm(v[rows], mi[rows], np.repeat(cl, V, axis=0)[rows], 1, M, K).astype(np.float64)
    ref = dense @ B.astype(np.float64)
    assert_fp16_close(Y[rows], ref, f"gpt3 {R}x{K}x{C} V{V} M{M} sampled rows")
    assert_fp16_close(Yt[rows], ref, f"gpt3 {R}x{K}x{C} V{V} M{M} sampled rows, interleaved storage")
