"""GPU parity: 2:4 and V:2:M prune/encode must match the oracle bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _check_nm(A, what):
    snm = _snm()
    v, m = snm.prune_encode_nm(to_dev(A))
    ov, om = oracle.prune_encode_nm(A)
    assert_bits_equal(to_host(v), ov, what + " values")
    assert_bits_equal(to_host(m), om, what + " meta")


@pytest.mark.parametrize("R,K", [(1, 16), (3, 48), (7, 16), (33, 80), (256, 256), (100, 4096)])
def test_nm_small_and_ragged(R, K):
    _check_nm(workloads.small_matrix(R * 7 + K, (R, K)), f"{R}x{K}")


def test_nm_ties_signed_zeros_and_specials():
    A = workloads.ties_matrix(11, (64, 128), levels=3)
    _check_nm(A, "ties")
    B = np.zeros((8, 32), dtype=np.float16)
    B[0, :8] = [np.nan, 1.0, -np.inf, 2.0, 0.0, -0.0, 0.0, -0.0]
    B[1, :8] = [6e-8, -6e-8, 1e-7, 0.0, 65504, -65504, np.inf, 1.0]     # subnormals, max, inf
    B[2, :4] = [-0.0, 0.0, -0.0, 0.0]
    _check_nm(B, "specials")


def test_nm_strided_rows():
    snm = _snm()
    import torch
    A = workloads.small_matrix(5, (64, 96))
    big = torch.zeros((64, 136), dtype=torch.float16, device="cuda")
    big[:, :96] = to_dev(A)
    v, m = snm.prune_encode_nm(big[:, :96])         # lda = 136
    ov, om = oracle.prune_encode_nm(A)
    assert_bits_equal(to_host(v), ov, "strided values")
    assert_bits_equal(to_host(m), om, "strided meta")


def test_nm_workload_tiny():
    A, _ = workloads.weight_and_activations(workloads.WORKLOADS["nm_tiny"])
    _check_nm(A, "nm_tiny 256x256")


def test_nm_workload_decode_full():
    # 4096 x 4096, sigma 0.02: thousands of exact ties and fp16 subnormals
    A, _ = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    assert np.count_nonzero(np.abs(A) < np.float16(6.1e-5)) > 0
    _check_nm(A, "nm_decode 4096x4096")


def _check_vnm(A, V, M, what):
    snm = _snm()
    v, mi, cl = snm.prune_encode_vnm(to_dev(A), V, M)
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    assert_bits_equal(to_host(cl), ocl, what + " colloc")
    assert_bits_equal(to_host(mi), omi, what + " midx")
    assert_bits_equal(to_host(v), ov, what + " values")


@pytest.mark.parametrize("R,K,V,M", [
    (64, 64, 64, 8), (128, 512, 64, 8), (256, 1024, 128, 16), (32, 160, 32, 10),
    (16, 4096, 16, 256), (8, 64, 1, 4), (4, 128, 2, 8), (96, 256, 32, 4), (128, 320, 64, 5),
    # the largest V; an odd V
    (512, 256, 256, 16), (6, 64, 3, 8),
])
def test_vnm_small(R, K, V, M):
    _check_vnm(workloads.small_matrix(R + K + V + M, (R, K), 0.02), V, M, f"{R}x{K} V{V} M{M}")


def test_vnm_padded_rows_odd_m():
    # K = 460, M = 5: several workgroup chunks, the last one 12 groups = 60 columns (not a
    # multiple of 8 elements); A is a view with leading dimension 464
    import torch
    snm = _snm()
    R, K, V, M = 128, 460, 64, 5
    A = workloads.small_matrix(77, (R, K), 0.02)
    buf = torch.zeros((R, 464), dtype=torch.float16, device="cuda")
    buf[:, :K] = to_dev(A)
    v, mi, cl = snm.prune_encode_vnm(buf[:, :K], V, M)
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    assert_bits_equal(to_host(cl), ocl, "padded colloc")
    assert_bits_equal(to_host(mi), omi, "padded midx")
    assert_bits_equal(to_host(v), ov, "padded values")


def test_vnm_ties():
    _check_vnm(workloads.ties_matrix(3, (128, 256), levels=3), 64, 8, "ties V64 M8")


def test_vnm_m4_equals_nm():
    snm = _snm()
    A = workloads.small_matrix(9, (64, 128))
    v, mi, cl = snm.prune_encode_vnm(to_dev(A), 32, 4)
    v2, m2 = snm.prune_encode_nm(to_dev(A))
    assert_bits_equal(to_host(v), to_host(v2), "M=4 values")
    assert_bits_equal(to_host(mi), to_host(m2), "M=4 meta")
    assert np.all(to_host(cl) == np.arange(4, dtype=np.uint8))


def test_vnm_workload_64_2_8_full():
    A, _ = workloads.weight_and_activations(workloads.WORKLOADS["vnm_64_2_8"])
    _check_vnm(A, 64, 8, "vnm 11008x4096 V64 M8")


def test_vnm_workload_128_2_16_full():
    w = workloads.WORKLOADS["vnm_128_2_16"]
    A = workloads.normal_f16(np.random.default_rng(w.seed), (w.R, w.K), w.sigma_a)
    _check_vnm(A, 128, 16, "vnm 8192x8192 V128 M16")


def test_encode_is_deterministic():
    snm = _snm()
    A = to_dev(workloads.small_matrix(12, (512, 1024)))
    a1 = [to_host(x) for x in snm.prune_encode_nm(A)]
    a2 = [to_host(x) for x in snm.prune_encode_nm(A)]
    for x, y in zip(a1, a2):
        assert_bits_equal(x, y, "repeat")


def _permuted_columns(seed, V, M, G, big):
    """Every group's M columns hold row permutations of one column of values, so the exact
    column sums of squares are equal within a group. small: |a| <= 1/16, every float64 sum
    of the squares is exact in any order (the scores tie; the lower column wins). big: each
    column mixes values near 8 with values near 2^-18, so the float64 row-order sum rounds
    and permuted columns get scores that differ in their last bits."""
    rng = np.random.default_rng(seed)
    A = np.empty((V, G * M), dtype=np.float16)
    for g in range(G):
        if big:
            x = np.where(rng.random(V) < 0.5, rng.uniform(4, 12, V), rng.uniform(1, 2, V) * 2.0 ** -18)
        else:
            x = rng.uniform(-1, 1, V) / 16
        x = (x * np.where(rng.random(V) < 0.5, -1, 1)).astype(np.float16)
        for j in range(M):
            A[:, g * M + j] = x[rng.permutation(V)]
    return A


@pytest.mark.parametrize("big", [False, True])
def test_vnm_scores_order_of_summation(big):
    """The encoder sums column scores in any order where float64 is exact and in row order
    where it is not; both must give the oracle's column selection bit for bit."""
    V, M, G = 128, 16, 32
    A = _permuted_columns(41 + big, V, M, G, big)
    A = np.concatenate([A, A[::-1]], axis=0)   # two V-blocks
    _check_vnm(A, V, M, f"permuted columns, {'rounded' if big else 'exact'} sums")
    if not big:   # every group's scores tie: the lowest four columns
        ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
        assert np.all(ocl.reshape(-1, 4) == np.arange(4, dtype=np.uint8))


@pytest.mark.parametrize("R,K,V,M,pad", [
    (8192, 3104, 32, 8, 0),     # 388 groups per row: the last workgroup chunk is ragged
    (8192, 2048, 128, 16, 8),   # rows 8 elements longer than K (a view of a wider array)
    (4096, 4096, 64, 4, 0),     # M = 4: every column kept
])
def test_vnm_encoder_large_shapes(R, K, V, M, pad):
    """Large encodes, canonical and row-group interleaved: many workgroup chunks with a
    ragged last one, rows of a wider array, M = 4."""
    import torch
    snm = _snm()
    A = workloads.small_matrix(R + K + V + M + pad, (R, K), 0.02)
    buf = torch.zeros((R, K + pad), dtype=torch.float16, device="cuda")
    buf[:, :K] = to_dev(A)
    v, mi, cl = snm.prune_encode_vnm(buf[:, :K], V, M)
    vt, mit, clt = snm.prune_encode_vnm_tiled(buf[:, :K], V, M) if V % 32 == 0 else (None, None, None)
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    what = f"{R}x{K} V{V} M{M} pad {pad}"
    assert_bits_equal(to_host(cl), ocl, what + " colloc")
    assert_bits_equal(to_host(mi), omi, what + " midx")
    assert_bits_equal(to_host(v), ov, what + " values")
    if vt is not None:
        from _vnm_tiled import untile
        uv, umi = untile(to_host(vt), to_host(mit), M)
        assert_bits_equal(to_host(clt), ocl, what + " colloc (interleaved)")
        assert_bits_equal(umi, omi, what + " midx (interleaved)")
        assert_bits_equal(uv, ov, what + " values (interleaved)")
