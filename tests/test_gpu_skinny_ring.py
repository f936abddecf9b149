"""GPU parity of the decode product's LDS-ring kernel (column-major B = the activations X[C][K]
as stored, C <= 32, one product; operand-major A with K a multiple of 512, canonical A with K a
multiple of 1024, K up to 8192): one to sixteen ring phases, ragged rows and columns (copies of
columns past C come from column C - 1, canonical rows past R read row R - 1), partially filled
copy waves, padded column strides, the exact decode with B = I, and the shapes that fall back
to the register kernel."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _colmajor(X, pad=0):
    """X [C][K] on the device as a K x C column-major view, columns `pad` elements apart
    beyond K."""
    C, K = X.shape
    Xp = np.zeros((C, K + pad), dtype=np.float16)
    Xp[:, :K] = X
    return to_dev(Xp)[:, :K].t()


@pytest.mark.parametrize("R,K,C", [(16, 512, 8), (33, 1024, 5), (100, 1536, 16), (48, 2048, 20),
                                   (17, 4096, 1), (64, 8192, 32), (80, 2560, 31), (1, 512, 17)])
def test_ring_spmm(R, K, C):
    snm = _snm()
    A = workloads.small_matrix(R * 5 + K + C, (R, K), 0.02)
    X = workloads.small_matrix(R + K * 5 + C, (C, K))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    Y = snm.spmm_nm_tiled(vt, mt, R, _colmajor(X))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"ring {R}x{K}x{C}")


@pytest.mark.parametrize("pad", [8, 64, 520])
def test_ring_padded_columns(pad):
    snm = _snm()
    R, K, C = 64, 3072, 24
    A = workloads.small_matrix(91 + pad, (R, K), 0.02)
    X = workloads.small_matrix(92 + pad, (C, K))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    Y = snm.spmm_nm_tiled(vt, mt, R, _colmajor(X, pad))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"ring pad {pad}")


@pytest.mark.parametrize("C", [16, 32])
def test_ring_identity_is_exact_decode(C):
    # B = the first C columns of the 1024 x 1024 identity: every output is one stored value
    snm = _snm()
    R, K = 48, 1024
    A = workloads.small_matrix(93 + C, (R, K))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    X = np.ascontiguousarray(np.eye(K, dtype=np.float16)[:, :C].T)
    Y = snm.spmm_nm_tiled(vt, mt, R, _colmajor(X))
    ov, om = oracle.prune_encode_nm(A)
    ref = oracle.decode_nm(ov, om, K)[:, :C]
    assert np.array_equal(to_host(Y).astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("R,K,C", [(32, 1040, 8), (32, 8704, 16), (16, 256, 32)])
def test_ring_ineligible_shapes_fall_back(R, K, C):
    # K not a multiple of 512, K past 8192, K below one phase: the register kernel
    snm = _snm()
    A = workloads.small_matrix(R + K + 7, (R, K), 0.02)
    X = workloads.small_matrix(R + K + 8, (C, K))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    Y = snm.spmm_nm_tiled(vt, mt, R, _colmajor(X))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"fallback {R}x{K}x{C}")


def _canonical(A, X, pad=0):
    snm = _snm()
    v, m = snm.prune_encode_nm(to_dev(A))
    return to_host(snm.spmm_nm(v, m, _colmajor(X, pad)))


@pytest.mark.parametrize("R,K,C", [(16, 1024, 8), (33, 2048, 5), (100, 3072, 16), (48, 2048, 20),
                                   (17, 4096, 1), (64, 8192, 32), (1, 1024, 17), (4096, 4096, 32)])
def test_ring_spmm_canonical(R, K, C):
    A = workloads.small_matrix(R * 7 + K + C, (R, K), 0.02)
    X = workloads.small_matrix(R + K * 7 + C, (C, K))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(_canonical(A, X), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)),
                      f"canonical ring {R}x{K}x{C}")


def test_ring_canonical_padded_columns_and_identity():
    R, K, C = 40, 2048, 24
    A = workloads.small_matrix(95, (R, K), 0.02)
    X = workloads.small_matrix(96, (C, K))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(_canonical(A, X, pad=72), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), "canonical pad")
    Xi = np.ascontiguousarray(np.eye(K, dtype=np.float16)[:, :32].T)
    ref = oracle.decode_nm(ov, om, K)[:, :32]
    assert np.array_equal(_canonical(A, Xi).astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("R,K,C", [(32, 1536, 8), (32, 9216, 16)])
def test_ring_canonical_ineligible_shapes_fall_back(R, K, C):
    # K not a multiple of 1024, K past 8192: the register kernel
    A = workloads.small_matrix(R + K + 9, (R, K), 0.02)
    X = workloads.small_matrix(R + K + 10, (C, K))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(_canonical(A, X), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"canonical fallback {K}")
