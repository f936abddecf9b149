"""GPU parity of the operand-major ("tiled") 2:4 storage: encode must equal the oracle's
canonical arrays after a host-side un-tiling written from the layout definition in snm.h,
padding must be zero, and the product must match the float64 oracle."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def untile(values_t, meta_t, R, K):
    """Operand-major -> canonical. Block (rt, kc), lane 16q + i, slot j holds canonical value
    (row 16rt + i, column 32kc + 8q + j); its metadata word is canonical word 4kc + q."""
    RT, KC = -(-R // 16), -(-K // 64)
    vt = np.asarray(values_t).reshape(RT, KC, 4, 16, 8)
    vals = vt.transpose(0, 3, 1, 2, 4).reshape(RT * 16, KC * 32)
    mt = np.asarray(meta_t).view(np.uint16).reshape(RT, KC, 4, 16)
    words = mt.transpose(0, 3, 1, 2).reshape(RT * 16, KC * 4)
    return vals, words


def _check_encode(A):
    snm = _snm()
    R, K = A.shape
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    vals, words = untile(to_host(vt), to_host(mt), R, K)
    ov, om = oracle.prune_encode_nm(A)
    assert_bits_equal(vals[:R, :K // 2], ov, "values")
    assert_bits_equal(np.ascontiguousarray(words[:R, :K // 16]).view(np.uint8), om, "meta")
    # padding rows / positions are zero
    assert not vals[R:].view(np.uint16).any() and not vals[:, K // 2:].view(np.uint16).any()
    assert not words[R:].any() and not words[:, K // 16:].any()


@pytest.mark.parametrize("R,K", [(16, 64), (1, 16), (33, 80), (100, 4096), (48, 1040)])
def test_tiled_encode(R, K):
    _check_encode(workloads.small_matrix(R + K, (R, K)))


def test_tiled_encode_ties_and_decode_workload():
    _check_encode(workloads.ties_matrix(7, (40, 192), levels=3))
    A, _ = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    _check_encode(A)


@pytest.mark.parametrize("R,K,C", [(16, 64, 8), (33, 80, 5), (100, 4096, 16), (64, 1040, 32),
                                   (17, 208, 24), (64, 512, 40), (130, 1040, 100), (32, 256, 300)])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_tiled_spmm(R, K, C, layout):
    snm = _snm()
    A = workloads.small_matrix(R * 3 + K + C, (R, K))
    B = workloads.small_matrix(R + K * 3 + C, (K, C))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    Bd = to_dev(B) if layout == "row" else to_dev(np.ascontiguousarray(B.T)).t()
    Y = snm.spmm_nm_tiled(vt, mt, R, Bd)
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), f"tiled {R}x{K}x{C} {layout}")


def test_tiled_identity_is_exact_decode():
    snm = _snm()
    A = workloads.small_matrix(77, (40, 128))
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    for C, Bd in ((128, to_dev(np.eye(128, dtype=np.float16))),):
        Y = snm.spmm_nm_tiled(vt, mt, 40, Bd)
        ov, om = oracle.prune_encode_nm(A)
        assert np.array_equal(to_host(Y).astype(np.float64), oracle.decode_nm(ov, om, 128).astype(np.float64))
    # narrow products (C <= 32 path): B = the first 16 columns of the identity
    Y = snm.spmm_nm_tiled(vt, mt, 40, to_dev(np.eye(128, dtype=np.float16)[:, :16].copy()))
    ov, om = oracle.prune_encode_nm(A)
    assert np.array_equal(to_host(Y).astype(np.float64), oracle.decode_nm(ov, om, 128)[:, :16].astype(np.float64))


def test_tiled_decode_workload_full():
    # the benchmark's configuration: 4096 x 4096, N in {8, 16, 32}, B as X[N][K]
    snm = _snm()
    A, Bs = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    ov, om = oracle.prune_encode_nm(A)
    for B in Bs:
        ref = oracle.spmm_nm(ov, om, B)
        Y = snm.spmm_nm_tiled(vt, mt, 4096, to_dev(np.ascontiguousarray(B.T)).t())
        assert_fp16_close(to_host(Y), ref, f"tiled decode N={B.shape[1]} col-major")
        Y = snm.spmm_nm_tiled(vt, mt, 4096, to_dev(B))
        assert_fp16_close(to_host(Y), ref, f"tiled decode N={B.shape[1]} row-major")
