"""GPU parity of the row-group interleaved V:2:M storage (snm_prune_encode_vnm_tiled,
snm_spmm_vnm_tiled): the encoder must equal the oracle's canonical arrays after the host
model un-tiles them (bit for bit), and the product on arrays the host model tiles from the
oracle's encoding must match the float64 oracle. Shapes cover every wide-kernel tile
(V = 32 / 64 / 128, 128-, 64- and 32-position stages), ragged last stages and column tiles,
both encoder kernels (tile in LDS or not), and the two full-size V:2:M workloads."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal
from _vnm_tiled import tile, untile

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


@pytest.mark.parametrize("R,K,V,M", [(64, 256, 32, 8), (128, 512, 64, 16), (256, 1024, 128, 16),
                                     (96, 320, 32, 10), (64, 160, 32, 5), (256, 640, 256, 40),
                                     (128, 400, 128, 100)])
def test_vnm_tiled_encode(R, K, V, M):
    snm = _snm()
    A = workloads.small_matrix(R + K + V + M, (R, K), 0.02)
    vt, mt, cl = snm.prune_encode_vnm_tiled(to_dev(A), V, M)
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    v, mi = untile(to_host(vt), to_host(mt), M)
    assert_bits_equal(v, ov, f"values {R}x{K} V{V} M{M}")
    assert_bits_equal(mi, omi, f"midx {R}x{K} V{V} M{M}")
    assert_bits_equal(to_host(cl), ocl, f"colloc {R}x{K} V{V} M{M}")


@pytest.mark.parametrize("R,K,C,V,M", [
    (64, 288, 64, 32, 8),      # 4K/M = 144: 128-position stages, ragged
    (128, 288, 136, 64, 8),    # 64-position stages, ragged, ragged column tile
    (256, 320, 256, 128, 16),  # 4K/M = 80: ragged
    (256, 2048, 200, 128, 16),
    (384, 640, 136, 128, 10),
    (192, 2048, 64, 64, 8),
    (128, 204, 520, 64, 17),
    (32, 256, 8, 32, 8),       # a single 8-column tile
])
def test_vnm_tiled_spmm(R, K, C, V, M):
    snm = _snm()
    A = workloads.small_matrix(3 * R + K + C + V + M, (R, K), 0.02)
    B = workloads.small_matrix(R + K + C, (K, C))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    vt, mt = tile(ov, omi, M)
    Y = snm.spmm_vnm_tiled(to_dev(vt), to_dev(mt), to_dev(ocl), to_dev(B), V, M)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"tiled vnm {R}x{K}x{C} V{V} M{M}")


def test_vnm_tiled_identity_is_exact_decode():
    snm = _snm()
    V, M, K, C = 64, 8, 768, 256
    A = workloads.small_matrix(91, (2 * V, K))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    vt, mt = tile(ov, omi, M)
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K).astype(np.float64)
    Y = snm.spmm_vnm_tiled(to_dev(vt), to_dev(mt), to_dev(ocl), to_dev(np.eye(K, dtype=np.float16)[:, :C].copy()), V, M)
    assert np.array_equal(to_host(Y).astype(np.float64), dense[:, :C])


def test_vnm_tiled_workload_64_2_8_full():
    snm = _snm()
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["vnm_64_2_8"])
    vt, mt, cl = snm.prune_encode_vnm_tiled(to_dev(A), 64, 8)
    ov, omi, ocl = oracle.prune_encode_vnm(A, 64, 8)
    v, mi = untile(to_host(vt), to_host(mt), 8)
    assert_bits_equal(v, ov, "values")
    assert_bits_equal(mi, omi, "midx")
    Y = snm.spmm_vnm_tiled(vt, mt, cl, to_dev(B), 64, 8)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, 64, 8, B), "tiled vnm_64_2_8")


def test_vnm_tiled_workload_128_2_16_sampled_rows():
    # 8192 x 8192 x 4096 in the launch configuration the benchmark times (128 x 256 tiles)
    snm = _snm()
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["vnm_128_2_16"])
    vt, mt, cl = snm.prune_encode_vnm_tiled(to_dev(A), 128, 16)
    Y = snm.spmm_vnm_tiled(vt, mt, cl, to_dev(B), 128, 16)
    ov, omi, ocl = oracle.prune_encode_vnm(A, 128, 16)
    v, mi = untile(to_host(vt), to_host(mt), 16)
    assert_bits_equal(v, ov, "values")
    assert_bits_equal(mi, omi, "midx")
    rows = np.sort(np.random.default_rng(1).choice(8192, size=512, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 31, 32, 127, 128, 8191]]))
    Yh = to_host(Y)[rows]
    dense = oracle.decode_vnm(ov, omi, ocl, 128, 16, 8192)[rows]
    ref = dense.astype(np.float64) @ B.astype(np.float64)
    assert_fp16_close(Yh, ref, "tiled vnm_128_2_16 sampled rows")
    # same kernel, same arithmetic order: identical to the canonical storage's product
    v0, m0, c0 = snm.prune_encode_vnm(to_dev(A), 128, 16)
    Y0 = snm.spmm_vnm(v0, m0, c0, to_dev(B), 128, 16)
    assert np.array_equal(to_host(Y0).view(np.uint16), to_host(Y).view(np.uint16))
