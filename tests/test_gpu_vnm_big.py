"""GPU parity of the large-tile V:2:M product (spmm_vnm_big.hip: 128 x 512 workgroup tiles,
accumulators in the AGPR file), which the V:2:M entry points select for V % 128 == 0 when
K' = 4K/M is a multiple of 32 in [256, 12224] and the grid has at least 256 workgroups.
Shapes cover the shortest reduction (two rounds of four stages, no steady round), longer
ones, ragged last rounds (K' not a multiple of 128: one to three padding stages whose
copies repeat the last stage and whose products are skipped), a ragged last column tile, a grid whose size is not a multiple of 8 (no XCD
renumbering), both storages of A, and the exact decode with B = I. The configuration-5
workload and the GPT-3 layer shape, which also run this kernel, are checked in
test_gpu_vnm_tiled.py, test_gpu_spmm.py and test_gpu_vnm_sweep.py."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal
from _vnm_tiled import tile

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


@pytest.mark.parametrize("R,K,C,M", [
    (4096, 1024, 4096, 16),    # K' = 256: the first and last rounds only
    (4096, 2048, 4088, 16),    # K' = 512: two steady rounds; ragged last column tile
    (4096, 1024, 4096, 8),     # K' = 512, 2:8
    (8576, 512, 1544, 8),      # 67 V-blocks x 4 column tiles = 268 workgroups (no renumbering)
    (4096, 720, 4096, 10),     # K' = 288: nine stages, the last round padded by three
    (4096, 1600, 4096, 20),    # K' = 320: ten stages, padded by two
    (4096, 1408, 4088, 16),    # K' = 352: eleven stages, padded by one; ragged column tile
])
@pytest.mark.parametrize("storage", ["canonical", "interleaved"])
def test_big_matches_oracle(R, K, C, M, storage):
    snm = _snm()
    V = 128
    print(f"big {R}x{K}x{C} V{V} M{M} {storage}", flush=True)
    A = workloads.small_matrix(R + K + C + M, (R, K), 0.02)
    B = workloads.small_matrix(R + 2 * K + C, (K, C))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    if storage == "canonical":
        Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    else:
        vt, mt = tile(ov, omi, M)
        Y = snm.spmm_vnm_tiled(to_dev(vt), to_dev(mt), to_dev(ocl), to_dev(B), V, M)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"{R}x{K}x{C} M{M} {storage}")


@pytest.mark.parametrize("storage", ["canonical", "interleaved"])
@pytest.mark.parametrize("K", [1024, 1408])
def test_big_identity_is_exact_decode(storage, K):
    # B = I: every output is one product, so the kernel must return the decoded matrix
    # exactly (16384 x 1024 with 2:16: 128 V-blocks x 2 column tiles = 256 workgroups;
    # K = 1408: K' = 352, a last round with one padding stage, 384 workgroups)
    snm = _snm()
    R, V, M = 16384, 128, 16
    A = workloads.small_matrix(99, (R, K))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K)
    B = np.eye(K, dtype=np.float16)
    if storage == "canonical":
        Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    else:
        vt, mt = tile(ov, omi, M)
        Y = snm.spmm_vnm_tiled(to_dev(vt), to_dev(mt), to_dev(ocl), to_dev(B), V, M)
    assert_bits_equal(to_host(Y), dense, f"B = I, {storage}")


@pytest.mark.parametrize("R,K,C,V,M", [
    (1024, 4160, 4096, 64, 20),    # K' = 832: 13 stages of 64, the last round padded by three
    (1024, 1152, 4096, 64, 8),     # K' = 576: nine stages, padded by three
    (1024, 2560, 4088, 128, 16),   # K' = 640: ten stages, padded by two; V = 128 on 64-row tiles
    (1024, 1760, 4096, 64, 10),    # K' = 704: eleven stages, padded by one
])
@pytest.mark.parametrize("storage", ["canonical", "interleaved"])
def test_big64_ragged_rounds_match_oracle(R, K, C, V, M, storage):
    # the 64-row large-tile kernel (16 x 16 = 256 workgroups, above its 128-workgroup rule)
    snm = _snm()
    print(f"big64 {R}x{K}x{C} V{V} M{M} {storage}", flush=True)
    A = workloads.small_matrix(R + 3 * K + C + M, (R, K), 0.02)
    B = workloads.small_matrix(R + 5 * K + C, (K, C))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    if storage == "canonical":
        Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    else:
        vt, mt = tile(ov, omi, M)
        Y = snm.spmm_vnm_tiled(to_dev(vt), to_dev(mt), to_dev(ocl), to_dev(B), V, M)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"big64 {R}x{K}x{C} M{M} {storage}")
