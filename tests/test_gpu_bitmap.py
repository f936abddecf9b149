"""GPU parity of the bitmap (Coruscant) format: the encoder bit for bit against the oracle,
the product element by element against the oracle's float64 product, edge cases, and the
pages' decode shapes (7168 and 9216 square, 30-70 % sparsity, N = 8) on sampled rows."""
import numpy as np
import pytest

import oracle
from oracle import bitmap as BM
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _check_encode(A, what, lda_pad=0):
    import torch
    snm = _snm()
    R, K = A.shape
    if lda_pad:
        buf = torch.zeros((R, K + lda_pad), dtype=torch.float16, device="cuda")
        buf[:, :K] = to_dev(A)
        dA = buf[:, :K]
    else:
        dA = to_dev(A)
    bm, off, vals = snm.bitmap_encode(dA)
    obm, ooff, ovals = BM.encode_bitmap(A)
    assert_bits_equal(to_host(bm).view(np.uint64), obm, what + " bitmaps")
    assert_bits_equal(to_host(off).view(np.uint32), ooff, what + " offsets")
    assert_bits_equal(to_host(vals), ovals, what + " values")
    return bm, off, vals


@pytest.mark.parametrize("R,K,s", [(16, 64, 0.5), (17, 192, 0.3), (100, 640, 0.7), (33, 1024, 0.0),
                                   (5, 128, 1.0), (64, 4096, 0.5), (3, 64 * 37, 0.6)])
def test_bitmap_encode(R, K, s):
    rng = np.random.default_rng(R * 31 + K)
    A = workloads.normal_f16(rng, (R, K))
    A[rng.random((R, K)) < s] = 0
    _check_encode(A, f"{R}x{K} s={s}")
    _check_encode(A, f"{R}x{K} s={s} padded lda", lda_pad=8)


def test_bitmap_encode_special_values():
    A = np.zeros((4, 128), dtype=np.float16)
    A[0, 3] = np.float16(-0.0)
    A[0, 5] = np.float16(6e-8)
    A[1, :] = np.float16(1.0)
    A[2, 64:] = np.float16(-2.0)
    A[3, ::3] = np.float16(np.inf)
    _check_encode(A, "specials")


@pytest.mark.parametrize("R,K,C,s", [(16, 64, 8, 0.5), (17, 192, 1, 0.3), (100, 640, 16, 0.7),
                                     (64, 4096, 8, 0.5), (130, 64 * 37, 24, 0.6), (48, 1024, 32, 0.0),
                                     (40, 9216, 8, 0.5), (7, 256, 13, 1.0), (8190, 512, 32, 0.5)])
def test_bitmap_spmm(R, K, C, s):
    snm = _snm()
    rng = np.random.default_rng(R + K + C)
    A = workloads.normal_f16(rng, (R, K), 0.02)
    A[rng.random((R, K)) < s] = 0
    B = workloads.normal_f16(rng, (K, C))
    obm, ooff, ovals = BM.encode_bitmap(A)
    ref = BM.spmm_bitmap(obm, ooff, ovals, B)
    bm, off, vals = snm.bitmap_encode(to_dev(A))
    for lay, dB in (("col", to_dev(np.ascontiguousarray(B.T)).t()), ("row", to_dev(B))):
        Y = snm.spmm_bitmap(bm, off, vals, dB)
        assert_fp16_close(to_host(Y), ref, f"bitmap spmm {R}x{K}x{C} s={s} {lay}")


def test_bitmap_spmm_identity_exact():
    # B = I[:, :C]: each output is one product, so Y must be A's first C columns exactly
    snm = _snm()
    rng = np.random.default_rng(4)
    A = workloads.normal_f16(rng, (50, 256))
    A[rng.random(A.shape) < 0.5] = 0
    bm, off, vals = snm.bitmap_encode(to_dev(A))
    for C in (8, 32):
        Bm = np.eye(256, dtype=np.float16)[:, :C].copy()
        Y = to_host(snm.spmm_bitmap(bm, off, vals, to_dev(np.ascontiguousarray(Bm.T)).t()))
        assert np.array_equal(Y.astype(np.float64), A[:, :C].astype(np.float64))


@pytest.mark.parametrize("n,s,N", [(7168, 0.3, 8), (7168, 0.5, 32), (9216, 0.5, 8), (9216, 0.7, 8)])
def test_bitmap_decode_shapes_sampled(n, s, N):
    # the pages' kernel shapes (7168 rows take the 32-row workgroups with column-major B,
    # 9216 the 16-row ones); the encoding of the first and last 64 rows against the oracle
    # (offsets relative to each block's first tile), every column of 96 sampled output rows
    # against A @ B in float64
    snm = _snm()
    A = workloads.pruned_unstructured(11, n, n, s)
    B = workloads.normal_f16(np.random.default_rng(12), (n, N))
    bm, off, vals = snm.bitmap_encode(to_dev(A))
    Y = to_host(snm.spmm_bitmap(bm, off, vals, to_dev(np.ascontiguousarray(B.T)).t()))
    bmh, offh, valh = to_host(bm).view(np.uint64), to_host(off).view(np.uint32).astype(np.int64), to_host(vals)
    T = n // 64
    for r0 in (0, n - 64):
        obm, ooff, ovals = BM.encode_bitmap(A[r0:r0 + 64])
        assert_bits_equal(bmh[r0:r0 + 64], obm, f"bitmaps rows {r0}+")
        rel = offh[r0 * T:(r0 + 64) * T + 1] - offh[r0 * T]
        assert np.array_equal(rel, ooff.astype(np.int64)), f"offsets rows {r0}+"
        assert_bits_equal(valh[offh[r0 * T]:offh[(r0 + 64) * T]], ovals, f"values rows {r0}+")
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([rng.choice(n, 96, replace=False), [0, n - 1]]))
    ref = A[rows].astype(np.float64) @ B.astype(np.float64)
    assert_fp16_close(Y[rows], ref, f"bitmap {n}x{n} s={s} N={N} sampled rows")
    assert int(offh[-1]) == int(np.sum((np.count_nonzero(A.reshape(n * T, 64), axis=1) + 7) // 8 * 8))


def test_bitmap_spmm_empty_reduction_writes_zeros():
    """K = 0 through the C entry point with the (empty) bitmap arrays passed as NULL, as the
    header allows: every output is 0, both B layouts, one and two column tiles."""
    import torch
    from structured_sparse_matrix_amd._lib import load, check
    lib = load()
    stream = torch.cuda.current_stream().cuda_stream
    for C, layout in ((8, 1), (32, 1), (8, 0), (24, 0)):
        R = 40
        B = torch.zeros((max(C, 8), 8), dtype=torch.float16, device="cuda")   # a readable pointer, never read
        Y = torch.full((R, C), 7.0, dtype=torch.float16, device="cuda")
        ldb = 8 if layout == 1 else C   # column-major B needs ldb >= K (0) and ldb % 8 == 0
        check("snm_spmm_bitmap", lib.snm_spmm_bitmap(None, None, None, R, 0, B.data_ptr(), C, ldb, layout,
                                                     Y.data_ptr(), C, stream))
        torch.cuda.synchronize()
        assert not to_host(Y).view(np.uint16).any(), f"C={C} layout={layout}"
