"""Pins of the bitmap-format oracle (Coruscant, Sec. 3.1, Fig. 7, Sec. 3.2): the page's
compression figures, round trips, brute-force products and the format's invariants."""
import numpy as np
import pytest

from oracle import bitmap as BM
import workloads


def _with_nnz_per_tile(counts, seed=0):
    """One row per entry of counts: a 64-wide tile with that many random non-zeros."""
    rng = np.random.default_rng(seed)
    A = np.zeros((len(counts), 64), dtype=np.float16)
    for r, c in enumerate(counts):
        pos = rng.choice(64, size=c, replace=False)
        A[r, pos] = (rng.standard_normal(c) + np.sign(rng.standard_normal(c)) * 3).astype(np.float16)
    return A


def test_page_compression_figures():
    # Sec. 3.1: values + 64-bit bitmaps take 56.25 % of the dense fp16 matrix at 50 %
    # sparsity and 36.25 % at 70 % (19.2 non-zeros per 64-element tile on average)
    A = _with_nnz_per_tile([32] * 10)
    bm, off, vals = BM.encode_bitmap(A)
    nnz = sum(bin(int(b)).count("1") for b in bm.ravel())
    assert nnz == 320
    assert (nnz * 2 + bm.size * 8) / A.nbytes == 0.5625
    assert BM.format_bytes(bm, off, vals, with_offsets=False) / A.nbytes == 0.5625   # 32 needs no padding
    A = _with_nnz_per_tile([19, 19, 19, 19, 20] * 4, seed=1)
    bm, off, vals = BM.encode_bitmap(A)
    nnz = sum(bin(int(b)).count("1") for b in bm.ravel())
    assert abs((nnz * 2 + bm.size * 8) / A.nbytes - 0.3625) < 1e-12
    # with the padding to multiples of 8 values the stored size is at most 14 B per tile more
    unpadded = nnz * 2 + bm.size * 8
    assert unpadded <= BM.format_bytes(bm, off, vals, with_offsets=False) <= unpadded + 14 * bm.size


@pytest.mark.parametrize("R,K,s", [(4, 64, 0.5), (7, 192, 0.3), (16, 640, 0.7), (3, 128, 0.0), (5, 64, 1.0)])
def test_round_trip_and_invariants(R, K, s):
    rng = np.random.default_rng(R * K)
    A = workloads.normal_f16(rng, (R, K))
    A[rng.random((R, K)) < s] = 0
    bm, off, vals = BM.encode_bitmap(A)
    assert bm.shape == (R, K // 64) and off.shape == (R * K // 64 + 1,) and off.dtype == np.uint32
    assert off[0] == 0 and np.all(off % 8 == 0) and np.all(np.diff(off.astype(np.int64)) >= 0)
    pop = np.array([bin(int(b)).count("1") for b in bm.ravel()])
    assert np.array_equal(np.diff(off.astype(np.int64)), (pop + 7) // 8 * 8)
    assert pop.sum() == np.count_nonzero(A)
    back = BM.decode_bitmap(bm, off, vals, K)
    assert np.array_equal(back.view(np.uint16), A.view(np.uint16))
    # padding slots hold +0
    for t in range(R * K // 64):
        pad = vals[off[t] + pop[t]:off[t + 1]]
        assert np.all(pad.view(np.uint16) == 0)


def test_signed_zero_and_subnormal():
    A = np.zeros((1, 64), dtype=np.float16)
    A[0, 3] = np.float16(-0.0)
    A[0, 5] = np.float16(6e-8)            # smallest subnormal: a non-zero
    A[0, 63] = np.float16(-2.5)
    bm, off, vals = BM.encode_bitmap(A)
    assert int(bm[0, 0]) == (1 << 5) | (1 << 63)
    assert list(vals[:2].view(np.uint16)) == [A[0, 5].view(np.uint16), A[0, 63].view(np.uint16)]
    back = BM.decode_bitmap(bm, off, vals, 64)
    assert back[0, 3].view(np.uint16) == 0     # -0 is not stored and decodes as +0


def test_dense_and_empty_extremes():
    A = workloads.normal_f16(np.random.default_rng(3), (2, 128)) + np.float16(10)
    bm, off, vals = BM.encode_bitmap(A)
    assert np.all(bm == np.uint64(0xFFFFFFFFFFFFFFFF))
    assert list(off) == [0, 64, 128, 192, 256]
    assert np.array_equal(vals.view(np.uint16), A.reshape(-1).view(np.uint16))
    Z = np.zeros((3, 192), dtype=np.float16)
    bm, off, vals = BM.encode_bitmap(Z)
    assert np.all(bm == 0) and np.all(off == 0) and vals.size == 0


def test_spmm_brute_force():
    rng = np.random.default_rng(9)
    A = workloads.normal_f16(rng, (5, 128))
    A[rng.random(A.shape) < 0.6] = 0
    B = workloads.normal_f16(rng, (128, 3))
    bm, off, vals = BM.encode_bitmap(A)
    Y = BM.spmm_bitmap(bm, off, vals, B)
    for i in range(5):
        for j in range(3):
            ref = sum(float(A[i, k]) * float(B[k, j]) for k in range(128))
            assert abs(Y[i, j] - ref) < 1e-12
