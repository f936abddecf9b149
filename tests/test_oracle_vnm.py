"""Pins of the V:N:M oracle (CPU only): special cases, closed forms, brute force."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.nm import _unpack_codes
import workloads


def test_m4_reduces_to_2_4():
    # with M = 4 every block keeps columns 0..3, so V:2:4 is plain 2:4
    for A in (workloads.small_matrix(1, (64, 64)), workloads.ties_matrix(2, (64, 64))):
        v4, mi, cl = oracle.prune_encode_vnm(A, V=32, M=4)
        v, m = oracle.prune_encode_nm(A)
        assert np.array_equal(v4.view(np.uint16), v.view(np.uint16))
        assert np.array_equal(mi, m)
        assert np.all(cl == np.arange(4, dtype=np.uint8))


@pytest.mark.parametrize("M", [8, 16])
def test_v1_is_top2_of_m_by_magnitude(M):
    # V = 1: the column score is a^2, so the two stages keep the two largest |a| of M
    A = workloads.small_matrix(3, (8, 4 * M))
    values, midx, colloc = oracle.prune_encode_vnm(A, V=1, M=M)
    dense = oracle.decode_vnm(values, midx, colloc, 1, M, A.shape[1])
    for r in range(A.shape[0]):
        for g in range(A.shape[1] // M):
            seg = [abs(float(x)) for x in A[r, g * M:(g + 1) * M]]
            order = sorted(range(M), key=lambda i: (-seg[i], i))[:2]
            expect = np.zeros(M, dtype=np.float16)
            expect[order] = A[r, g * M + np.array(order)]
            assert np.array_equal(dense[r, g * M:(g + 1) * M], expect)


def _brute_force_vnm(A, V, M):
    """Enumerate every 4-column subset of each block with exact (rational) sums of squares;
    valid iff every kept score >= every dropped score; take the lexicographically smallest.
    Then the 2:4 step over the four kept columns, enumerating the 6 pairs the same way."""
    R, K = A.shape
    G = K // M
    colloc = np.zeros((R // V, G, 4), dtype=np.uint8)
    dense = np.zeros_like(A)
    for b in range(R // V):
        for g in range(G):
            score = [sum(Fraction(float(A[b * V + r, g * M + c])) ** 2 for r in range(V)) for c in range(M)]
            for cols in itertools.combinations(range(M), 4):
                rest = [c for c in range(M) if c not in cols]
                if not rest or min(score[c] for c in cols) >= max(score[c] for c in rest):
                    break
            colloc[b, g] = cols
            for r in range(V):
                mags = [abs(Fraction(float(A[b * V + r, g * M + c]))) for c in cols]
                for pair in itertools.combinations(range(4), 2):
                    rest = [i for i in range(4) if i not in pair]
                    if min(mags[i] for i in pair) >= max(mags[i] for i in rest):
                        break
                for p in pair:
                    dense[b * V + r, g * M + cols[p]] = A[b * V + r, g * M + cols[p]]
    return colloc, dense


@pytest.mark.parametrize("V,M,seed", [(4, 8, 0), (2, 16, 1), (8, 6, 2), (4, 8, 3)])
def test_brute_force_two_stage(V, M, seed):
    K = 4 * M
    A = workloads.small_matrix(seed, (2 * V, K)) if seed != 3 else workloads.ties_matrix(seed, (2 * V, K), levels=3)
    values, midx, colloc = oracle.prune_encode_vnm(A, V, M)
    bc, bd = _brute_force_vnm(A, V, M)
    assert np.array_equal(colloc, bc)
    dense = oracle.decode_vnm(values, midx, colloc, V, M, K)
    assert np.array_equal(dense.view(np.uint16), bd.view(np.uint16)) or np.array_equal(dense, bd)


def test_shapes_and_overhead(golden):
    g = golden("venom_format.json")
    R, K, V, M = 256, 512, 128, 16
    A = workloads.small_matrix(4, (R, K), 0.02)
    values, midx, colloc = oracle.prune_encode_vnm(A, V, M)
    assert values.shape == (R, K // M * 2)
    assert midx.size * 8 == values.size * g["m_indices_bits_per_value"]
    assert colloc.shape == (R // V, K // M, 4)
    # metadata overhead per stored fp16 value at V = 128: (2 + 4*8/(2V)) / 16 = 0.1328125
    overhead = (midx.size * 8 + colloc.size * 8) / (values.size * 16)
    assert overhead == pytest.approx(g["overhead_at_V128"], abs=5e-5)
    assert overhead == (2 + 4 * g["column_loc_bits_per_entry_max"] / (2 * V)) / 16


@pytest.mark.parametrize("V,M", [(64, 8), (128, 16), (32, 10), (32, 256)])
def test_invariants(V, M):
    K = 4 * M
    A = workloads.small_matrix(5, (2 * V, K), 0.02)
    values, midx, colloc = oracle.prune_encode_vnm(A, V, M)
    assert np.all(np.diff(colloc.astype(int), axis=-1) > 0) and np.all(colloc < M)
    codes = _unpack_codes(midx)
    assert set(np.unique(codes).tolist()) <= set(oracle.NM_LEGAL_CODES)
    dense = oracle.decode_vnm(values, midx, colloc, V, M, K)
    nz = (dense.reshape(2 * V, K // M, M) != 0).sum(-1)
    assert np.all(nz == 2)        # Gaussian data: no zeros, so exactly 2 nonzeros per row and group
    # every row of a block only uses that block's four selected columns
    used = dense.reshape(2, V, K // M, M) != 0
    sel = np.zeros((2, K // M, M), dtype=bool)
    for b in range(2):
        for gg in range(K // M):
            sel[b, gg, colloc[b, gg]] = True
    assert np.all(~used | sel[:, None])


def test_selected_columns_have_largest_block_norm():
    V, M = 16, 8
    A = workloads.small_matrix(6, (V, 4 * M))
    _, _, colloc = oracle.prune_encode_vnm(A, V, M)
    norms = np.linalg.norm(A.astype(np.float64).reshape(V, 4, M), axis=0)   # (groups, M)
    for g in range(4):
        kept = set(colloc[0, g].tolist())
        assert min(norms[g, list(kept)]) >= max(norms[g, [c for c in range(M) if c not in kept]])


def test_identity_b_and_brute_product():
    V, M = 8, 8
    A = workloads.small_matrix(7, (16, 32))
    values, midx, colloc = oracle.prune_encode_vnm(A, V, M)
    dense = oracle.decode_vnm(values, midx, colloc, V, M, 32)
    assert np.array_equal(oracle.spmm_vnm(values, midx, colloc, V, M, np.eye(32, dtype=np.float16)),
                          dense.astype(np.float64))
    B = workloads.small_matrix(8, (32, 3))
    Y = oracle.spmm_vnm(values, midx, colloc, V, M, B)
    codes = _unpack_codes(midx)
    for r in range(16):
        for c in range(3):
            acc = 0.0
            for g in range(4):
                for j, p in enumerate((codes[r, g] & 3, codes[r, g] >> 2)):
                    col = g * M + int(colloc[r // V, g, p])
                    acc += float(values[r, 2 * g + j]) * float(B[col, c])
            assert abs(Y[r, c] - acc) <= 1e-12 * (1 + abs(acc))


def test_rejects_bad_shapes():
    A = np.zeros((10, 32), dtype=np.float16)
    with pytest.raises(ValueError):
        oracle.prune_encode_vnm(A, V=4, M=8)
    with pytest.raises(ValueError):
        oracle.prune_encode_vnm(np.zeros((8, 24), dtype=np.float16), V=4, M=8)   # K/M odd
