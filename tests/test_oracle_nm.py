"""Pins of the 2:4 oracle against what the pages and the mathematics fix (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle.nm import _unpack_codes
import workloads


def _worked(golden):
    g = golden("worked_example_2x8.json")
    return g, np.array(g["dense"], dtype=np.float16)


def test_worked_example_values_and_indices(golden):
    g, A = _worked(golden)
    values, meta = oracle.prune_encode_nm(A)
    np.testing.assert_array_equal(values, np.array(g["values"], dtype=np.float16))
    codes = _unpack_codes(meta)
    for r in range(2):
        for grp in range(2):
            s0, s1 = codes[r, grp] & 3, codes[r, grp] >> 2
            assert [s0, s1] == g["kept_slots"][r][grp]
            assert [format(s0, "02b"), format(s1, "02b")] == g["indices"][r][2 * grp: 2 * grp + 2]


def test_worked_example_metadata_bytes(golden):
    # Slots (0,2),(1,3) -> codes 0x8, 0xd -> byte 0xd8; (1,2),(0,3) -> 0x9, 0xc -> 0xc9.
    _, A = _worked(golden)
    _, meta = oracle.prune_encode_nm(A)
    assert meta.tolist() == [[0xD8], [0xC9]]


def test_worked_example_dot_product(golden):
    g, A = _worked(golden)
    values, meta = oracle.prune_encode_nm(A)
    b = workloads.small_matrix(11, (8, 1))
    y = oracle.spmm_nm(values, meta, b)[0, 0]
    expect = sum(float(np.float16(w)) * float(b[k, 0]) for k, w in g["row0_dot_terms"])
    assert y == expect
    # 4 multiply-adds, not 8: exactly four nonzeros in the decoded row
    assert np.count_nonzero(oracle.decode_nm(values, meta, 8)[0]) == g["row0_macs"]


def test_local_slot_to_global_column(golden):
    g, A = _worked(golden)
    values, meta = oracle.prune_encode_nm(A)
    dense = oracle.decode_nm(values, meta, 8)
    lg = g["local_to_global"]
    col = 4 * lg["group"] + lg["slot"]
    assert col == lg["column"]
    assert dense[0, col] == np.float16(0.7) and dense[0, col] == values[0, 2]


def test_metadata_codes_are_the_dfss_table(golden):
    legal = set(golden("dfss_metadata_codes.json")["codes_2of4_fp16"])
    assert legal == set(oracle.NM_LEGAL_CODES)
    # every pair of slots is reachable, and produces one of those codes
    seen = set()
    for pair in itertools.combinations(range(4), 2):
        row = np.zeros((1, 8), dtype=np.float16)
        row[0, list(pair)] = [2.0, 3.0]
        _, meta = oracle.prune_encode_nm(row)
        seen.add(int(meta[0, 0] & 0xF))
    assert seen == legal
    # 1:2 on 32-bit data = two 16-bit halves kept together: only 0x4 (slots 0,1) and 0xe (2,3)
    for pair, code in (((0, 1), 0x4), ((2, 3), 0xE)):
        row = np.zeros((1, 8), dtype=np.float16)
        row[0, list(pair)] = [5.0, 5.0]
        assert int(oracle.prune_encode_nm(row)[1][0, 0] & 0xF) == code
    assert set(golden("dfss_metadata_codes.json")["codes_1of2_fp32"]) == {0x4, 0xE}


def test_word_bit_layout(golden):
    # group k of a 16-bit word sits at bits [4k, 4k+3]; the word is stored little-endian
    pairs = [(0, 1), (1, 3), (2, 3), (0, 2)]
    row = np.zeros((1, 16), dtype=np.float16)
    for g, (a, b) in enumerate(pairs):
        row[0, 4 * g + a] = 1.0
        row[0, 4 * g + b] = -2.0
    _, meta = oracle.prune_encode_nm(row)
    word = int(meta[0, 0]) | (int(meta[0, 1]) << 8)
    for g, (a, b) in enumerate(pairs):
        assert (word >> (4 * g)) & 0xF == a | (b << 2)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codes_legal_and_two_per_group(seed):
    for A in (workloads.small_matrix(seed, (32, 64)), workloads.ties_matrix(seed, (32, 64))):
        values, meta = oracle.prune_encode_nm(A)
        codes = _unpack_codes(meta)
        assert set(np.unique(codes).tolist()) <= set(oracle.NM_LEGAL_CODES)
        assert values.shape == (32, 32) and meta.shape == (32, 8)
        dense = oracle.decode_nm(values, meta, 64)
        # every kept value came from its own position, every dropped one is zeroed
        kept = dense.view(np.uint16) == A.view(np.uint16)
        assert np.all(kept | (dense == 0))


def test_legal_but_sparse_group_still_stores_two():
    # a group with fewer than two nonzeros still stores two values (one or both zero)
    A = np.zeros((2, 8), dtype=np.float16)
    A[0, 2] = 3.0
    values, meta = oracle.prune_encode_nm(A)
    assert values.shape == (2, 4)
    codes = _unpack_codes(meta)
    assert codes[0, 0] == (0 | (2 << 2))   # slot 2 (the nonzero) and slot 0 (lowest zero)
    assert codes[0, 1] == 0x4 and codes[1, 0] == 0x4  # all-zero groups keep slots 0, 1


def test_storage_arithmetic(golden):
    g = golden("worked_example_2x8.json")
    _, A = _worked(golden)
    values, meta = oracle.prune_encode_nm(A)
    n_vals = values.size
    assert values.size * 16 == g["bits"]["fp16_values"]
    assert n_vals * 2 == g["bits"]["fp16_indices"] == meta.size * 8
    assert values.size * 16 + meta.size * 8 == g["bits"]["fp16_total"]
    assert A.size * 16 == g["bits"]["fp16_dense"]
    assert values.size * 8 + meta.size * 8 == g["bits"]["int8_total"]
    assert (g["bits"]["fp16_total"] / g["bits"]["fp16_dense"]) == 1 - g["savings"]["fp16"]
    assert (g["bits"]["int8_total"] / g["bits"]["int8_dense"]) == 1 - g["savings"]["int8"]
    # one group of four: 2 values + 2 two-bit indices
    assert 2 * 16 + 2 * 2 == g["group_bits"]["fp16_compressed"]
    assert 2 * 8 + 2 * 2 == g["group_bits"]["int8_compressed"]
    # "Check yourself": 512 x 1024 -> metadata bits
    c = g["check_yourself_metadata_bits"]
    _, meta = oracle.prune_encode_nm(np.zeros((c["R"], c["C"]), dtype=np.float16))
    assert meta.size * 8 == c["bits"]


def test_magnitude_key_orders_like_abs():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    fin = np.isfinite(vals)
    k = oracle.magnitude_key(vals[fin])
    a = np.abs(vals[fin].astype(np.float64))
    order = np.argsort(a, kind="stable")
    assert np.all(np.diff(k[order]) >= 0)
    # equal keys <-> equal magnitudes (so +0 and -0 tie)
    assert np.array_equal(np.unique(k).size, np.unique(a).size)


def _brute_force_encode(A):
    """Enumerate all 6 slot pairs per group; a pair S is valid iff every kept key >= every
    dropped key; take the lexicographically smallest valid pair."""
    R, K = A.shape
    keys = (A.view(np.uint16) & 0x7FFF).astype(int)
    vals = np.zeros((R, K // 2), dtype=np.float16)
    codes = np.zeros((R, K // 4), dtype=int)
    for r in range(R):
        for g in range(K // 4):
            kk = [int(keys[r, 4 * g + i]) for i in range(4)]
            for pair in itertools.combinations(range(4), 2):
                rest = [i for i in range(4) if i not in pair]
                if min(kk[i] for i in pair) >= max(kk[i] for i in rest):
                    break
            vals[r, 2 * g] = A[r, 4 * g + pair[0]]
            vals[r, 2 * g + 1] = A[r, 4 * g + pair[1]]
            codes[r, g] = pair[0] | (pair[1] << 2)
    return vals, codes


@pytest.mark.parametrize("maker,seed", [("small_matrix", 3), ("ties_matrix", 4), ("ties_matrix", 5)])
def test_brute_force_encode(maker, seed):
    A = getattr(workloads, maker)(seed, (12, 32))
    values, meta = oracle.prune_encode_nm(A)
    bv, bc = _brute_force_encode(A)
    assert np.array_equal(values.view(np.uint16), bv.view(np.uint16))
    assert np.array_equal(_unpack_codes(meta).astype(int), bc)


def test_non_finite_ranking():
    A = np.array([[np.nan, 1.0, -np.inf, 2.0, 0.0, -0.0, 0.0, -0.0]], dtype=np.float16)
    values, meta = oracle.prune_encode_nm(A)
    c = _unpack_codes(meta)[0]
    assert c[0] == 0 | (2 << 2)        # NaN and -Inf outrank finite values
    assert c[1] == 0x4                  # +0 and -0 tie: lowest slots win
    assert values.view(np.uint16)[0, 3] == np.float16(-0.0).view(np.uint16)


def test_brute_force_spmm_triple_loop():
    A = workloads.small_matrix(6, (8, 16))
    B = workloads.small_matrix(7, (16, 5))
    values, meta = oracle.prune_encode_nm(A)
    Y = oracle.spmm_nm(values, meta, B)
    codes = _unpack_codes(meta)
    for r in range(8):
        for c in range(5):
            acc = 0.0
            for g in range(4):
                s0, s1 = int(codes[r, g] & 3), int(codes[r, g] >> 2)
                acc += float(values[r, 2 * g]) * float(B[4 * g + s0, c])
                acc += float(values[r, 2 * g + 1]) * float(B[4 * g + s1, c])
            assert abs(Y[r, c] - acc) <= 1e-12 * (1 + abs(acc))


def test_identity_b_returns_decode():
    A = workloads.small_matrix(8, (16, 32))
    values, meta = oracle.prune_encode_nm(A)
    Y = oracle.spmm_nm(values, meta, np.eye(32, dtype=np.float16))
    dense = oracle.decode_nm(values, meta, 32)
    assert np.array_equal(Y, dense.astype(np.float64))   # every output is a single exact product
    # the decoded matrix keeps exactly the two largest |a| of each group
    A64 = np.abs(A.astype(np.float64)).reshape(16, 8, 4)
    kept = np.abs(dense.astype(np.float64)).reshape(16, 8, 4)
    assert np.allclose(np.sort(A64, -1)[..., 2:], np.sort(kept, -1)[..., 2:])


def test_config_tiny_shapes_and_tie_counts():
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["nm_tiny"])
    values, meta = oracle.prune_encode_nm(A)
    assert values.shape == (256, 128) and meta.shape == (256, 32)
    assert B.shape == (256, 64)
