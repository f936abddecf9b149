"""Pins of the DFSS data-type variants of the oracle (bf16 2:4, fp32 1:2), CPU only.

Each pin checks the oracle against something other than its own formula: torch's
float32 -> bfloat16 conversion (round to nearest even), hand-worked bf16 grid points,
brute force with Python floats, the fp16 2:4 oracle (pinned by the worked example) on
values exact in both formats, the 2:4 decoder over the same bytes seen as 16-bit halves,
and textbook masked softmax attention.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import variants as ov
from oracle.nm import _unpack_codes


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- bf16 conversions

def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # float32 subnormals
        rng.uniform(-3.4e38, 3.4e38, 2000).astype(np.float32),      # near the top, some overflow
        np.array([0.0, -0.0, 3.3895314e38, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45], np.float32),
        # exact ties between two bf16 neighbours
        (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 64, 2, dtype=np.float32)).astype(np.float32),
    ])
    np.testing.assert_array_equal(ov.f64_to_bf16(x.astype(np.float64)), _torch_bf16_bits(x))


def test_bf16_rounding_worked_points():
    # neighbours of 1.0 are 1 and 1 + 2**-7; 1 + 2**-8 is the midpoint -> even (1.0)
    assert ov.f64_to_bf16(1 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2**-8 lies between 1 + 2**-7 (odd last bit) and 1 + 2**-6 -> even (1 + 2**-6)
    assert ov.f64_to_bf16(1 + 3 * 2.0 ** -8) == 0x3F82
    # just above the midpoint rounds up; rounding through float32 first would give 1.0
    assert ov.f64_to_bf16(1 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert ov.f64_to_bf16(-2.0) == 0xC000
    assert ov.f64_to_bf16(-0.0) == 0x8000 and ov.f64_to_bf16(0.0) == 0
    assert ov.f64_to_bf16(2.0 ** -133) == 0x0001                      # smallest subnormal
    assert ov.f64_to_bf16(2.0 ** -134) == 0x0000                      # tie with 0 -> even
    assert ov.f64_to_bf16(3 * 2.0 ** -134) == 0x0002                  # tie 1|2 -> even
    assert ov.f64_to_bf16(ov.BF16_MAX) == 0x7F7F
    assert ov.f64_to_bf16(2.0 ** 128) == 0x7F80
    assert ov.f64_to_bf16(-np.inf) == 0xFF80


def test_bf16_round_trip_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    x = ov.bf16_to_f64(finite)
    np.testing.assert_array_equal(ov.f64_to_bf16(x), finite)
    assert ov.bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert ov.bf16_to_f64(np.uint16(0x7F7F)) == ov.BF16_MAX
    assert ov.bf16_to_f64(np.uint16(0x0001)) == 2.0 ** -133


# ---------------------------------------------------------------- bf16 2:4

def _brute_2of4(vals):
    """Lexicographically smallest pair of slots whose magnitudes all reach those dropped."""
    for s in itertools.combinations(range(4), 2):
        kept = [abs(vals[i]) for i in s]
        dropped = [abs(vals[i]) for i in range(4) if i not in s]
        if min(kept) >= max(dropped):
            return s
    raise AssertionError("no valid pair")


def test_bf16_prune_brute_force():
    rng = np.random.default_rng(1)
    # few distinct magnitudes so that ties (and +-0) are common
    x = rng.choice([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 1.5, 3.0, -3.0], size=(64, 32))
    bits = ov.f64_to_bf16(x)
    values, meta = ov.prune_encode_nm_bf16(bits)
    codes = _unpack_codes(meta)
    xs = ov.bf16_to_f64(bits)
    for r in range(x.shape[0]):
        for g in range(8):
            s0, s1 = _brute_2of4(list(xs[r, 4 * g: 4 * g + 4]))
            assert (codes[r, g] & 3, codes[r, g] >> 2) == (s0, s1)
            assert values[r, 2 * g] == bits[r, 4 * g + s0] and values[r, 2 * g + 1] == bits[r, 4 * g + s1]


def test_bf16_prune_equals_fp16_prune_on_common_values():
    # values exact in both formats (small multiples of 1/4): the selections must agree
    # with the fp16 2:4 oracle, which the worked example pins
    rng = np.random.default_rng(2)
    x = rng.integers(-40, 41, size=(32, 64)) / 4.0
    v16, m16 = oracle.prune_encode_nm(x.astype(np.float16))
    vb, mb = ov.prune_encode_nm_bf16(ov.f64_to_bf16(x))
    np.testing.assert_array_equal(mb, m16)
    np.testing.assert_array_equal(ov.bf16_to_f64(vb), v16.astype(np.float64))


def test_bf16_decode_and_spmm():
    rng = np.random.default_rng(3)
    bits = ov.f64_to_bf16(rng.standard_normal((8, 16)))
    values, meta = ov.prune_encode_nm_bf16(bits)
    dense = ov.decode_nm_bf16(values, meta, 16)
    assert (np.count_nonzero(dense.reshape(8, 4, 4), axis=2) <= 2).all()
    kept = dense != 0
    np.testing.assert_array_equal(dense[kept], ov.bf16_to_f64(bits)[kept])
    B = ov.f64_to_bf16(rng.standard_normal((16, 5)))
    Bf = ov.bf16_to_f64(B)
    Y = ov.spmm_nm_bf16(values, meta, B)
    for r in range(8):
        for c in range(5):
            assert Y[r, c] == pytest.approx(sum(dense[r, k] * Bf[k, c] for k in range(16)), rel=1e-14, abs=1e-300)
    # identity B: the product returns the decoded operand exactly
    I = ov.f64_to_bf16(np.eye(16))
    np.testing.assert_array_equal(ov.spmm_nm_bf16(values, meta, I), dense)


def test_bf16_scores_exact_integers():
    # small integers: every dot product is exact, so S is one bf16 rounding of an integer
    rng = np.random.default_rng(4)
    Q = rng.integers(-8, 9, size=(2, 8, 64)).astype(np.float64)
    K = rng.integers(-8, 9, size=(2, 32, 64)).astype(np.float64)
    S = ov.scores_bf16(ov.f64_to_bf16(Q), ov.f64_to_bf16(K), 0.125)
    exact = np.einsum("bqd,bkd->bqk", Q, K) * 0.125
    np.testing.assert_array_equal(S, _torch_bf16_bits(exact.astype(np.float32)))


def test_bf16_sddmm_identity_keys():
    # Lk == d and K = I: S = Q * scale exactly (scale a power of two)
    rng = np.random.default_rng(5)
    Qb = ov.f64_to_bf16(rng.standard_normal((1, 16, 32)))
    Kb = ov.f64_to_bf16(np.eye(32)[None])
    values, meta, S = ov.sddmm_prune_nm_bf16(Qb, Kb, 0.125)
    np.testing.assert_array_equal(S[0], ov.f64_to_bf16(ov.bf16_to_f64(Qb[0]) * 0.125))
    v2, m2 = ov.prune_encode_nm_bf16(S[0])
    np.testing.assert_array_equal(values[0], v2)
    np.testing.assert_array_equal(meta[0], m2)


def test_bf16_attention_equals_fp16_attention_on_common_values():
    rng = np.random.default_rng(6)
    S = rng.integers(-16, 17, size=(2, 8, 32)) / 8.0        # exact in fp16 and bf16
    V = rng.integers(-8, 9, size=(2, 32, 4)) / 4.0
    meta = np.stack([oracle.prune_encode_nm(S[i].astype(np.float16))[1] for i in range(2)])
    P16, O16 = oracle.attention.attention_from_pattern(S.astype(np.float16), meta, V.astype(np.float16))
    Pb, Ob = ov.attention_bf16_from_pattern(ov.f64_to_bf16(S), meta, ov.f64_to_bf16(V))
    np.testing.assert_allclose(Pb, P16, rtol=1e-15, atol=0)
    np.testing.assert_allclose(Ob, O16, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- fp32 1:2

def test_1of2_codes_are_the_dfss_table(golden):
    codes = golden("dfss_metadata_codes.json")["codes_1of2_fp32"]
    assert sorted(codes) == sorted([ov.CODE_FIRST, ov.CODE_SECOND])
    # as 2:4 codes over the 16-bit halves: (0, 1) and (2, 3)
    assert ov.CODE_FIRST == 0 | (1 << 2) and ov.CODE_SECOND == 2 | (3 << 2)
    rng = np.random.default_rng(7)
    _, meta = ov.prune_encode_1of2(rng.standard_normal((16, 64)).astype(np.float32))
    assert set(np.unique(_unpack_codes(meta)).tolist()) <= {0x4, 0xE}


def test_1of2_brute_force_with_ties_and_signed_zero():
    rng = np.random.default_rng(8)
    x = rng.choice([0.0, -0.0, 0.25, -0.25, 1.0, -1.0, 7.5], size=(32, 16)).astype(np.float32)
    values, meta = ov.prune_encode_1of2(x)
    codes = _unpack_codes(meta)
    for r in range(32):
        for p in range(8):
            a, b = float(x[r, 2 * p]), float(x[r, 2 * p + 1])
            first = abs(a) >= abs(b)
            assert codes[r, p] == (0x4 if first else 0xE)
            want = x[r, 2 * p] if first else x[r, 2 * p + 1]
            assert values[r, p].view(np.uint32) == want.view(np.uint32)   # bit copy (keeps -0)


def test_1of2_is_2of4_over_16bit_halves():
    # the format read by the 2:4 decoder over the same bytes seen as fp16 halves gives
    # the same dense matrix, bit for bit
    rng = np.random.default_rng(9)
    x = rng.standard_normal((12, 40)).astype(np.float32)
    values, meta = ov.prune_encode_1of2(x)
    halves = oracle.decode_nm(values.view(np.float16), meta, 80)          # 12 x 80 halves
    as32 = np.ascontiguousarray(halves).view(np.float32)                  # 12 x 40
    np.testing.assert_array_equal(as32.astype(np.float64), ov.decode_1of2(values, meta, 40))


def test_1of2_spmm_brute_force_and_identity():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((6, 12)).astype(np.float32)
    values, meta = ov.prune_encode_1of2(x)
    B = rng.standard_normal((12, 3)).astype(np.float32)
    Y = ov.spmm_1of2(values, meta, B)
    for r in range(6):
        for c in range(3):
            terms = [float(x[r, 2 * p + (abs(x[r, 2 * p + 1]) > abs(x[r, 2 * p]))]) *
                     float(B[2 * p + (abs(x[r, 2 * p + 1]) > abs(x[r, 2 * p])), c]) for p in range(6)]
            assert Y[r, c] == pytest.approx(sum(terms), rel=1e-14)
    np.testing.assert_array_equal(ov.spmm_1of2(values, meta, np.eye(12, dtype=np.float32)),
                                  ov.decode_1of2(values, meta, 12))


def test_1of2_scores_exact_integers_and_identity():
    rng = np.random.default_rng(11)
    Q = rng.integers(-8, 9, size=(2, 8, 64)).astype(np.float32)
    K = rng.integers(-8, 9, size=(2, 16, 64)).astype(np.float32)
    S = ov.scores_f32(Q, K, 0.125)
    exact = np.einsum("bqd,bkd->bqk", Q.astype(np.float64), K.astype(np.float64)) * 0.125
    np.testing.assert_array_equal(S, exact.astype(np.float32))
    Qr = rng.standard_normal((1, 8, 16)).astype(np.float32)
    v, m, S2 = ov.sddmm_prune_1of2(Qr, np.eye(16, dtype=np.float32)[None], 0.125)
    np.testing.assert_array_equal(S2[0], Qr[0] * np.float32(0.125))
    v2, m2 = ov.prune_encode_1of2(S2[0])
    np.testing.assert_array_equal(v[0], v2)
    np.testing.assert_array_equal(m[0], m2)


def test_1of2_attention_is_masked_textbook_attention():
    rng = np.random.default_rng(12)
    S = rng.standard_normal((2, 8, 24)).astype(np.float32)
    V = rng.standard_normal((2, 24, 5)).astype(np.float32)
    meta = np.stack([ov.prune_encode_1of2(S[i])[1] for i in range(2)])
    P, O = ov.attention_1of2_from_pattern(S, meta, V)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=1e-14)
    for i in range(2):
        mask = ov.decode_1of2(ov.prune_encode_1of2(S[i])[0], meta[i], 24) != 0
        ref = oracle.full_attention(S[i], V[i], mask=mask)
        np.testing.assert_allclose(O[i], ref, rtol=1e-12, atol=1e-14)
