"""The host model of the row-group interleaved V:2:M storage (tests/_vnm_tiled.py) against
its definition, element by element with explicit loops, and as a round trip."""
import numpy as np

from _vnm_tiled import tile, untile


def test_tile_places_every_chunk_and_word_where_the_header_says():
    R, K, M = 64, 256, 8
    W = K // (4 * M)
    rng = np.random.default_rng(5)
    values = rng.integers(0, 1 << 16, size=(R, 2 * K // M), dtype=np.uint16).view(np.float16)
    midx = rng.integers(0, 256, size=(R, K // (2 * M)), dtype=np.uint8)
    vt, mt = tile(values, midx, M)
    flat_v = vt.reshape(-1).view(np.uint16)
    flat_w = mt.reshape(-1).view(np.uint16)
    words = midx.view(np.uint16)
    for r in range(R):
        for c in range(W):
            base = ((r // 32) * W + c) * 256 + (r % 32) * 8
            assert np.array_equal(flat_v[base:base + 8], values[r, 8 * c:8 * c + 8].view(np.uint16))
            assert flat_w[((r // 32) * W + c) * 32 + (r % 32)] == words[r, c]


def test_untile_inverts_tile():
    R, K, M = 96, 640, 10
    rng = np.random.default_rng(6)
    values = rng.standard_normal((R, 2 * K // M)).astype(np.float16)
    midx = rng.integers(0, 256, size=(R, K // (2 * M)), dtype=np.uint8)
    v2, m2 = untile(*tile(values, midx, M), M)
    assert np.array_equal(v2.view(np.uint16), values.view(np.uint16))
    assert np.array_equal(m2, midx)
