"""Host-side checks of the benchmark: the byte and flop counts its roofline fractions divide
by, against the counts worked out from the formats' definitions for the five workloads, and
its refusal of more than one GPU (before anything touches a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _fp16_compressed_nm(R, K):
    # 2:4: half the values kept (2 bytes each) and one 4-bit code per group of four
    return R * (K // 2) * 2 + R * (K // 4) // 2


def test_decode_bytes_match_the_format():
    # A 4096 x 4096 pruned 2:4, B 4096 x N, Y 4096 x N, fp16 (the decode-shaped workload)
    for n, expect in ((8, 19_005_440), (16, 19_136_512), (32, 19_398_656)):
        assert bench.spmm_bytes(n) == expect
        assert expect == _fp16_compressed_nm(4096, 4096) + 4096 * n * 2 * 2


def test_vnm_bytes_match_the_format():
    # V:2:M: 2 of every M columns kept per row (fp16), a 4-bit code per kept pair's group of
    # four selected columns, four column indices (one byte each) per V-block and group
    def by_definition(R, K, C, V, M):
        values = R * (K // M) * 2 * 2
        midx = R * (K // M) // 2
        colloc = (R // V) * (K // M) * 4
        return values + midx + colloc + K * C * 2 + R * C * 2
    assert bench.vnm_bytes(11008, 4096, 256, 64, 8) == by_definition(11008, 4096, 256, 64, 8) == 33_447_936
    assert bench.vnm_bytes(8192, 8192, 4096, 128, 16) == by_definition(8192, 8192, 4096, 128, 16) == 153_223_168


def test_large_tile_gather_bytes():
    # 128 x 512 tiles; per 32 positions of K' = 4K/M: 32 gathered B rows of 512 columns
    # (32 KiB), the tile's values (128 rows x 16 kept x 2 B) and index words as dwords
    tiles = (8192 // 128) * (4096 // 512)
    stages = (4 * 8192 // 16) // 32
    assert bench.big_lds_bytes(8192, 8192, 4096, 128, 16) == tiles * stages * (32 * 512 * 2 + 128 * 16 * 2 + 1024)
    # at least the gathered B rows every V-block needs: K' rows of C columns, fp16
    assert bench.big_lds_bytes(8192, 8192, 4096, 128, 16) >= (8192 // 128) * 2048 * 4096 * 2


def test_encode_bytes():
    assert bench.ENCODE_BYTES == 4096 * 4096 * 2 + _fp16_compressed_nm(4096, 4096)
    assert bench.vnm_encode_bytes(8192, 8192, 128, 16) == \
        8192 * 8192 * 2 + bench.vnm_bytes(8192, 8192, 4096, 128, 16) - 2 * (8192 * 4096 * 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 2, r.stderr[-1000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("argv", [["--help"]])
def test_help(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "--workload" in r.stdout
