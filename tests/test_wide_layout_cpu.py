"""Host-side checks of the wide-tile SpMM's LDS layout (csrc/wide_layout.hpp), compiled
with the host C++ compiler: the DMA chunk placement must be a bijection onto the B tile,
and every ds_read_b64_tr_b16 of a half-wave must touch each of the 64 four-byte banks
exactly once."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "structured_sparse_matrix_amd", "csrc")

CHECKER = r"""
#include "wide_layout.hpp"
#include <cstdio>
#include <set>
using namespace snm::wide;

template <int BN, int KS>
int check() {
  int bad = 0;
  // 1) chunk o -> (x, c) -> b_offset(x, c) == o, and every (x, c) reached once
  std::set<std::pair<int, int>> seen;
  for (unsigned o = 0; o < (unsigned)(KS * BN * 2); o += 16) {
    const int x = b_row_of<BN>(o), c = b_col_of<BN>(o);
    if (x < 0 || x >= KS || c < 0 || c + 8 > BN || c % 8) { ++bad; continue; }
    if (b_offset<BN>(x, c) != o) ++bad;
    if (!seen.insert({x, c}).second) ++bad;
  }
  if ((int)seen.size() != KS * BN / 8) ++bad;
  // 2) transpose reads of one 32-column operand: half-wave = lanes 0..31 reading rows
  //    x0 + lane%16/4 at columns c0 + 16*(lane/16) + 4*(lane%4); 8 bytes = 2 banks each
  for (int x0 = 0; x0 + 4 <= KS; x0 += 4)
    for (int c0 = 0; c0 + 32 <= BN; c0 += 32) {
      int hits[64] = {0};
      for (int l = 0; l < 32; ++l) {
        const unsigned a = b_offset<BN>(x0 + (l & 15) / 4, c0 + 16 * (l / 16) + 4 * (l & 3));
        if (a % 8) ++bad;
        ++hits[(a / 4) % 64];
        ++hits[(a / 4 + 1) % 64];
      }
      for (int b = 0; b < 64; ++b)
        if (hits[b] != 1) { ++bad; break; }
    }
  // 3) rows x + 4, x + 16, x + 20 (x % 8 < 4) are constant row offsets from row x
  for (int x = 0; x + 20 < KS; ++x) {
    if (x % 8 >= 4) continue;
    for (int c = 0; c < BN; c += 4) {
      if (b_offset<BN>(x + 4, c) != b_offset<BN>(x, c) + 4u * 2u * BN) ++bad;
      if (b_offset<BN>(x + 16, c) != b_offset<BN>(x, c) + 16u * 2u * BN) ++bad;
      if (b_offset<BN>(x + 20, c) != b_offset<BN>(x, c) + 20u * 2u * BN) ++bad;
    }
  }
  std::printf("BN=%d KS=%d bad=%d\n", BN, KS, bad);
  return bad;
}

// A and metadata regions of a stage of KS positions for a BM-row tile: the DMA writes must
// cover each (row, chunk) / (row, word) exactly once at the offset the operand reads use,
// and a quarter-wave of operand reads (rows r0..r0+15 of a 32-row tile, one chunk) must
// hit each 16-byte bank group of a 256-byte line once.
template <int KS, int BM>
int check_a() {
  int bad = 0;
  const int nblk = BM * KS / 1024;
  std::set<unsigned> offs;
  for (int b = 0; b < nblk; ++b)
    for (int l = 0; l < 64; ++l) {
      const int R = a_dma_row<KS>(b, l), c = a_dma_chunk<KS>(b, l);
      if (R < 0 || R >= BM || c < 0 || c >= KS / 16) { ++bad; continue; }
      if (a_offset<KS>(R, c) != (unsigned)(b * 1024 + l * 16)) ++bad;
      offs.insert(a_offset<KS>(R, c));
    }
  if ((int)offs.size() != nblk * 64) ++bad;
  for (int t = 0; t < BM / 32; ++t)
    for (int c = 0; c < KS / 16; ++c)
      for (int q = 0; q < 2; ++q) {
        int hits[16] = {0};
        for (int i = 0; i < 16; ++i) ++hits[(a_offset<KS>(t * 32 + 16 * q + i, c) / 16) % 16];
        for (int k = 0; k < 16; ++k)
          if (hits[k] != 1) { ++bad; break; }
      }
  std::set<unsigned> moffs;
  const int nm = BM / m_rows_per_block<KS>();
  if (nm != nblk) ++bad;
  for (int b = 0; b < nm; ++b)
    for (int l = 0; l < 64; ++l) {
      const int R = m_dma_row<KS>(b, l), w = m_dma_word<KS>(l);
      if (R >= BM || w >= KS / 16) { ++bad; continue; }
      if (m_offset<KS>(R, w) != (unsigned)(b * 256 + l * 4)) ++bad;
      moffs.insert(m_offset<KS>(R, w));
    }
  if ((int)moffs.size() != nm * 64) ++bad;
  // constant distances between the operand reads of tiles 32 rows apart and of steps
  for (int R = 0; R + 32 < BM; ++R)
    for (int c = 0; c < KS / 16; ++c) {
      if (a_offset<KS>(R + 32, c) != a_offset<KS>(R, c) + a_tile_delta<KS>()) ++bad;
      if (m_offset<KS>(R + 32, c) != m_offset<KS>(R, c) + m_tile_delta<KS>()) ++bad;
      if (c + 2 < KS / 16 && m_offset<KS>(R, c + 2) != m_offset<KS>(R, c) + 8u) ++bad;
    }
  std::printf("A/meta KS=%d BM=%d bad=%d\n", KS, BM, bad);
  return bad;
}

int main() {
  int bad = check<64, 32>() + check<64, 64>() + check<64, 128>() + check<64, 256>() + check<128, 32>() + check<128, 64>() +
            check<128, 128>() + check<256, 32>() + check<256, 64>();
  bad += check_a<32, 128>() + check_a<64, 128>() + check_a<64, 64>() + check_a<32, 64>() +
         check_a<128, 128>() + check_a<128, 64>() + check_a<128, 32>() + check_a<256, 128>();
  return bad ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_wide_lds_layout():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check.cpp")
        exe = os.path.join(d, "check")
        with open(src, "w") as f:
            f.write(CHECKER)
        subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
