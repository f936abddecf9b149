// LDS layout of the wide-tile SpMM (spmm_wide.hip): pure index arithmetic, constexpr so
// that the same functions run in the kernels and in host-side checks.
//
// One ring stage holds, for KS = 32 * KSTEPS consecutive positions of the compressed
// reduction space:
//   B tile      KS rows x BN fp16 columns, row pitch 2*BN bytes. The row's 32-byte cells
//               (16 columns each) are XOR-permuted by a function of the row so that a
//               ds_read_b64_tr_b16 -- which touches rows x0..x0+3 of one 16-column cell in
//               each 16-lane group, and cells 2j, 2j+1 in the two groups of a half-wave --
//               hits every bank at most once per half-wave.
//   A blocks    (BM/32) * KSTEPS blocks of 1 KiB: the 32x32x32 sparse-MFMA A operand of one
//               32-row tile and one 32-position step, lane-major (lane l's 16 bytes at
//               16*l), exactly as one 16-byte-per-lane DMA instruction writes them.
//   metadata    the same number of 256-byte blocks: lane l's 16-bit index word at 4*l (the
//               2-byte DMA form writes one zero-extended dword per lane).
#pragma once

#include <stdint.h>

namespace snm {
namespace wide {

// XOR applied to the cell index of row x of a BN-column B tile.
template <int BN>
constexpr int cell_xor(int x) {
  return BN >= 256 ? (((x & 3) << 1) | (((x >> 3) & 1) << 3))
       : BN == 128 ? ((x & 3) << 1)
       : BN == 64  ? (((x >> 1) & 1) << 1)
                   : 0;
}

// Byte offset of (row x, column c) in the B tile; c is a multiple of 4 (a transpose-read
// lane address) or of 8 (a 16-byte DMA chunk).
template <int BN>
constexpr uint32_t b_offset(int x, int c) {
  return (uint32_t)x * (2u * BN) + (uint32_t)(((c >> 4) ^ cell_xor<BN>(x)) << 5) + (uint32_t)(c & 15) * 2u;
}

// Inverse of b_offset for a 16-byte chunk: which tile row and first column the chunk at
// byte offset o (a multiple of 16) of the B tile holds.
template <int BN>
constexpr int b_row_of(uint32_t o) { return (int)(o / (2u * BN)); }
template <int BN>
constexpr int b_col_of(uint32_t o) {
  const int x = b_row_of<BN>(o);
  const int p = (int)(o % (2u * BN));
  return (((p >> 5) ^ cell_xor<BN>(x)) << 4) + ((p >> 4) & 1) * 8;
}

}  // namespace wide
}  // namespace snm
