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
//   A values    a stage holds KS bytes of every row (KS/2 values); one 16-byte-per-lane DMA
//               instruction fills a 1 KiB block of RPD = 1024/KS consecutive rows, row-major,
//               whose 16-byte chunks are XOR-permuted by a function of the row so that the
//               sparse-MFMA operand read (16 bytes of rows r..r+15 at one logical chunk per
//               quarter-wave) touches every bank once. With KS = 64 one instruction reads 16
//               rows x 64 bytes of the canonical array instead of 32 rows x 32 bytes.
//   metadata    WPR = KS/16 index words per row; one 2-byte-per-lane DMA instruction (which
//               writes one zero-extended dword per lane) fills a 256-byte block of RPM =
//               64/WPR rows, lane = row * WPR + word.
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

// ---- A values: stage of KS positions (KS bytes per row), blocks of RPD rows ----------------
template <int KS>
constexpr int a_rows_per_block() { return 1024 / KS; }
// XOR applied to the 16-byte chunk index of tile row R (16 consecutive rows get distinct
// 16-byte slots of a 256-byte bank line)
template <int KS>
constexpr int a_chunk_xor(int R) { return (R / (256 / KS)) % (KS / 16); }
// byte offset inside the stage's A region of (row R of the tile, logical 16-byte chunk c)
template <int KS>
constexpr uint32_t a_offset(int R, int c) {
  return (uint32_t)(R / a_rows_per_block<KS>()) * 1024u +
         (uint32_t)(R % a_rows_per_block<KS>()) * (uint32_t)KS +
         (uint32_t)((c ^ a_chunk_xor<KS>(R)) * 16);
}
// DMA lane l of block b: tile row and logical chunk it fetches
template <int KS>
constexpr int a_dma_row(int b, int l) { return b * a_rows_per_block<KS>() + l / (KS / 16); }
template <int KS>
constexpr int a_dma_chunk(int b, int l) {
  return (l % (KS / 16)) ^ a_chunk_xor<KS>(a_dma_row<KS>(b, l));
}

// ---- metadata: WPR words per row per stage, blocks of RPM rows ------------------------------
template <int KS>
constexpr int m_words_per_row() { return KS / 16; }
template <int KS>
constexpr int m_rows_per_block() { return 64 / m_words_per_row<KS>(); }
template <int KS>
constexpr uint32_t m_offset(int R, int w) {
  return (uint32_t)(R / m_rows_per_block<KS>()) * 256u +
         (uint32_t)((R % m_rows_per_block<KS>()) * m_words_per_row<KS>() + w) * 4u;
}
template <int KS>
constexpr int m_dma_row(int b, int l) { return b * m_rows_per_block<KS>() + l / m_words_per_row<KS>(); }
template <int KS>
constexpr int m_dma_word(int l) { return l % m_words_per_row<KS>(); }

// Constant distances used by the kernels' operand reads: row R + 32 of A lies 32 KS bytes
// after row R (same chunk), its metadata 8 KS bytes after; the index word w + 2 of a row
// lies 8 bytes after word w; in the B tile, rows x + 4, x + 16 and x + 20 of a row x with
// x % 8 < 4 share x's cell swizzle, so they lie 4, 16 and 20 rows (times 2 BN bytes) after.
template <int KS>
constexpr uint32_t a_tile_delta() { return 32u * KS; }
template <int KS>
constexpr uint32_t m_tile_delta() { return 8u * KS; }

}  // namespace wide
}  // namespace snm
