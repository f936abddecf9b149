// Pruning + compression kernels: 2:4 ("2:4 sparsity on sparse tensor cores", lecture
// notes: "The definition", "The compressed format") and V:2:M ("VENOM: A vectorized N:M
// format ...", SC'23, Sec. 3, Fig. 2 and Fig. 3). Both are HBM-streaming kernels: the
// selection is local to a group and every output address is known in advance. The 2:4
// encoders read and write with non-temporal (streaming) accesses: each byte is touched once
// and the stores are whole 16-byte chunks (measured 8 % faster on the 4096 x 4096 encode,
// the products after it unchanged). The V:2:M encoders store 4-byte pieces, for which
// streaming stores measured slower, and keep ordinary stores.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace snm {

// Slots kept by 2:4 selection of four fp16 bit patterns: the two largest magnitudes
// (bits & 0x7FFF), equal magnitudes resolved toward the lower slot. Returns the 4-bit
// group code s0 | s1 << 2 (s0 < s1) and the two kept bit patterns.
__device__ __forceinline__ uint32_t select_2of4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                uint32_t& v0, uint32_t& v1) {
  // Distinct composite keys: magnitude, then reversed slot (lower slot ranks higher).
  const uint32_t c0 = ((a0 & 0x7FFFu) << 2) | 3u;
  const uint32_t c1 = ((a1 & 0x7FFFu) << 2) | 2u;
  const uint32_t c2 = ((a2 & 0x7FFFu) << 2) | 1u;
  const uint32_t c3 = ((a3 & 0x7FFFu) << 2) | 0u;
  const uint32_t g01 = c0 > c1, g02 = c0 > c2, g03 = c0 > c3;
  const uint32_t g12 = c1 > c2, g13 = c1 > c3, g23 = c2 > c3;
  // rank = number of larger keys; keep rank < 2
  const uint32_t r0 = (1u - g01) + (1u - g02) + (1u - g03);
  const uint32_t r1 = g01 + (1u - g12) + (1u - g13);
  const uint32_t r2 = g02 + g12 + (1u - g23);
  const uint32_t r3 = g03 + g13 + g23;
  const uint32_t keep = (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) |
                        ((uint32_t)(r3 < 2) << 3);
  const uint32_t s0 = __builtin_ctz(keep);
  const uint32_t s1 = 31u - __builtin_clz(keep);
  v0 = s0 == 0 ? a0 : (s0 == 1 ? a1 : a2);   // s0 <= 2
  v1 = s1 == 3 ? a3 : (s1 == 2 ? a2 : a1);   // s1 >= 1
  return s0 | (s1 << 2);
}

// One thread per 16 consecutive elements of a row (four groups = one metadata word):
// two 16-byte loads, one 16-byte value store and one 2-byte metadata store; a wave
// covers 1 KiB of contiguous input.
__global__ void __launch_bounds__(256)
k_prune_encode_nm(const uint16_t* __restrict__ A, int64_t R, int64_t K, int64_t lda,
                  uint16_t* __restrict__ values, uint16_t* __restrict__ meta) {
  const int64_t words_per_row = K >> 4;
  const int64_t total = R * words_per_row;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = w / words_per_row;
    const int64_t c = w - r * words_per_row;
    const u4* src = reinterpret_cast<const u4*>(A + r * lda + (c << 4));
    const u4 x0 = __builtin_nontemporal_load(src);
    const u4 x1 = __builtin_nontemporal_load(src + 1);
    uint32_t e[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    uint32_t out[4];
    uint32_t word = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t lo = e[2 * g], hi = e[2 * g + 1];
      uint32_t v0, v1;
      const uint32_t code = select_2of4(lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16, v0, v1);
      out[g] = v0 | (v1 << 16);
      word |= code << (4 * g);
    }
    u4 o = {out[0], out[1], out[2], out[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<u4*>(values + r * (K >> 1) + (c << 3)));
    __builtin_nontemporal_store((uint16_t)word, meta + r * words_per_row + c);
  }
}

// 2:4 prune into the operand-major layout: block (rt, kc) holds the sparse-MFMA A operand
// of rows 16rt..16rt+15 and positions 64kc..64kc+63 -- lane l = 16q + i carries row
// 16rt + i, positions 64kc + 16q + [0, 16): 8 values (16 bytes) and one metadata word.
// One thread per lane of a block: a wave reads 16 rows x 128 contiguous bytes and writes
// one contiguous 1 KiB value block and one 128-byte metadata block. Rows past R and
// positions past K are zero-filled (values 0, metadata word 0).
__global__ void __launch_bounds__(256)
k_prune_encode_nm_tiled(const uint16_t* __restrict__ A, int64_t R, int64_t K, int64_t lda,
                        uint16_t* __restrict__ values_t, uint16_t* __restrict__ meta_t) {
  const int64_t KC = (K + 63) >> 6;
  const int64_t total = ((R + 15) >> 4) * KC * 64;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(g & 63);
    const int64_t blk = g >> 6;
    const int64_t rt = blk / KC;
    const int64_t kc = blk - rt * KC;
    const int64_t row = rt * 16 + (lane & 15);
    const int64_t pos = kc * 64 + 16 * (lane >> 4);
    u4 o = {0u, 0u, 0u, 0u};
    uint32_t word = 0;
    if (row < R && pos < K) {
      const u4* src = reinterpret_cast<const u4*>(A + row * lda + pos);
      const u4 x0 = __builtin_nontemporal_load(src);
      const u4 x1 = __builtin_nontemporal_load(src + 1);
      const uint32_t e[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const uint32_t lo = e[2 * gi], hi = e[2 * gi + 1];
        uint32_t v0, v1;
        const uint32_t code = select_2of4(lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16, v0, v1);
        o[gi] = v0 | (v1 << 16);
        word |= code << (4 * gi);
      }
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u4*>(values_t + g * 8));
    __builtin_nontemporal_store((uint16_t)word, meta_t + g);
  }
}

// V:2:M. One workgroup per (block of V rows, chunk of GC groups of M columns).
//   Phase 1: one thread per column sums the squares of the block's V entries in float64,
//            rows in ascending order (a fp16 square is exact in float64, so the sum is the
//            same sequential float64 sum on any implementation).
//   Phase 2: per group, the four columns of largest score (ties to the lower column),
//            ascending -> column-loc.
//   Phase 3: one thread per (row, four groups): 2:4 among the four selected values,
//            16-byte value store + one 16-bit m-index word.
constexpr int kVnmThreads = 256;
constexpr int kVnmMaxCols = 1024;

// Where the V:2:M encoders put a row's value pair of group g (element index) and the index
// word of groups 4w .. 4w + 3 (word index). Canonical: row-major arrays. Row-group
// interleaved ("tiled", R % 32 == 0): per group of 32 rows, 16-byte chunk c (the 8 values
// of groups 4c .. 4c + 3) of the 32 rows is stored together, row after row, and likewise
// their 2-byte index words, so that a copy of any run of chunks of 32 consecutive rows
// reads whole cache lines.
__device__ __forceinline__ int64_t vnm_value_at(int64_t row, int64_t g, int64_t G, int tiled) {
  return tiled ? (((row >> 5) * (G >> 2) + (g >> 2)) << 8) + ((row & 31) << 3) + ((g & 3) << 1)
               : row * 2 * G + 2 * g;
}
__device__ __forceinline__ int64_t vnm_word_at(int64_t row, int64_t w, int64_t G, int tiled) {
  return tiled ? (((row >> 5) * (G >> 2) + w) << 5) + (row & 31) : row * (G >> 2) + w;
}

__global__ void __launch_bounds__(kVnmThreads)
k_prune_encode_vnm(const uint16_t* __restrict__ A, int64_t R, int64_t K, int64_t lda, int V, int M,
                   int GC, uint16_t* __restrict__ values, uint16_t* __restrict__ midx,
                   uint8_t* __restrict__ colloc, int tiled) {
  __shared__ double score[kVnmMaxCols];
  __shared__ uint8_t keep[kVnmMaxCols];
  __shared__ uint8_t sel[kVnmMaxCols / 4 * 4];   // [group in chunk][4]
  const int64_t G = K / M;
  const int64_t nchunks = (G + GC - 1) / GC;
  const int64_t vb = blockIdx.x / nchunks;
  const int64_t g0 = (blockIdx.x - vb * nchunks) * GC;
  const int ng = (int)((G - g0) < GC ? (G - g0) : GC);   // groups in this chunk (multiple of 4)
  const int ncols = ng * M;
  const uint16_t* Ablk = A + vb * V * lda + g0 * M;

  for (int c = threadIdx.x; c < ncols; c += kVnmThreads) {
    double s = 0.0;
    int r = 0;
    for (; r + 8 <= V; r += 8) {     // eight independent loads in flight, sums in row order
      uint16_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) h[t] = Ablk[(int64_t)(r + t) * lda + c];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const double a = (double)bits_f16(h[t]);
        s = __builtin_fma(a, a, s);   // a*a is exact, so this equals s + a*a rounded once
      }
    }
    for (; r < V; ++r) {
      const double a = (double)bits_f16(Ablk[(int64_t)r * lda + c]);
      s = __builtin_fma(a, a, s);
    }
    score[c] = s;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ncols; c += kVnmThreads) {
    const int gi = c / M;
    const int base = gi * M;
    const double sc = score[c];
    int rank = 0;
    for (int j = 0; j < M; ++j) {
      const double sj = score[base + j];
      rank += (sj > sc) | ((sj == sc) & (base + j < c));
    }
    keep[c] = rank < 4;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ncols; c += kVnmThreads) {
    if (!keep[c]) continue;
    const int gi = c / M;
    const int base = gi * M;
    int p = 0;
    for (int j = base; j < c; ++j) p += keep[j];
    if (p < 4) {      // always true for finite scores; guards unspecified non-finite input
      sel[gi * 4 + p] = (uint8_t)(c - base);
      colloc[((vb * G) + g0 + gi) * 4 + p] = (uint8_t)(c - base);
    }
  }
  __syncthreads();
  const int words = ng >> 2;
  for (int it = threadIdx.x; it < V * words; it += kVnmThreads) {
    const int r = it / words;
    const int w = it - r * words;
    const uint16_t* arow = Ablk + (int64_t)r * lda;
    uint32_t out[4];
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gi = 4 * w + q;
      const uint16_t* ag = arow + gi * M;
      uint32_t v0, v1;
      const uint32_t code = select_2of4(ag[sel[gi * 4 + 0]], ag[sel[gi * 4 + 1]], ag[sel[gi * 4 + 2]],
                                        ag[sel[gi * 4 + 3]], v0, v1);   // sel < M (phase 2)
      out[q] = v0 | (v1 << 16);
      word |= code << (4 * q);
    }
    const int64_t row = vb * V + r;
    u4 o = {out[0], out[1], out[2], out[3]};
    *reinterpret_cast<u4*>(values + vnm_value_at(row, g0 + 4 * w, G, tiled)) = o;
    midx[vnm_word_at(row, (g0 >> 2) + w, G, tiled)] = (uint16_t)word;
  }
}

// V:2:M with the workgroup's V x (GC*M) tile of A staged in LDS first (a full tile by the
// global -> LDS DMA path, every copy of the workgroup in flight; a ragged one by batches of
// eight 16-byte loads per thread), then the column scores (float64, rows in ascending order,
// four rows of a column per transpose read), the column-loc selection and the 2:4 encoding
// (one thread per (row, four groups), lanes on consecutive rows) all read LDS: one HBM read
// of A, no dependent global loads. Used whenever a tile of at least one metadata word of
// groups fits. Tiles of up to 64 KiB for tall blocks (V >= 128: fewer, longer score chains)
// and 32 KiB otherwise (more workgroups per CU to overlap the phases); measured on MI355X.
constexpr int kVnmTileBytes = 64 * 1024;
static int vnm_tile_bytes(int V) { return V >= 128 ? kVnmTileBytes : kVnmTileBytes / 2; }
// Row pitch (elements) of the staged tile for rows of `pitch` elements (a multiple of 8):
// an odd number of 16-byte chunks.
__host__ __device__ __forceinline__ int vnm_lds_pitch(int pitch) { return ((pitch >> 3) | 1) << 3; }

template <bool TILED>
__global__ void __launch_bounds__(kVnmThreads)
k_prune_encode_vnm_lds(const uint16_t* __restrict__ A, int64_t R, int64_t K, int64_t lda, int V,
                       int M, int GC, uint16_t* __restrict__ values, uint16_t* __restrict__ midx,
                       uint8_t* __restrict__ colloc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t G = K / M;
  const int64_t nchunks = (G + GC - 1) / GC;
  const int64_t vb = blockIdx.x / nchunks;
  const int64_t g0 = (blockIdx.x - vb * nchunks) * GC;
  const int ng = (int)((G - g0) < GC ? (G - g0) : GC);   // groups in this chunk (multiple of 4)
  const int ncols = ng * M;
  const int pitch = GC * M;                              // columns of a full tile
  // Staged rows are an odd number of 16-byte chunks apart (one pad chunk after rows of an
  // even number): phase 3 reads one column across consecutive rows (a lane per row), and
  // with an odd stride sixteen consecutive rows start in sixteen different bank groups
  // (a 384-byte row, V:2:16 with 12 groups, would otherwise put them on two banks).
  const int pitchp = vnm_lds_pitch(pitch);
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
  double* score = reinterpret_cast<double*>(smem + (size_t)V * pitchp * 2);
  uint8_t* sel = reinterpret_cast<uint8_t*>(score + pitch);   // [group in chunk][4]
  uint8_t* keep = sel + GC * 4;
  const uint16_t* Ablk = A + vb * V * lda + g0 * M;
  auto tcol = [&](int r, int col) -> int { return r * pitchp + col; };   // element of (r, col)

  // ---- stage the tile
  if (ncols == pitch && (((uintptr_t)Ablk) & 15) == 0 && (lda & 7) == 0) {
    // a full tile is dense in LDS up to the pad chunks: 16-byte slot ci = row-major slot
    // index, so each wave's DMA instruction fills 1 KiB of consecutive slots and every copy
    // of the workgroup is in flight at once; a pad slot takes a second copy of its row's
    // first chunk
    const int c8 = ncols >> 3;
    const int c8p = pitchp >> 3;
    const int n = V * c8p;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t tile_lds = lds_addr(smem);
    for (int b0 = 64 * wave; b0 < n; b0 += kVnmThreads) {
      const int ci = b0 + lane;
      if (ci < n) {   // the last instruction may be partial: its idle lanes write nothing
        const int r = ci / c8p;
        const int q = ci - r * c8p;
        const int c = (q < c8 ? q : 0) * 8;
        dma_v<16>(Ablk + (int64_t)r * lda + c, tile_lds + (uint32_t)b0 * 16u);
      }
    }
    wait_vmcnt<0>();
  } else if ((((uintptr_t)Ablk) & 15) == 0 && (ncols & 7) == 0 && (lda & 7) == 0) {
    // eight 16-byte loads in flight per thread before their LDS writes
    const int c8 = ncols >> 3;
    const int n = V * c8;
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kVnmThreads) {
      u4 v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = i0 + t * kVnmThreads;
        if (i < n) {
          const int r = i / c8;
          const int c = (i - r * c8) * 8;
          v[t] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(Ablk + (int64_t)r * lda + c));
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = i0 + t * kVnmThreads;
        if (i < n) {
          const int r = i / c8;
          const int c = (i - r * c8) * 8;
          *reinterpret_cast<u4*>(tile + r * pitchp + c) = v[t];
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < V * ncols; i += kVnmThreads) {
      const int r = i / ncols;
      const int c = i - r * ncols;
      tile[r * pitchp + c] = Ablk[(int64_t)r * lda + c];
    }
  }
  __syncthreads();
  // ---- phase 1: column scores, float64 sums in row order
  if (V % 16 == 0) {
    // each lane owns one column: a transpose read (ds_read_b64_tr_b16) gives it four
    // consecutive rows of that column, so a column of V rows costs V/4 LDS reads instead of
    // V. Lane gl of a 16-lane group reads row r0 + gl/4, columns cg + 4 (gl % 4) .. + 3; in
    // a group that straddles the end of the staged columns, the reads past them fall on the
    // row's pad chunk, the next row or, for the last row, the score array after the tile,
    // and are never used.
    const int lane = threadIdx.x & 63;
    const int gl = lane & 15;
    const uint32_t tile_lds = lds_addr(smem);
    for (int cw = (int)(threadIdx.x & ~63); cw < ncols; cw += kVnmThreads) {   // wave-uniform
      const int cg = cw + (lane & 48);
      const int c = cg + gl;
      // first of the four columns this lane reads (a group wholly past the staged columns
      // reads column 0 instead, unused)
      const int rc = (cg < ncols ? cg : 0) + 4 * (gl & 3);
      double s = 0.0;
      for (int r0 = 0; r0 < V; r0 += 16) {
        h4 q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) q[t] = lds_read_tr16(tile_lds + (uint32_t)(tcol(r0 + 4 * t + (gl >> 2), rc) * 2));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const double a = (double)q[t][e];
            s = __builtin_fma(a, a, s);   // a*a is exact, so this equals s + a*a rounded once
          }
      }
      if (c < ncols) score[c] = s;
    }
  } else
  for (int c = threadIdx.x; c < ncols; c += kVnmThreads) {
    double s = 0.0;
    int r = 0;
    for (; r + 8 <= V; r += 8) {
      uint16_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) h[t] = tile[tcol(r + t, c)];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const double a = (double)bits_f16(h[t]);
        s = __builtin_fma(a, a, s);   // a*a is exact, so this equals s + a*a rounded once
      }
    }
    for (; r < V; ++r) {
      const double a = (double)bits_f16(tile[tcol(r, c)]);
      s = __builtin_fma(a, a, s);
    }
    score[c] = s;
  }
  __syncthreads();
  // ---- phase 2: the four columns of largest score per group (ties to the lower column)
  for (int c = threadIdx.x; c < ncols; c += kVnmThreads) {
    const int gi = c / M;
    const int base = gi * M;
    const double sc = score[c];
    int rank = 0;
    int j = 0;
    for (; j + 4 <= M; j += 4) {
      double sj[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) sj[t] = score[base + j + t];
#pragma unroll
      for (int t = 0; t < 4; ++t) rank += (sj[t] > sc) | ((sj[t] == sc) & (base + j + t < c));
    }
    for (; j < M; ++j) {
      const double sj = score[base + j];
      rank += (sj > sc) | ((sj == sc) & (base + j < c));
    }
    keep[c] = rank < 4;
  }
  __syncthreads();
  // position of each kept column among its group's kept columns (ascending column order)
  const bool wave_groups = (64 % M) == 0;   // groups never straddle a wave
  for (int c0 = 0; c0 < ncols; c0 += kVnmThreads) {
    const int c = c0 + (int)threadIdx.x;
    const bool kc = c < ncols && keep[c];
    int p;
    const int gi = c / M;
    const int base = gi * M;
    if (wave_groups) {
      const uint64_t kb = __ballot(kc);
      const int lane = threadIdx.x & 63;
      const int lb = lane - (c - base);              // lane of the group's first column
      const uint64_t below = ((uint64_t)1 << lane) - 1;
      const uint64_t grp = lb > 0 ? ~(((uint64_t)1 << lb) - 1) : ~(uint64_t)0;
      p = __popcll(kb & below & grp);
    } else {
      p = 0;
      if (kc)
        for (int j = base; j < c; ++j) p += keep[j];
    }
    if (kc && p < 4) {   // p < 4 always for finite scores; guards unspecified non-finite input
      sel[gi * 4 + p] = (uint8_t)(c - base);
      colloc[((vb * G) + g0 + gi) * 4 + p] = (uint8_t)(c - base);
    }
  }
  __syncthreads();
  // ---- phase 3: 2:4 among the selected columns, one thread per (row, four groups): lanes
  // take consecutive rows of one run of four groups, so the groups' column selections are
  // the same across the wave, each thread writes one 16-byte piece of values and one index
  // word, and in the row-group interleaved storage 32 consecutive rows of a run of four
  // groups are 512 contiguous bytes.
  const int nw = ng >> 2;
  const int nitems = V * nw;
  for (int it = threadIdx.x; it < nitems; it += kVnmThreads) {
    const int w = it / V;
    const int r = it - w * V;
    uint32_t out[4];
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = 4 * w + q;
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(sel + g * 4);
      const int cb = g * M;
      const uint32_t p01 = (uint32_t)tile[tcol(r, cb + (int)(sw & 0xFFu))] |
                           ((uint32_t)tile[tcol(r, cb + (int)((sw >> 8) & 0xFFu))] << 16);
      const uint32_t p23 = (uint32_t)tile[tcol(r, cb + (int)((sw >> 16) & 0xFFu))] |
                           ((uint32_t)tile[tcol(r, cb + (int)(sw >> 24))] << 16);
      uint32_t kept;
      word |= select_2of4_keys(p01, p23, kept) << (4 * q);
      out[q] = kept;
    }
    const int64_t row = vb * V + r;
    u4 o = {out[0], out[1], out[2], out[3]};
    *reinterpret_cast<u4*>(values + vnm_value_at(row, g0 + 4 * w, G, TILED)) = o;
    midx[vnm_word_at(row, (g0 >> 2) + w, G, TILED)] = (uint16_t)word;
  }
}

hipError_t launch_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, void* values,
                                  void* meta, hipStream_t stream) {
  const int64_t total = R * (K >> 4);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;   // grid-stride beyond 64 workgroups per CU
  hipLaunchKernelGGL(k_prune_encode_nm, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)A, R, K, lda, (uint16_t*)values, (uint16_t*)meta);
  return hipGetLastError();
}

hipError_t launch_prune_encode_nm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, void* values_t,
                                        void* meta_t, hipStream_t stream) {
  const int64_t total = ((R + 15) >> 4) * ((K + 63) >> 6) * 64;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(k_prune_encode_nm_tiled, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)A, R, K, lda, (uint16_t*)values_t, (uint16_t*)meta_t);
  return hipGetLastError();
}

int vnm_chunk_groups(int M) {
  int gc = (256 / M) & ~3;
  return gc < 4 ? 4 : gc;
}

// Groups per workgroup of the LDS-staged kernel: the most whose V x GC*M tile fits
// kVnmTileBytes with the score arrays, in steps of 4 groups (one metadata word; with M
// even that also keeps every chunk on a 16-byte boundary) or of 8 for odd M; 0 if not
// even one step fits.
static int vnm_lds_groups(int V, int M) {
  const int per_group = M * (V * 2 + 8 + 2);   // tile column + score + keep/sel bytes
  const int step = (M % 2 == 0) ? 4 : 8;
  int gc = vnm_tile_bytes(V) / per_group / step * step;
  if (gc > 256) gc = 256;
  return gc >= step ? gc : 0;
}

hipError_t launch_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                                   void* values, void* midx, void* colloc, bool tiled,
                                   hipStream_t stream) {
  if (R == 0 || K == 0) return hipSuccess;
  const int GL = vnm_lds_groups(V, M);
  if (GL > 0) {
    const int64_t G = K / M;
    const int64_t nchunks = (G + GL - 1) / GL;
    const int64_t blocks = (R / V) * nchunks;
    const size_t lds = (size_t)V * vnm_lds_pitch(GL * M) * 2 + (size_t)GL * M * (8 + 1) + (size_t)GL * 4;   // tile, score, keep, sel
    static std::atomic<uint64_t> lds_set{0};
    auto kern = tiled ? k_prune_encode_vnm_lds<true> : k_prune_encode_vnm_lds<false>;
    static std::atomic<uint64_t> lds_set_t{0};
    if (hipError_t e = ensure_lds_limit(tiled ? lds_set_t : lds_set, (const void*)kern, 96 * 1024)) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kVnmThreads), lds, stream,
                       (const uint16_t*)A, R, K, lda, V, M, GL, (uint16_t*)values, (uint16_t*)midx,
                       (uint8_t*)colloc);
    return hipGetLastError();
  }
  const int GC = vnm_chunk_groups(M);
  const int64_t G = K / M;
  const int64_t nchunks = (G + GC - 1) / GC;
  const int64_t blocks = (R / V) * nchunks;
  hipLaunchKernelGGL(k_prune_encode_vnm, dim3((unsigned)blocks), dim3(kVnmThreads), 0, stream,
                     (const uint16_t*)A, R, K, lda, V, M, GC, (uint16_t*)values, (uint16_t*)midx,
                     (uint8_t*)colloc, (int)tiled);
  return hipGetLastError();
}

}  // namespace snm
