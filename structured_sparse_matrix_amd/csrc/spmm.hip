// Structured-sparse x dense products on the CDNA4 sparse matrix cores.
//
// Y = decode(values, meta) * B for 2:4 ("2:4 sparsity on sparse tensor cores", lecture
// notes: "How the tensor core uses it" -- the 2-bit tags select which K/2 elements of
// each B column are multiplied) and for V:2:M ("VENOM ...", SC'23, Sec. 4 and Fig. 4 --
// per block of V rows the K/M*4 rows of B named by column-loc are gathered, which turns
// the product into a 2:4 product over K' = 4K/M).
//
// One kernel template serves both: it runs 2:4 over a "compressed space" of length Kc
// (Kc = K for 2:4, Kc = 4K/M for V:2:M). The only difference is how the rows of the B
// tile are fetched: contiguous rows (2:4) or rows gathered through column-loc (V:2:M).
//
// Work decomposition
//   workgroup tile  BM x BN outputs, BM = WM*TM*16 rows, BN = WN*TN*16 columns;
//   WK waves split the reduction inside the workgroup (summed through LDS at the end).
//   superchunk      KS = 64*KSUB consecutive positions of the compressed space, i.e.
//                   KSUB sparse-MFMA operands; in operand t lane quarter q holds
//                   positions 64t + 16q + [0, 16) (the instruction's own order, so the
//                   operand-major storage of snm_spmm_nm_tiled is one 1 KiB block).
//   A operand       loaded straight from HBM into registers (non-temporal, read once);
//                   the canonical metadata word is the sparse-MFMA index operand as is.
//   B operand       the KS x BN tile is staged in LDS (rows as stored, 32-byte cells
//                   XOR-swizzled so that one transpose read touches every bank pair at
//                   most twice) and read column-wise with ds_read_b64_tr_b16.
//   pipelining      the next superchunk's A fragments and B rows are loaded into
//                   registers while the current one is multiplied.
#include "device_common.hpp"
#include "launch.hpp"
#include "variant.hpp"

namespace snm {

struct SpmmArgs {
  const uint16_t* values;   // fp16 bits, R x Kc/2 per batch entry
  const uint8_t* meta;      // R x Kc/8 bytes per batch entry
  const uint16_t* B;        // fp16 bits, K x C (row-major, ldb)
  uint16_t* Y;              // fp16 bits, R x C (ldy)
  const uint8_t* colloc;    // V:2:M only: (R/V) x (K/M) x 4
  int64_t R, Kc, K, C, ldb, ldy;
  int64_t batch, stride_values, stride_meta, stride_B, stride_Y;
  int64_t n_row_tiles, n_col_tiles;
  int V, M;
  int b_vec;                // B rows are 16-byte aligned: load 8 columns at a time
};

// Byte offset, inside a B tile of BN fp16 columns, of (row x, column c) with c a multiple
// of 4. Cells of 32 bytes (16 columns) are XOR-permuted inside 256-byte lines (one line
// spans all 64 LDS banks) so that the 16 rows one transpose read touches -- rows
// {0..3, 8..11, 16..19, 24..27} + const -- fall on 8 distinct cells, each at most twice.
template <int BN>
__device__ __forceinline__ uint32_t btile_offset(int x, int c) {
  const int cr = c >> 4;
  const uint32_t inner = (uint32_t)(c & 15) * 2u;
  if constexpr (BN >= 128) {
    const int hx = (x & 3) | ((x >> 1) & 4);
    return (uint32_t)x * (BN * 2) + (uint32_t)((cr ^ hx) * 32) + inner;
  } else if constexpr (BN == 64) {
    const int L = x >> 1;
    int u = ((x & 1) << 2) | cr;
    u ^= (L & 1) | (((L >> 2) & 1) << 1);
    return (uint32_t)L * 256u + (uint32_t)u * 32u + inner;
  } else if constexpr (BN == 32) {
    const int L = x >> 2;
    int u = ((x & 3) << 1) | cr;
    u ^= (L >> 1) & 1;
    return (uint32_t)L * 256u + (uint32_t)u * 32u + inner;
  } else {
    static_assert(BN == 16, "BN must be 16, 32, 64 or a multiple of 128");
    const int L = x >> 3;
    int u = x & 7;
    u ^= (L & 1) << 2;
    return (uint32_t)L * 256u + (uint32_t)u * 32u + inner;
  }
}

template <int WM, int WN, int WK, int TM, int TN, int KSUB, bool GATHER, bool BCOL, bool ATILED = false>
struct SpmmCfg {
  static constexpr int kWaves = WM * WN * WK;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = WM * TM * 16;
  static constexpr int BN = WN * TN * 16;
  static constexpr int KS = 64 * KSUB;                 // compressed positions per superchunk
  static constexpr int kTileRows = WK * KS;            // B rows staged per iteration
  static constexpr int kChunksPerRow = BN / 8;         // 16-byte chunks per B row
  static constexpr int kChunksPerCol = kTileRows / 8;  // 16-byte chunks per B column (BCOL)
  static constexpr int kChunks = kTileRows * kChunksPerRow;
  static constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
  // column-major B is staged as [column][k]: a 16-byte pad per column rotates the banks
  static constexpr int kColPitch = kTileRows * 2 + 16;
  static constexpr int kLdsB = BCOL ? BN * kColPitch : kTileRows * BN * 2;
  static constexpr int kLdsRed = (WK - 1) * WM * WN * TM * TN * 64 * 16;
  static constexpr int kLds = kLdsB > kLdsRed ? kLdsB : kLdsRed;
  static_assert(kChunks % kThreads == 0, "B tile must split evenly over the workgroup");
};

template <int WM, int WN, int WK, int TM, int TN, int KSUB, bool GATHER, bool BCOL, bool ATILED>
__global__ void __launch_bounds__(64 * WM * WN * WK)
k_spmm(SpmmArgs a) {
  using Cfg = SpmmCfg<WM, WN, WK, TM, TN, KSUB, GATHER, BCOL, ATILED>;
  static_assert(!(GATHER && BCOL), "gathered rows need row-major B");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, KS = Cfg::KS;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds_base = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;
  const int wm = (wave / WN) % WM;
  const int wk = wave / (WN * WM);
  const int q = lane >> 4;      // lane quarter
  const int li = lane & 15;

  const int64_t tile = blockIdx.x;
  const int64_t rt = tile % a.n_row_tiles;
  const int64_t ct = tile / a.n_row_tiles;
  const int64_t row0 = rt * BM;
  const int64_t col0 = ct * BN;
  const int64_t nsuper = (a.Kc + KS - 1) / KS;
  const int64_t vals_row = a.Kc >> 1;     // elements
  const int64_t meta_row = a.Kc >> 3;     // bytes
  const int64_t KCt = (a.Kc + 63) >> 6;   // operand-major: 64-position blocks per row tile
  const int64_t G = GATHER ? a.K / a.M : 0;
  const int64_t vb = GATHER ? row0 / a.V : 0;

  for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
    const uint16_t* __restrict__ vals = a.values + b * a.stride_values;
    const uint8_t* __restrict__ meta = a.meta + b * a.stride_meta;
    const uint16_t* __restrict__ Bm = a.B + b * a.stride_B;
    uint16_t* __restrict__ Y = a.Y + b * a.stride_Y;

    // ---- register staging ------------------------------------------------------------
    u4 bstage[Cfg::kChunksPerThread];
    h8 afrag[TM][KSUB];
    uint32_t aidx[TM][KSUB];

    auto load_b = [&](int64_t s0) {
#pragma unroll
      for (int i = 0; i < Cfg::kChunksPerThread; ++i) {
        const int chunk = tid + i * Cfg::kThreads;
        u4 v = {0u, 0u, 0u, 0u};
        if constexpr (BCOL) {
          // eight consecutive k of one column
          const int c = chunk / Cfg::kChunksPerCol;
          const int kc = chunk - c * Cfg::kChunksPerCol;
          const int64_t kg = s0 * KS + kc * 8;
          const int64_t col = col0 + c;
          if (kg < a.Kc && col < a.C) {
            const uint16_t* src = Bm + col * a.ldb + kg;
            if (a.b_vec) {
              v = *reinterpret_cast<const u4*>(src);
            } else {
              v[0] = src[0] | ((uint32_t)src[1] << 16);
              v[1] = src[2] | ((uint32_t)src[3] << 16);
              v[2] = src[4] | ((uint32_t)src[5] << 16);
              v[3] = src[6] | ((uint32_t)src[7] << 16);
            }
          }
        } else {
          const int j = chunk / Cfg::kChunksPerRow;           // tile row
          const int cc = chunk - j * Cfg::kChunksPerRow;      // 16-byte chunk in the row
          const int64_t kg = s0 * KS + j;                     // compressed-space position
          const int64_t col = col0 + cc * 8;
          if (kg < a.Kc) {
            int64_t brow;
            if constexpr (GATHER) {
              const int64_t g = kg >> 2;
              const int cl = a.colloc[(vb * G + g) * 4 + (kg & 3)];
              brow = g * a.M + (cl < a.M ? cl : a.M - 1);   // column-loc entries are < M by contract
            } else {
              brow = kg;
            }
            const uint16_t* src = Bm + brow * a.ldb + col;
            if (a.b_vec && col + 8 <= a.C) {
              v = *reinterpret_cast<const u4*>(src);
            } else {
              uint16_t e[8];
#pragma unroll
              for (int t = 0; t < 8; ++t) e[t] = (col + t < a.C) ? src[t] : (uint16_t)0;
              v[0] = e[0] | ((uint32_t)e[1] << 16);
              v[1] = e[2] | ((uint32_t)e[3] << 16);
              v[2] = e[4] | ((uint32_t)e[5] << 16);
              v[3] = e[6] | ((uint32_t)e[7] << 16);
            }
          }
        }
        bstage[i] = v;
      }
    };
    auto store_b = [&]() {
#pragma unroll
      for (int i = 0; i < Cfg::kChunksPerThread; ++i) {
        const int chunk = tid + i * Cfg::kThreads;
        if constexpr (BCOL) {
          const int c = chunk / Cfg::kChunksPerCol;
          const int kc = chunk - c * Cfg::kChunksPerCol;
          *reinterpret_cast<u4*>(smem + c * Cfg::kColPitch + kc * 16) = bstage[i];
        } else {
          const int j = chunk / Cfg::kChunksPerRow;
          const int cc = chunk - j * Cfg::kChunksPerRow;
          *reinterpret_cast<u4*>(smem + btile_offset<BN>(j, cc * 8)) = bstage[i];
        }
      }
    };
    auto load_a = [&](int64_t s0) {
      const int64_t s = s0 + wk;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int64_t rtile = (row0 >> 4) + wm * TM + tm;
        const int64_t row = rtile * 16 + li;
#pragma unroll
        for (int t = 0; t < KSUB; ++t) {
          const int64_t kd = s * KS + 64 * t + 16 * q;   // first dense position of this lane
          h8 v = {};
          uint32_t id = 0;
          if constexpr (ATILED) {
            // operand-major: block (rtile, kd/64) is 64 lanes x 16 bytes (+ 64 metadata words);
            // padded rows are stored as zeros, so only the tile and position range matter
            if (s < nsuper && kd < a.Kc && rtile * 16 < a.R) {
              const int64_t blk = rtile * KCt + (kd >> 6);
              v = __builtin_bit_cast(h8, __builtin_nontemporal_load(
                                             reinterpret_cast<const u4*>(vals + (blk * 64 + lane) * 8)));
              id = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(meta + (blk * 64 + lane) * 2));
            }
          } else {
            if (s < nsuper && kd < a.Kc && row < a.R) {
              v = __builtin_bit_cast(h8, __builtin_nontemporal_load(
                                             reinterpret_cast<const u4*>(vals + row * vals_row + (kd >> 1))));
              id = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(meta + row * meta_row + (kd >> 3)));
            }
          }
          afrag[tm][t] = v;
          aidx[tm][t] = id;
        }
      }
    };

    f4 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f4{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_b(0);
    for (int64_t s0 = 0; s0 < nsuper; s0 += WK) {
      store_b();
      __syncthreads();
      h8 acur[TM][KSUB];
      uint32_t icur[TM][KSUB];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int t = 0; t < KSUB; ++t) { acur[tm][t] = afrag[tm][t]; icur[tm][t] = aidx[tm][t]; }
      if (s0 + WK < nsuper) {   // next superchunks in flight during this one's products
        load_a(s0 + WK);
        load_b(s0 + WK);
      }
      if (s0 + wk < nsuper) {
        const int xbase = wk * KS;
#pragma unroll
        for (int t = 0; t < KSUB; ++t) {
          // operand rows: e < 8 -> 64t + 8q + e ; e >= 8 -> 64t + 32 + 8q + e - 8
          const int r1 = 64 * t + 8 * q + (li >> 2);
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            h16 bf;
            if constexpr (BCOL) {
              // [column][k] tile: eight consecutive k of one column are one 16-byte read
              const int col = (wn * TN + tn) * 16 + li;
              const int k1 = xbase + r1 - (li >> 2);
              const h8 lo = *reinterpret_cast<const h8*>(smem + col * Cfg::kColPitch + k1 * 2);
              const h8 hi = *reinterpret_cast<const h8*>(smem + col * Cfg::kColPitch + (k1 + 32) * 2);
#pragma unroll
              for (int e = 0; e < 8; ++e) { bf[e] = lo[e]; bf[8 + e] = hi[e]; }
            } else {
              const int c = (wn * TN + tn) * 16 + 4 * (li & 3);
              const h4 b0 = lds_read_tr16(lds_base + btile_offset<BN>(xbase + r1, c));
              const h4 b1 = lds_read_tr16(lds_base + btile_offset<BN>(xbase + r1 + 4, c));
              const h4 b2 = lds_read_tr16(lds_base + btile_offset<BN>(xbase + r1 + 32, c));
              const h4 b3 = lds_read_tr16(lds_base + btile_offset<BN>(xbase + r1 + 36, c));
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                bf[e] = b0[e];
                bf[4 + e] = b1[e];
                bf[8 + e] = b2[e];
                bf[12 + e] = b3[e];
              }
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) acc[tm][tn] = smfmac16<0>(acur[tm][t], bf, acc[tm][tn], icur[tm][t]);
          }
        }
      }
      __syncthreads();
    }

    // ---- reduce the WK partial sums of the workgroup -------------------------------------
    if constexpr (WK > 1) {
      float* red = reinterpret_cast<float*>(smem);
      const int slot = ((wm * WN + wn) * TM) * TN;
      if (wk > 0) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            *reinterpret_cast<f4*>(red + ((((wk - 1) * WM * WN * TM * TN) + slot + tm * TN + tn) * 64 + lane) * 4) =
                acc[tm][tn];
      }
      __syncthreads();
      if (wk == 0) {
        for (int w = 1; w < WK; ++w)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
              acc[tm][tn] += *reinterpret_cast<const f4*>(
                  red + ((((w - 1) * WM * WN * TM * TN) + slot + tm * TN + tn) * 64 + lane) * 4);
      }
      __syncthreads();
    }
    if (wk == 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int64_t col = col0 + (wn * TN + tn) * 16 + li;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t row = row0 + (wm * TM + tm) * 16 + 4 * q + i;
            if (row < a.R && col < a.C) Y[row * a.ldy + col] = f16_bits(to_f16(acc[tm][tn][i]));
          }
        }
    }
  }
}

// ---- host side: pick a tile shape for the problem and launch ------------------------------

template <int WM, int WN, int WK, int TM, int TN, int KSUB, bool GATHER, bool BCOL = false, bool ATILED = false>
static hipError_t launch_cfg(SpmmArgs a, hipStream_t stream) {
  using Cfg = SpmmCfg<WM, WN, WK, TM, TN, KSUB, GATHER, BCOL, ATILED>;
  a.n_row_tiles = (a.R + Cfg::BM - 1) / Cfg::BM;
  a.n_col_tiles = (a.C + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = a.n_row_tiles * a.n_col_tiles;
  if (tiles == 0 || a.batch == 0) return hipSuccess;
  const unsigned gy = (unsigned)(a.batch < 65535 ? a.batch : 65535);
  auto kern = k_spmm<WM, WN, WK, TM, TN, KSUB, GATHER, BCOL, ATILED>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, Cfg::kLds)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, gy), dim3(Cfg::kThreads), Cfg::kLds, stream, a);
  return hipGetLastError();
}

hipError_t launch_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                          int64_t C, int64_t ldb, int b_layout, void* Y, int64_t ldy, int64_t batch,
                          int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                          int64_t stride_Y, hipStream_t stream) {
  const bool generic = forced_variant() == Variant::kGeneric;
  if (C <= 32 && !generic) {   // decode regime: weight streaming, see spmm_skinny.hip
    log_variant("spmm_nm", R, K, C,
                batch == 1 && skinny_ring_selected(K, B, C, ldb, b_layout, false) ? "skinny ring" : "skinny");
    return launch_spmm_nm_skinny(values, meta, R, K, B, C, ldb, b_layout, Y, ldy, batch,
                                 stride_values, stride_meta, stride_B, stride_Y, stream);
  }
  if (b_layout == 0 && !generic && spmm_wide_eligible(R, K, 0, 4, B, C, ldb, batch, stride_B)) {
    log_variant("spmm_nm", R, K, C, "wide");
    return launch_spmm_wide(values, meta, nullptr, R, K, 0, 4, B, C, ldb, Y, ldy, batch,
                            stride_values, stride_meta, stride_B, stride_Y, stream);
  }
  log_variant("spmm_nm", R, K, C, "generic");
  SpmmArgs a{};
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.colloc = nullptr;
  a.R = R; a.Kc = K; a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = batch;
  a.stride_values = stride_values; a.stride_meta = stride_meta;
  a.stride_B = stride_B; a.stride_Y = stride_Y;
  a.V = 0; a.M = 4;
  a.b_vec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0) && (batch <= 1 || stride_B % 8 == 0);
  if (b_layout == 1) {
    if (C <= 64) return launch_cfg<4, 1, 1, 2, 4, 4, false, true>(a, stream);
    return launch_cfg<2, 2, 1, 2, 4, 2, false, true>(a, stream);
  }
  if (C <= 64) return launch_cfg<4, 1, 1, 2, 4, 4, false>(a, stream);
  return launch_cfg<2, 2, 1, 2, 4, 2, false>(a, stream);
}

hipError_t launch_spmm_nm_tiled(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                int64_t ldy, hipStream_t stream) {
  if (C <= 32 && forced_variant() != Variant::kGeneric) {
    log_variant("spmm_nm_tiled", R, K, C, skinny_ring_selected(K, B, C, ldb, b_layout, true) ? "skinny ring" : "skinny");
    return launch_spmm_nm_tiled_skinny(values_t, meta_t, R, K, B, C, ldb, b_layout, Y, ldy, stream);
  }
  log_variant("spmm_nm_tiled", R, K, C, "generic");
  SpmmArgs a{};
  a.values = (const uint16_t*)values_t;
  a.meta = (const uint8_t*)meta_t;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.colloc = nullptr;
  a.R = R; a.Kc = K; a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = 1;
  a.V = 0; a.M = 4;
  a.b_vec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0);
  // row tiles of a workgroup must be 16-row aligned tiles of the operand-major array: BM
  // is a multiple of 16, which every configuration satisfies
  if (b_layout == 1) {
    if (C <= 64) return launch_cfg<4, 1, 1, 2, 4, 4, false, true, true>(a, stream);
    return launch_cfg<2, 2, 1, 2, 4, 2, false, true, true>(a, stream);
  }
  if (C <= 64) return launch_cfg<4, 1, 1, 2, 4, 4, false, false, true>(a, stream);
  return launch_cfg<2, 2, 1, 2, 4, 2, false, false, true>(a, stream);
}

hipError_t launch_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R,
                           int64_t K, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                           int64_t ldy, hipStream_t stream) {
  if (forced_variant() != Variant::kGeneric && spmm_wide_eligible(R, 4 * (K / M), V, M, B, C, ldb, 1, 0))
    return launch_spmm_wide(values, midx, colloc, R, 4 * (K / M), V, M, B, C, ldb, Y, ldy, 1, 0, 0,
                            0, 0, stream);   // logs the tile it picks
  log_variant("spmm_vnm", R, K, C, "generic");
  SpmmArgs a{};
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)midx;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.colloc = (const uint8_t*)colloc;
  a.R = R; a.Kc = 4 * (K / M); a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = 1;
  a.stride_values = 0; a.stride_meta = 0; a.stride_B = 0; a.stride_Y = 0;
  a.V = V; a.M = M;
  a.b_vec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0);
  // The row tile must not straddle two V-blocks: BM divides V.
  if (V % 64 == 0) return launch_cfg<2, 2, 1, 2, 4, 2, true>(a, stream);   // BM = 64, BN = 128
  if (V % 32 == 0) return launch_cfg<2, 2, 1, 1, 4, 2, true>(a, stream);   // BM = 32, BN = 128
  return launch_cfg<1, 4, 1, 1, 2, 2, true>(a, stream);                    // BM = 16, BN = 128
}

hipError_t launch_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc,
                                 int64_t R, int64_t K, int V, int M, const void* B, int64_t C,
                                 int64_t ldb, void* Y, int64_t ldy, hipStream_t stream) {
  const int64_t Kc = 4 * (K / M);
  if (V % 32 != 0 || !spmm_wide_supported(R, Kc, V, M, B, C, ldb, 1, 0)) return hipErrorInvalidValue;
  return launch_spmm_wide(values_t, midx_t, colloc, R, Kc, V, M, B, C, ldb, Y, ldy, 1, 0, 0, 0, 0,
                          stream, true);
}

}  // namespace snm
