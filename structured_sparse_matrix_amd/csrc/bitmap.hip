// Bitmap-compressed unstructured sparsity ("Coruscant: Co-Designing GPU Kernel and Sparse
// Tensor Core ...", Sec. 3.1 and Fig. 7: 64-element tiles, each stored as its non-zero
// values plus a 64-bit bitmap, and tile offsets; Sec. 3.2: each tile's values padded to a
// multiple of 8 so one 16-byte load serves them) and its decode-shaped product.
//
// Design for MI355X (gfx950):
//   * a tile is 64 consecutive positions along K of one row, so one byte of its bitmap
//     covers exactly the 8 consecutive k that one lane holds in the dense
//     v_mfma_f32_16x16x32_f16 A operand; the 16-bit element ranks a lane needs are
//     popcounts of the bitmap below its byte.
//   * the encoder runs in three steps -- per-row bitmaps, padded counts and in-row
//     offsets; one workgroup scanning the row totals; the final offsets -- then writes
//     the values in a separate call, once the caller has allocated them.
//   * the product: one workgroup per 16 rows, eight waves splitting K; each wave copies its
//     rows' packed values for a phase of 4 tiles (16-byte aligned spans, because every
//     tile starts at a multiple of 8 values) into its own LDS region with the
//     global->LDS DMA, then expands each 8-position chunk through its bitmap byte with
//     LDS reads at the computed ranks, and runs a dense MFMA on the expanded operand.
//     Partial sums of the waves are added through LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace snm {
namespace {

constexpr int kTile = 64;

__device__ __forceinline__ uint32_t nz_mask8(const u4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m |= ((v[w] & 0x7FFFu) != 0u ? 1u : 0u) << (2 * w);
    m |= ((v[w] & 0x7FFF0000u) != 0u ? 1u : 0u) << (2 * w + 1);
  }
  return m;
}

// One wave per row, four rows per workgroup; every wave runs the same number of
// iterations (rows past R do no memory work) so the workgroup barriers are uniform.
// Per iteration a wave covers 512 positions = 8 tiles: lane l holds positions
// base + 8l .. + 7 (tile l / 8, byte l % 8 of its bitmap).
// Writes bitmaps, offsets[r*T + t] = offset of tile t relative to the row (t >= 1) and
// offsets[r*T] = the row's total padded count.
__global__ void __launch_bounds__(256) k_bitmap_count(const uint16_t* __restrict__ A, int64_t R,
                                                      int64_t K, int64_t lda,
                                                      uint64_t* __restrict__ bitmaps,
                                                      uint32_t* __restrict__ offsets) {
  __shared__ uint8_t sbyte[4][64];
  __shared__ uint32_t scount[4][8];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + w;
  const bool row_ok = r < R;
  const int64_t T = K / kTile;
  const int tin = lane >> 3, c = lane & 7;
  uint32_t running = 0;
  for (int64_t base = 0; base < K; base += 512) {
    const int64_t kt = base / kTile + tin;
    const bool ok = row_ok && kt < T;
    u4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u4*>(A + r * lda + base + 8 * lane);
    sbyte[w][lane] = (uint8_t)nz_mask8(v);
    __syncthreads();
    const uint64_t bm = *reinterpret_cast<const uint64_t*>(&sbyte[w][8 * tin]);
    const uint32_t pad = ok ? (((uint32_t)__popcll(bm) + 7u) & ~7u) : 0u;
    if (c == 0) scount[w][tin] = pad;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t x = scount[w][u];
      pre += u < tin ? x : 0u;
      tot += x;
    }
    if (ok && c == 0) {
      bitmaps[r * T + kt] = bm;
      if (kt > 0) offsets[r * T + kt] = running + pre;
    }
    running += tot;
    __syncthreads();   // LDS is rewritten by the next iteration
  }
  if (row_ok && lane == 0) offsets[r * T] = running;
}

// Exclusive scan of the row totals held at offsets[r*T] (one workgroup): afterwards
// offsets[r*T] is the absolute offset of row r's first tile and offsets[R*T] the total.
__global__ void __launch_bounds__(1024) k_bitmap_scan_rows(uint32_t* __restrict__ offsets, int64_t R,
                                                           int64_t T) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (R + 1023) / 1024;
  const int64_t r0 = tid * per;
  const int64_t r1 = r0 + per < R ? r0 + per : R;
  uint32_t s = 0;
  for (int64_t r = r0; r < r1; ++r) s += offsets[r * T];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive Hillis-Steele scan of the 1024 parts
    const uint32_t x = tid >= d ? part[tid - d] : 0u;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  uint32_t base = tid > 0 ? part[tid - 1] : 0u;
  for (int64_t r = r0; r < r1; ++r) {
    const uint32_t x = offsets[r * T];
    offsets[r * T] = base;
    base += x;
  }
  if (tid == 1023) offsets[R * T] = part[1023];
}

// offsets[r*T + t] += offsets[r*T] for t >= 1.
__global__ void __launch_bounds__(256) k_bitmap_fix_offsets(uint32_t* __restrict__ offsets, int64_t R,
                                                            int64_t T) {
  const int64_t n = R * T;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i % T;
    if (t != 0) offsets[i] += offsets[i - t];
  }
}

// Values: lane l (positions base + 8l .. + 7) writes its non-zeros at the tile's offset
// plus their rank in the tile; lane 7 of a tile writes the zero padding.
__global__ void __launch_bounds__(256) k_bitmap_values(const uint16_t* __restrict__ A, int64_t R,
                                                       int64_t K, int64_t lda,
                                                       const uint64_t* __restrict__ bitmaps,
                                                       const uint32_t* __restrict__ offsets,
                                                       uint16_t* __restrict__ values) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;   // no barriers in this kernel
  const int64_t T = K / kTile;
  const int tin = lane >> 3, c = lane & 7;
  for (int64_t base = 0; base < K; base += 512) {
    const int64_t kt = base / kTile + tin;
    if (kt >= T) continue;
    const u4 v = *reinterpret_cast<const u4*>(A + r * lda + base + 8 * lane);
    const uint64_t bm = bitmaps[r * T + kt];
    const uint64_t below = c == 0 ? 0ull : (bm & ((1ull << (8 * c)) - 1ull));
    uint32_t pos = offsets[r * T + kt] + (uint32_t)__popcll(below);
    const uint32_t m = (uint32_t)(bm >> (8 * c)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (m & (1u << e)) {
        const uint32_t word = v[e >> 1];
        values[pos] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xFFFFu));
        ++pos;
      }
    }
    if (c == 7) {
      const uint32_t cnt = (uint32_t)__popcll(bm);
      const uint32_t start = offsets[r * T + kt];
      for (uint32_t p = cnt; p < ((cnt + 7u) & ~7u); ++p) values[start + p] = 0;
    }
  }
}

// ---- product --------------------------------------------------------------------------
struct BitmapArgs {
  const uint64_t* bitmaps;
  const uint32_t* offsets;
  const uint16_t* values;
  const uint16_t* B;
  uint16_t* Y;
  int64_t R, K, C, ldb, ldy;
  int b_col;   // 1: B column-major (element (k, c) at B[c*ldb + k]) with 16-byte rows
};

__device__ __forceinline__ f4 mfma16x16x32(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One workgroup (kBmWaves waves) per 16-row tile; wave w takes a contiguous 1/kBmWaves of
// the row's tiles and walks it in phases of 4 tiles (256 positions). Eight waves and two
// workgroups per CU keep sixteen phases' loads in flight per CU. Lane l = 16q + i works on row
// i; in tile t it covers positions 32 blk + 8q + [0, 8), blk = 0, 1 (bitmap byte
// 4 blk + q) -- the dense MFMA A operand of k-block (t, blk).
// Per phase: (1) the packed values of the phase's 4 tiles of every row of the tile (a
// contiguous, 16-byte aligned span of at most 256 values) are copied by DMA into the
// wave's LDS region, row i at [512 i, 512 i + 512): DMA b covers rows 2b and 2b + 1, lane
// l one 16-byte chunk (lanes past a row's span stay inactive); (2) the B operands are
// loaded; (3) each chunk is expanded through its bitmap byte -- the e-th set bit takes
// the next value of the span, at LDS byte 512 i + 2 (tile offset - span start + rank) --
// and multiplied on the matrix core.
constexpr int kBmWaves = 8;
constexpr int kWaveBytes = 8192;                      // staged values of one wave
constexpr int kLutOff = kBmWaves * kWaveBytes + 16;   // + a pad that over-reads may touch
constexpr int kLutBytes = 256 * 16 + 256 * 8;
constexpr int kBitmapLds = kLutOff + kLutBytes;

template <int CT, bool BCOL>
__global__ void __launch_bounds__(64 * kBmWaves) __attribute__((amdgpu_waves_per_eu(4)))
k_spmm_bitmap(BitmapArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];   // 8 KiB per wave, then the expansion table
  // Expansion table, one entry per bitmap byte m: four dwords of 16-bit keep masks (0xFFFF
  // where bit e of m is set) and two dwords of eight byte offsets (2 rank_e, rank_e = set
  // bits of m below e). Expanding a chunk is then one address add and one read per
  // position, and one AND per pair of positions.
  for (int m = threadIdx.x; m < 256; m += 64 * kBmWaves) {
    uint32_t mk[4], rk[2] = {0u, 0u}, r = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rk[e >> 2] |= (2u * r) << (8 * (e & 3));
      r += (m >> e) & 1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mk[i] = (((m >> (2 * i)) & 1) ? 0xFFFFu : 0u) | (((m >> (2 * i + 1)) & 1) ? 0xFFFF0000u : 0u);
    *reinterpret_cast<u4*>(smem + kLutOff + 16 * m) = u4{mk[0], mk[1], mk[2], mk[3]};
    *reinterpret_cast<u2*>(smem + kLutOff + 4096 + 8 * m) = u2{rk[0], rk[1]};
  }
  __syncthreads();
  constexpr int kPhaseTiles = 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q = lane >> 4;
  const int li = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t row = row0 + li;
  const bool row_ok = row < a.R;
  const int64_t T = a.K / kTile;
  const int64_t tw = (T + kBmWaves - 1) / kBmWaves;     // tiles per wave
  const int64_t tbeg = (int64_t)w * tw;
  const int64_t tend = tbeg + tw < T ? tbeg + tw : T;
  uint8_t* const wl = smem + w * kWaveBytes;
  const uint32_t wl_lds = lds_addr(wl);

  f4 acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t kt0 = tbeg; kt0 < tend; kt0 += kPhaseTiles) {
    const int nt = (int)(tend - kt0 < kPhaseTiles ? tend - kt0 : kPhaseTiles);
    // (1) metadata of the lane's row and the DMA of every row's span
    uint64_t bm[kPhaseTiles];
    uint32_t off[kPhaseTiles];
    uint32_t span0 = 0, span1 = 0;
#pragma unroll
    for (int t = 0; t < kPhaseTiles; ++t) { bm[t] = 0ull; off[t] = 0u; }
    if (row_ok) {
      const int64_t tb = row * T + kt0;
#pragma unroll
      for (int t = 0; t < kPhaseTiles; ++t)
        if (t < nt) { bm[t] = a.bitmaps[tb + t]; off[t] = a.offsets[tb + t]; }
      span0 = a.offsets[tb];
      span1 = a.offsets[tb + nt];
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = 2 * b + (lane >> 5);                        // row of the tile this lane copies
      const uint32_t s0 = (uint32_t)__shfl((int)span0, r);
      const uint32_t s1 = (uint32_t)__shfl((int)span1, r);
      const uint32_t ch = (uint32_t)(lane & 31);
      if (8u * ch < s1 - s0) lds_dma16(a.values + s0 + 8u * ch, wl_lds + (uint32_t)b * 1024u);
    }
    // (2) B operands (column-major B: 16 contiguous bytes per lane)
    h8 bop[kPhaseTiles][2][CT];
#pragma unroll
    for (int t = 0; t < kPhaseTiles; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          h8 bv = {};
          const int64_t k = (kt0 + t) * kTile + 32 * blk + 8 * q;
          const int64_t col = 16 * ct + li;
          if (t < nt && col < a.C) {
            if constexpr (BCOL) {
              bv = *reinterpret_cast<const h8*>(a.B + col * a.ldb + k);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) bv[e] = bits_f16(a.B[(k + e) * a.ldb + col]);
            }
          }
          bop[t][blk][ct] = bv;
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the DMA has landed in LDS
    // (3) expand and multiply
    const uint32_t rbase = 512u * (uint32_t)li;
#pragma unroll
    for (int t = 0; t < kPhaseTiles; ++t) {
      if (t >= nt) break;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int byte = 4 * blk + q;
        const uint64_t below = byte == 0 ? 0ull : (bm[t] & ((1ull << (8 * byte)) - 1ull));
        // first value of the chunk; a position past the last set bit reads at most one
        // value beyond the row's span (inside the wave region, or the pad after the last)
        const uint32_t a0 = rbase + 2u * ((off[t] - span0) + (uint32_t)__popcll(below));
        const uint32_t m = (uint32_t)(bm[t] >> (8 * byte)) & 0xFFu;
        const u4 keep = *reinterpret_cast<const u4*>(smem + kLutOff + 16u * m);
        const u2 rk = *reinterpret_cast<const u2*>(smem + kLutOff + 4096u + 8u * m);
        u4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = rk[i >> 1];
          const int sh = 16 * (i & 1);
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(wl + a0 + ((w >> sh) & 0xFFu));
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(wl + a0 + ((w >> (sh + 8)) & 0xFFu));
          pk[i] = (lo | (hi << 16)) & keep[i];
        }
        const h8 av = __builtin_bit_cast(h8, pk);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma16x16x32(av, bop[t][blk][ct], acc[ct]);
        // scheduling fence: expand block by block (hoisting every block's LDS reads would
        // hold all their results in registers)
        asm volatile("" ::: "memory");
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS reads done before the next DMA
  }

  // ---- sum the partial tiles of the waves and store Y -------------------------------------
  __syncthreads();
  f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) red[(w * CT + ct) * 64 + lane] = acc[ct];
  __syncthreads();
  // D layout of the 16x16 MFMA: column l % 16, element r -> row 4 (l / 16) + r
  for (int e = tid; e < 16 * 16 * CT; e += 64 * kBmWaves) {
    const int rr = e / (16 * CT);
    const int cc = e - rr * 16 * CT;
    const int ct = cc >> 4;
    const int ln = ((rr >> 2) << 4) | (cc & 15);
    const float* rp = reinterpret_cast<const float*>(red);
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kBmWaves; ++ww) s += rp[((ww * CT + ct) * 64 + ln) * 4 + (rr & 3)];
    const int64_t orow = row0 + rr;
    if (orow < a.R && cc < a.C) a.Y[orow * a.ldy + cc] = f16_bits(to_f16(s));
  }
}

}  // namespace

hipError_t launch_bitmap_count(const void* A, int64_t R, int64_t K, int64_t lda, uint64_t* bitmaps,
                               uint32_t* offsets, hipStream_t stream) {
  const int64_t T = K / kTile;
  const unsigned g = (unsigned)((R + 3) / 4);
  hipLaunchKernelGGL(k_bitmap_count, dim3(g), dim3(256), 0, stream, (const uint16_t*)A, R, K, lda,
                     bitmaps, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bitmap_scan_rows, dim3(1), dim3(1024), 0, stream, offsets, R, T);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = R * T;
  const unsigned gf = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  hipLaunchKernelGGL(k_bitmap_fix_offsets, dim3(gf), dim3(256), 0, stream, offsets, R, T);
  return hipGetLastError();
}

hipError_t launch_bitmap_values(const void* A, int64_t R, int64_t K, int64_t lda,
                                const uint64_t* bitmaps, const uint32_t* offsets, void* values,
                                hipStream_t stream) {
  const unsigned g = (unsigned)((R + 3) / 4);
  hipLaunchKernelGGL(k_bitmap_values, dim3(g), dim3(256), 0, stream, (const uint16_t*)A, R, K, lda,
                     bitmaps, offsets, (uint16_t*)values);
  return hipGetLastError();
}

hipError_t launch_spmm_bitmap(const uint64_t* bitmaps, const uint32_t* offsets, const void* values,
                              int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb,
                              int b_layout, void* Y, int64_t ldy, hipStream_t stream) {
  BitmapArgs a{};
  a.bitmaps = bitmaps;
  a.offsets = offsets;
  a.values = (const uint16_t*)values;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.R = R; a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.b_col = b_layout == 1;
  const unsigned g = (unsigned)((R + 15) / 16);
  const size_t lds = (size_t)kBitmapLds;   // 69 KiB: two workgroups per CU
  const dim3 blk(64 * kBmWaves);
  auto go = [&](auto kern) -> hipError_t {
    static bool set[2][2] = {};
    bool& done = set[C > 16][b_layout == 1];
    if (!done) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      done = true;
    }
    hipLaunchKernelGGL(kern, dim3(g), blk, lds, stream, a);
    return hipGetLastError();
  };
  if (b_layout == 1) return C > 16 ? go(k_spmm_bitmap<2, true>) : go(k_spmm_bitmap<1, true>);
  return C > 16 ? go(k_spmm_bitmap<2, false>) : go(k_spmm_bitmap<1, false>);
}

}  // namespace snm
