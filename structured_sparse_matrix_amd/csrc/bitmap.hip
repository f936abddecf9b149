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
//   * the product: one workgroup per 16 rows (or per 32, two row groups sharing each B
//     operand, with column-major B when those workgroups fit on the CUs at once), eight
//     waves splitting K. Each wave walks its tiles in phases of 2, software-pipelined: the
//     tiles' bitmaps and offsets are copied into LDS (global->LDS DMA) two phases ahead,
//     their packed values (16-byte aligned spans, because every tile starts at a multiple
//     of 8 values) one phase ahead, into double-buffered per-wave regions whose rows are
//     padded to a 272-byte pitch so that the 16 rows' reads fall on different LDS banks.
//     Each 8-position chunk is expanded through its bitmap byte with LDS reads at the
//     computed ranks and fed to a dense MFMA. Partial sums of the waves are added through
//     LDS.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

#include <type_traits>

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
  // row totals eight at a time, the eight loads independent (one round trip per batch)
  constexpr int U = 8;
  uint32_t s = 0;
  for (int64_t r = r0; r < r1; r += U) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = r + u < r1 ? offsets[(r + u) * T] : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) s += x[u];
  }
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive Hillis-Steele scan of the 1024 parts
    const uint32_t x = tid >= d ? part[tid - d] : 0u;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  uint32_t base = tid > 0 ? part[tid - 1] : 0u;
  for (int64_t r = r0; r < r1; r += U) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = r + u < r1 ? offsets[(r + u) * T] : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (r + u < r1) offsets[(r + u) * T] = base;
      base += x[u];
    }
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

// Values: per 512-position chunk of a row (8 tiles, whose packed values are contiguous in
// the output), lane l (positions base + 8l .. + 7) writes its non-zeros into the wave's LDS
// copy of the chunk at the tile's offset plus their rank in the tile; the copy starts zeroed,
// so each tile's padding is +0; then the chunk leaves as whole 16-byte pieces (2-byte stores
// if the values array is not 16-byte aligned).
__global__ void __launch_bounds__(256) k_bitmap_values(const uint16_t* __restrict__ A, int64_t R,
                                                       int64_t K, int64_t lda,
                                                       const uint64_t* __restrict__ bitmaps,
                                                       const uint32_t* __restrict__ offsets,
                                                       uint16_t* __restrict__ values, int vec) {
  __shared__ __align__(16) uint16_t stage[4][512];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + w;
  if (r >= R) return;   // no barriers in this kernel: each wave works alone
  const int64_t T = K / kTile;
  const int tin = lane >> 3, c = lane & 7;
  uint16_t* const st = stage[w];
  for (int64_t base = 0; base < K; base += 512) {
    const int64_t kt0 = base / kTile;
    const int ntile = (int)(T - kt0 < 8 ? T - kt0 : 8);
    const uint32_t cbase = offsets[r * T + kt0];           // the chunk's first value
    const uint32_t n = offsets[r * T + kt0 + ntile] - cbase;   // its values, padding included (<= 512)
    *reinterpret_cast<u4*>(st + 8 * lane) = u4{0u, 0u, 0u, 0u};
    asm volatile("" ::: "memory");   // the wave's LDS operations stay in program order
    if (tin < ntile) {
      const int64_t kt = kt0 + tin;
      const u4 v = *reinterpret_cast<const u4*>(A + r * lda + base + 8 * lane);
      const uint64_t bm = bitmaps[r * T + kt];
      const uint64_t below = c == 0 ? 0ull : (bm & ((1ull << (8 * c)) - 1ull));
      uint32_t pos = offsets[r * T + kt] - cbase + (uint32_t)__popcll(below);
      const uint32_t m = (uint32_t)(bm >> (8 * c)) & 0xFFu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (m & (1u << e)) {
          const uint32_t word = v[e >> 1];
          st[pos] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xFFFFu));
          ++pos;
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (vec) {
      if ((uint32_t)lane < n / 8)
        __builtin_nontemporal_store(*reinterpret_cast<const u4*>(st + 8 * lane),
                                    reinterpret_cast<u4*>(values + cbase + 8 * lane));
    } else {
      for (uint32_t i = (uint32_t)lane; i < n; i += 64) values[cbase + i] = st[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next zeroing
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


template <int I>
using cint = std::integral_constant<int, I>;

// One workgroup (kBmWaves waves) per RG row groups of 16 rows; wave w takes a contiguous
// 1/kBmWaves of the rows' tiles and walks it in phases of kPT tiles. Lane l = 16q + i works
// on row i of every row group (each B operand feeds RG products); in
// tile t it covers positions 32 blk + 8q + [0, 8), blk = 0, 1 (bitmap byte 4 blk + q) --
// the dense MFMA A operand of k-block (t, blk).
// A phase goes through three steps, each overlapped with the previous phase's work:
//   (1) its metadata -- every row's bitmaps and tile offsets -- is copied by DMA into one of
//       the wave's two metadata buffers (issued two phases ahead);
//   (2) its packed values -- for each row the contiguous, 16-byte aligned span of its
//       tiles' values -- are copied by DMA into one of two value buffers, row i at
//       [272 i, 272 i + 256), with source addresses computed from (1) (one phase ahead),
//       and its B operands are loaded (one phase ahead);
//   (3) each chunk is expanded through its bitmap byte -- the e-th set bit takes the next
//       value of the span -- and multiplied on the matrix core.
// Each phase starts with one wait for everything issued during the previous phase, so the
// latencies of (1) and (2) run under the expansion and products of the phase before.
// The 16-byte pad after each staged row puts row i on banks 4i.. onwards: the expansion
// reads the same ranks in all 16 rows at once, which rows 256 bytes apart would send to one
// bank. Lanes with nothing to copy point their DMA at the first 16 bytes of the values (or
// are masked off past the last row) and land in their row's pad or past its span, which the
// expansion never uses.
constexpr int kBmWaves = 8;
constexpr int kPT = 2;                                   // tiles per phase
constexpr int kRowPitch = kPT * kTile * 2 + 16;          // a row's staged values + pad: 17 slots
constexpr int kSlots = 16 * (kRowPitch / 16);            // 16-byte slots of a value buffer (272)
constexpr int kRGVal = 16 * kRowPitch;                   // a row group's staged values (4352 bytes)
constexpr int kRGMeta = 448;                             // a row group's bitmaps 16 x 16 B, offsets 16 x 12 B
constexpr int kMetaOffs = 256;                           // offsets within a row group's metadata
constexpr int kLutBytes = 256 * 8 + 16 * 8;              // ranks per byte, keep masks per nibble
// Per wave with RG row groups: two metadata buffers, then two value buffers (two phases in
// flight); metadata first, so that a pair read one value before a row stays inside the
// wave's region. The expansion tables follow the waves' regions.
constexpr int bm_wave_bytes(int rg) { return 2 * rg * kRGMeta + 2 * rg * kRGVal; }   // 9600 per group
constexpr int bm_lds_bytes(int rg) { return kBmWaves * bm_wave_bytes(rg) + kLutBytes; }
static_assert(bm_lds_bytes(1) <= 80 * 1024, "one row group: two workgroups per CU");
static_assert(bm_lds_bytes(2) <= 160 * 1024, "two row groups: one workgroup per CU");

template <int CT, bool BCOL, int RG>
__global__ void __launch_bounds__(64 * kBmWaves) __attribute__((amdgpu_waves_per_eu(4 / RG, 4 / RG)))
k_spmm_bitmap(BitmapArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];   // per wave 9600 bytes per row group, then the table
  constexpr int kRG = RG;
  constexpr int kMetaBuf = kRG * kRGMeta;
  constexpr int kValBuf = kRG * kRGVal;
  constexpr int kValBase = 2 * kMetaBuf;
  constexpr int kWaveBytes = bm_wave_bytes(kRG);
  constexpr int kLutOff = kBmWaves * kWaveBytes;
  // Expansion tables: per bitmap byte m, eight byte offsets 2 rank_e (rank_e = set bits of
  // m below e); per bitmap nibble, two dwords of 16-bit keep masks (0xFFFF where the bit is
  // set). Expanding a chunk is then one add and one 2-byte read per position and one AND
  // per pair of positions. (4-byte reads of value pairs would halve the reads, but at
  // 2-byte alignment they stall the LDS: measured twice as slow.)
  for (int m = threadIdx.x; m < 256; m += 64 * kBmWaves) {
    uint32_t rk[2] = {0u, 0u}, r = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rk[e >> 2] |= (2u * r) << (8 * (e & 3));
      r += (m >> e) & 1;
    }
    *reinterpret_cast<u2*>(smem + kLutOff + 8 * m) = u2{rk[0], rk[1]};
    if (m < 16) {
      uint32_t mk[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        mk[i] = (((m >> (2 * i)) & 1) ? 0xFFFFu : 0u) | (((m >> (2 * i + 1)) & 1) ? 0xFFFF0000u : 0u);
      *reinterpret_cast<u2*>(smem + kLutOff + 2048 + 8 * m) = u2{mk[0], mk[1]};
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q = lane >> 4;
  const int li = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * 16 * kRG;
  const int64_t T = a.K / kTile;
  const int64_t RT = a.R * T;                          // bitmaps; offsets hold RT + 1
  const int64_t tw = (T + kBmWaves - 1) / kBmWaves;     // tiles per wave
  const int64_t tbeg = (int64_t)w * tw;
  const int64_t tend = tbeg + tw < T ? tbeg + tw : T;
  const int64_t nph = tend > tbeg ? (tend - tbeg + kPT - 1) / kPT : 0;
  uint8_t* const wl = smem + w * kWaveBytes;
  const uint32_t wl_lds = lds_addr(wl);
  constexpr int kMetaBase = 0;

  // Copy sources are the arrays themselves (wave-uniform bases) plus 32-bit lane byte
  // offsets: R K < 2^31, so every offset into the three arrays fits. The lane parts that do
  // not depend on the phase are computed once here.
  const uint32_t T32 = (uint32_t)T, RT32 = (uint32_t)RT;
  uint32_t bm_lane[kRG], of_lane[kRG];
  const int orr = lane < 48 ? lane / 3 : 0;
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const int64_t rbm = row0 + 16 * rg + (lane >> 2) < a.R ? row0 + 16 * rg + (lane >> 2) : a.R - 1;
    bm_lane[rg] = (uint32_t)(rbm * T) * 8u + (uint32_t)(lane & 1) * 4u;
    const int64_t rof = row0 + 16 * rg + orr < a.R ? row0 + 16 * rg + orr : a.R - 1;
    of_lane[rg] = (uint32_t)(rof * T) + (uint32_t)(lane < 48 ? lane - 3 * orr : 0);
  }
  const uint32_t bm_t = (uint32_t)((lane >> 1) & 1);
  // a matrix without non-zeros has no values to copy (and its values pointer may be NULL);
  // otherwise the first 16 bytes of values are a readable target for idle lanes. A wave
  // without tiles reads nothing (with K = 0 the arrays may all be NULL).
  const bool any_values = nph > 0 && a.offsets[RT] != 0u;

  // (1) metadata of phase p into metadata buffer mb: lane l copies bitmap word l % 2 of
  // tile (l / 2) % 2 of row l / 4, and (l < 48) offset entry l % 3 of row l / 3; rows past
  // R repeat row R - 1, tiles past the row's end repeat its last tile
  auto issue_meta = [&](int64_t p, int mb) {
    const uint32_t kt0 = (uint32_t)(tbeg + p * kPT);
    const uint32_t base = wl_lds + (uint32_t)(kMetaBase + mb * kMetaBuf);
    uint32_t t = kt0 + bm_t;
    t = t < T32 ? t : T32 - 1;
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      dma_s<4>(a.bitmaps, bm_lane[rg] + 8u * t, base + (uint32_t)(rg * kRGMeta));
      uint32_t idx = of_lane[rg] + kt0;
      idx = idx < RT32 ? idx : RT32;
      if (lane < 48) dma_s<4>(a.offsets, 4u * idx, base + (uint32_t)(rg * kRGMeta + kMetaOffs));
    }
  };
  // (2) values of phase p (its metadata in buffer mb) into value buffer vb: DMA b fills the
  // 16-byte slots 64 b .. 64 b + 63 of the buffer, slot = 17 r + c being chunk c of row r
  // (c = 16: the row's pad); the last DMA covers slots 256 .. 271 with lanes 0 .. 15
  auto issue_values = [&](int64_t p, int mb, int vb) {
    if (!any_values) return;
    const int64_t kt0 = tbeg + p * kPT;
    const int nt = (int)(tend - kt0 < kPT ? tend - kt0 : kPT);
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
    const uint8_t* offs = wl + kMetaBase + mb * kMetaBuf + rg * kRGMeta + kMetaOffs;
#pragma unroll
    for (int b = 0; b < (kSlots + 63) / 64; ++b) {
      const int slot = 64 * b + lane;
      const int r = slot / 17;
      const uint32_t ch = (uint32_t)(slot - 17 * r);
      const int rc = r < 16 ? r : 15;
      const uint32_t s0 = *reinterpret_cast<const uint32_t*>(offs + 12 * rc);
      const uint32_t s1 = *reinterpret_cast<const uint32_t*>(offs + 12 * rc + 4 * nt);
      const bool live = r < 16 && row0 + 16 * rg + r < a.R && 8u * ch < s1 - s0;   // ch = 16 is never live
      const uint32_t dst = wl_lds + (uint32_t)(kValBase + vb * kValBuf + rg * kRGVal + b * 1024);
      if (64 * b + 64 <= kSlots || slot < kSlots) dma_s<16>(a.values, live ? 2u * (s0 + 8u * ch) : 0u, dst);
    }
    }
  };
  // B operands of phase p. With one column tile and column-major B (16 contiguous bytes per
  // lane) they are loaded one phase ahead into a second register set; otherwise (two column
  // tiles, or row-major B's eight 2-byte loads per operand: too many registers to hold
  // twice) at the start of their own phase.
  constexpr bool kAheadB = BCOL && CT == 1;
  constexpr int NB = kAheadB ? 2 : 1;
  h8 bop[NB][kPT][2][CT];
  // column-major B: each lane's first operand of the wave's first tile; a phase, a tile and a
  // 32-position block are then uniform or constant steps from it
  const uint16_t* bcol_base[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    // columns past C are clamped to C - 1: they feed only output columns that are not stored
    const int64_t col = 16 * ct + li < a.C ? 16 * ct + li : a.C - 1;
    bcol_base[ct] = a.B + col * a.ldb + tbeg * kTile + 8 * q;
  }
  auto load_b = [&](int64_t p, auto par_c) {
    constexpr int P = decltype(par_c)::value;
    const int64_t kt0 = tbeg + p * kPT;
    const int nt = (int)(tend - kt0 < kPT ? tend - kt0 : kPT);
#pragma unroll
    for (int t = 0; t < kPT; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          h8 bv = {};
          const int64_t col = 16 * ct + li < a.C ? 16 * ct + li : a.C - 1;
          if (t < nt) {   // uniform: every lane loads (past C from column C - 1)
            if constexpr (BCOL) {
              bv = *reinterpret_cast<const h8*>(bcol_base[ct] + p * (kPT * kTile) + t * kTile + 32 * blk);
            } else {
              // the tile's rows from a uniform base with 32-bit lane offsets (B's row
              // stride is below 2^25 elements): one address register per load
              const uint8_t* bt = reinterpret_cast<const uint8_t*>(a.B + (kt0 + t) * kTile * a.ldb);
              const uint32_t o0 = (uint32_t)(((32 * blk + 8 * q) * a.ldb + col) * 2);
              const uint32_t ostep = (uint32_t)(a.ldb * 2);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                bv[e] = bits_f16(*reinterpret_cast<const uint16_t*>(bt + (o0 + (uint32_t)e * ostep)));
            }
          }
          bop[P][t][blk][ct] = bv;
        }
  };

  f4 acc[kRG][CT];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rg][ct] = f4{0.f, 0.f, 0.f, 0.f};

  auto phase = [&](int64_t p, auto par_c) {
    constexpr int P = decltype(par_c)::value;   // p % 2: its value and metadata buffers
    constexpr int PB = kAheadB ? P : 0;         // its B register set
    wait_vmcnt<0>();   // this phase's values and B, the next phase's metadata
    // the B operands have arrived: any wait the compiler adds for them goes here, where
    // nothing is outstanding
#pragma unroll
    for (int t = 0; t < kPT; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) asm volatile("" : "+v"(bop[PB][t][blk][ct]));
    const uint8_t* mbuf = wl + kMetaBase + P * kMetaBuf;
    uint64_t bm[kRG][kPT];
    uint32_t off[kRG][kPT];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
    for (int t = 0; t < kPT; ++t) {
      bm[rg][t] = *reinterpret_cast<const uint64_t*>(mbuf + rg * kRGMeta + 16 * li + 8 * t);
      off[rg][t] = *reinterpret_cast<const uint32_t*>(mbuf + rg * kRGMeta + kMetaOffs + 12 * li + 4 * t);
    }
    if (p + 1 < nph) {
      if constexpr (kAheadB) load_b(p + 1, cint<P ^ 1>{});
      issue_values(p + 1, P ^ 1, P ^ 1);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // metadata reads done: refill buffer P
    if (p + 2 < nph) issue_meta(p + 2, P);
    // (3) expand and multiply
    const int64_t kt0 = tbeg + p * kPT;
    const int nt = (int)(tend - kt0 < kPT ? tend - kt0 : kPT);

#pragma unroll
    for (int t = 0; t < kPT; ++t) {
      if (t >= nt) break;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
       for (int rg = 0; rg < kRG; ++rg) {
        const uint8_t* rowp = wl + kValBase + P * kValBuf + rg * kRGVal + kRowPitch * li;   // staged row li
        const uint32_t span0 = off[rg][0];
        const int byte = 4 * blk + q;
        const uint64_t below = byte == 0 ? 0ull : (bm[rg][t] & ((1ull << (8 * byte)) - 1ull));
        // the chunk's first value in the staged row; a position past the last set bit reads
        // at most one value beyond the row's span (byte 256: the row's pad)
        const uint8_t* cb = rowp + 2u * ((off[rg][t] - span0) + (uint32_t)__popcll(below));
        const uint32_t m = (uint32_t)(bm[rg][t] >> (8 * byte)) & 0xFFu;
        const u2 klo = *reinterpret_cast<const u2*>(smem + kLutOff + 2048u + 8u * (m & 15u));
        const u2 khi = *reinterpret_cast<const u2*>(smem + kLutOff + 2048u + 8u * (m >> 4));
        const u4 keep = {klo[0], klo[1], khi[0], khi[1]};
        const u2 rk = *reinterpret_cast<const u2*>(smem + kLutOff + 8u * m);
        u4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t rw = rk[i >> 1];
          const int sh = 16 * (i & 1);
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(cb + ((rw >> sh) & 0xFFu));
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(cb + ((rw >> (sh + 8)) & 0xFFu));
          pk[i] = (lo | (hi << 16)) & keep[i];
        }
        const h8 av = __builtin_bit_cast(h8, pk);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rg][ct] = mfma16x16x32(av, bop[PB][t][blk][ct], acc[rg][ct]);
        // scheduling fence: expand block by block (hoisting every block's LDS reads would
        // hold all their results in registers)
        asm volatile("" ::: "memory");
       }
      }
    }
    // one register set (kAheadB off): the next phase's B operands are requested once this
    // phase's products have been issued, and arrive under the wait that opens the next phase
    if constexpr (!kAheadB)
      if (p + 1 < nph) load_b(p + 1, cint<0>{});
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // value reads done: buffer P is free
  };

  if (nph > 0) {
    issue_meta(0, 0);
    if (nph > 1) issue_meta(1, 1);
    wait_vmcnt<0>();
    load_b(0, cint<0>{});
    issue_values(0, 0, 0);
  }
  for (int64_t p = 0; p < nph; p += 2) {
    phase(p, cint<0>{});
    if (p + 1 < nph) phase(p + 1, cint<1>{});
  }
  wait_vmcnt<0>();   // no copy in flight when the buffers are reused below

  // ---- sum the partial tiles of the waves and store Y -------------------------------------
  __syncthreads();
  f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) red[((w * kRG + rg) * CT + ct) * 64 + lane] = acc[rg][ct];
  __syncthreads();
  // D layout of the 16x16 MFMA: column l % 16, element r -> row 4 (l / 16) + r
  for (int e = tid; e < 16 * kRG * 16 * CT; e += 64 * kBmWaves) {
    const int rr = e / (16 * CT);
    const int cc = e - rr * 16 * CT;
    const int ct = cc >> 4;
    const int rg = rr >> 4;
    const int rl = rr & 15;
    const int ln = ((rl >> 2) << 4) | (cc & 15);
    const float* rp = reinterpret_cast<const float*>(red);
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kBmWaves; ++ww) s += rp[(((ww * kRG + rg) * CT + ct) * 64 + ln) * 4 + (rl & 3)];
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
  const int vec = ((uintptr_t)values & 15u) == 0;
  hipLaunchKernelGGL(k_bitmap_values, dim3(g), dim3(256), 0, stream, (const uint16_t*)A, R, K, lda,
                     bitmaps, offsets, (uint16_t*)values, vec);
  return hipGetLastError();
}

// The current device's compute-unit count, looked up once per device.
static hipError_t device_cu_count(int* cus) {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) return e;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
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
  // Two row groups per wave (32 rows per workgroup) apply every B operand to twice the rows
  // but leave room for one workgroup per CU (152 KiB of LDS). They are taken with
  // column-major B when the 32-row workgroups fit in one pass over the CUs; past that the
  // second pass costs more than the B loads saved. (Row-major B's two-column-tile form would
  // spill with two row groups.)
  int cus = 0;
  if (hipError_t e = device_cu_count(&cus)) return e;
  const bool two = b_layout == 1 && (R + 31) / 32 <= (int64_t)cus;
  const int rg = two ? 2 : 1;
  const unsigned g = (unsigned)((R + 16 * rg - 1) / (16 * rg));
  const size_t lds = (size_t)bm_lds_bytes(rg);   // 77 KiB (two workgroups per CU) or 152 KiB
  const dim3 blk(64 * kBmWaves);
  auto go = [&](auto kern) -> hipError_t {
    static std::atomic<uint64_t> lds_set[2][2][2] = {};
    if (hipError_t e = ensure_lds_limit(lds_set[two][C > 16][b_layout == 1], (const void*)kern, (int)lds)) return e;
    hipLaunchKernelGGL(kern, dim3(g), blk, lds, stream, a);
    return hipGetLastError();
  };
  if (two) return C > 16 ? go(k_spmm_bitmap<2, true, 2>) : go(k_spmm_bitmap<1, true, 2>);
  if (b_layout == 1) return C > 16 ? go(k_spmm_bitmap<2, true, 1>) : go(k_spmm_bitmap<1, true, 1>);
  return C > 16 ? go(k_spmm_bitmap<2, false, 1>) : go(k_spmm_bitmap<1, false, 1>);
}

}  // namespace snm
