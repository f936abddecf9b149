// Structured-sparse x dense products with wide outputs (C > 32): the compute-heavy regime
// of V:2:M ("VENOM ...", SC'23, Sec. 4 and Fig. 4: per block of V rows, the K/M*4 rows
// of B named by column-loc are gathered and the product becomes 2:4 over K' = 4K/M) and of
// 2:4 with many columns ("2:4 sparsity on sparse tensor cores", lecture notes: "How the
// tensor core uses it"), including the batched P.V product of dynamic 2:4 attention.
//
// Design for MI355X (gfx950), from measurements on the device:
//   * math: v_smfmac_f32_32x32x32_f16 -- the 32x32 form sustains about 5% more than the
//     16x16x64 form and needs half the operand bytes per flop.
//   * reuse: a gathered B row is shared only by the V rows of its V-block, so the L2->CU
//     stream of B is 1/BM bytes per flop whatever else is done; the workgroup tile is
//     therefore as tall as the V-block allows (BM = 128 or 64) and as wide as the register
//     file allows (BN up to 256, 128 fp32 accumulators per lane).
//   * feeding: an LDS ring of NST stages is filled by the global->LDS DMA path
//     (global_load_lds_dwordx4 and the 2-byte form) NST-1 stages ahead, with no register
//     staging; each wave waits only for its own DMA of the stage about to be read
//     (s_waitcnt vmcnt) and one barrier per stage publishes it and frees the oldest slot.
//   * every LDS destination of a DMA instruction is 64 consecutive lanes x 16 bytes, so
//     the B tile's bank swizzle is applied on the source side (wide_layout.hpp), the A
//     operand blocks are stored exactly in the instruction's lane order and read with one
//     ds_read_b128, and B operands are read with ds_read_b64_tr_b16.
//   * workgroups are spread over the 8 XCDs round-robin by the hardware; tiles are
//     renumbered so that the workgroups resident on one XCD share a column strip of B
//     (V:2:M: all V-blocks of one strip) and hit in that XCD's L2.
//   * ragged edges: DMA sources are clamped into the operands (rows >= R, columns >= C
//     and positions >= K' read valid memory whose products are never stored or are
//     multiplied by zeroed operands), so no lane ever skips a DMA and every wave's
//     vmcnt bookkeeping stays exact.
#include "elem.hpp"
#include "lds_dma.hpp"
#include "launch.hpp"
#include "variant.hpp"
#include "wide_layout.hpp"

#include <type_traits>

namespace snm {
namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

struct WideArgs {
  const uint16_t* values;   // fp16 bits, R x Kc/2 per batch entry
  const uint8_t* meta;      // R x Kc/8 bytes per batch entry
  const uint16_t* B;        // fp16 bits, row-major, ldb (a multiple of 8)
  uint16_t* Y;              // fp16 bits, R x C (ldy)
  const uint8_t* colloc;    // V:2:M: (R/V) x Kc bytes (Kc/4 groups x 4 column indices)
  const float* rowmax;      // softmax mode: fp32 per row (R per batch entry, stride_rowmax)
  int64_t R, Kc, C, ldb, ldy;
  int64_t stride_values, stride_meta, stride_B, stride_Y, stride_rowmax, batch;
  int64_t n_row_tiles, n_tiles;   // tiles per batch entry = n_row_tiles * column tiles
  int V, M;
  int xcd_remap;                  // total workgroups are a multiple of 8
  int y_vec;                      // Y rows start 16-byte aligned (16-byte output stores)
  int a_tiled;                    // V:2:M values and m-indices in the row-group interleaved
                                  // storage (per 32 rows: 16-byte chunk c of every row, then
                                  // chunk c + 1; 2-byte words likewise)
};

template <int WM, int WN, int TM, int TN, int KSTEPS, int NST, bool GATHER>
struct WideCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * TM * WM;
  static constexpr int BN = 32 * TN * WN;
  static constexpr int KS = 32 * KSTEPS;            // compressed positions per stage
  static constexpr int kBBytes = KS * BN * 2;
  static constexpr int kBlocks = (BM / 32) * KSTEPS; // A blocks (1 KiB) = metadata blocks (256 B)
  static constexpr int kAOff = kBBytes;
  static constexpr int kMOff = kBBytes + kBlocks * 1024;
  static constexpr int kStage = kMOff + kBlocks * 256;
  static constexpr int kRing = NST * kStage;
  // output tile staged as fp16 rows; the 64-byte pad makes rows r and r + 4 (written by one
  // transposing store instruction) fall on different banks
  static constexpr int kOutPitch = 2 * BN + 64;
  static constexpr int kOut = BM * kOutPitch;
  static constexpr int nB = kBBytes / 1024 / kWaves;   // DMA instructions per wave per stage
  static constexpr int nA = kBlocks / kWaves;
  static constexpr int kDma = nB + 2 * nA;
  static_assert(kBBytes % (1024 * kWaves) == 0, "B stage must split into whole DMA rows per wave");
  static_assert(kBlocks % kWaves == 0, "A blocks must split evenly over the waves");
  static_assert(NST >= 2, "the ring needs a stage in flight");
  static_assert(kDma * (NST - 2) < 64, "vmcnt holds at most 63 outstanding operations");
};


// ds_read_b64_tr_b16 (lane layout as lds_read_tr16) addressed from the dynamic LDS array
// itself, so that constant parts of the offset fold into the instruction.
__device__ __forceinline__ h4 tr16_at(uint8_t* smem, uint32_t byte_off) {
  typedef __fp16 fp4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) fp4 lds_fp4;
  lds_fp4* p = (lds_fp4*)((lds_u8*)smem + byte_off);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
}

template <int I>
using cint = std::integral_constant<int, I>;
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(cint<I>{});
    static_for<I + 1, N>(f);
  }
}

// Two workgroups per CU (two waves per SIMD): one workgroup's barrier and LDS latency hide
// behind the other's matrix-core work; this caps a lane at 256 registers.
//
// Per step (32 positions) a wave issues TM*TN sparse-MFMAs and almost no other vector
// work: DMA sources are a per-stage scalar base plus per-lane offsets fixed at start-up
// (only a gathered B row needs one multiply-add), the stage loop is unrolled by the ring
// depth so every LDS read is a lane-constant register plus an immediate, and all clamping
// of ragged edges is confined to the last, partial stage.
//
// SMAX (2:4 only): the stored values are attention scores and the product applies the
// softmax over each row's kept entries on the fly. Every A operand value v becomes
// fp16(exp(v - rowmax)) in registers before it enters the matrix core, the lane keeps an
// fp32 sum of exactly those fp16 numbers for its row, and the epilogue divides each
// output row by its sum. With WN == 1 no two waves exponentiate the same operand.
// PIPE: issue each step's products one step late (two operand buffers), so that the
// operand reads of the next step -- across a stage barrier too -- overlap the matrix core;
// off where the second buffer does not fit in the register file.
// BF: bf16 values, B and Y (v_smfmac_f32_32x32x32_bf16; same lane layout) instead of fp16.
template <int WM, int WN, int TM, int TN, int KSTEPS, int NST, bool GATHER, bool SMAX, bool PIPE, bool BF>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2)))
k_spmm_wide(WideArgs a) {
  static_assert(!(SMAX && GATHER), "the softmax mode is defined for 2:4 scores only");
  using Cfg = WideCfg<WM, WN, TM, TN, KSTEPS, NST, GATHER>;
  using E = Elem<BF>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, KS = Cfg::KS;
  constexpr int nB = Cfg::nB, nA = Cfg::nA;
  constexpr int kRowsPerDma = 1024 / (2 * BN);   // B tile rows one DMA instruction fills
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;
  const int wm = wave / WN;

  // ---- tile of this workgroup (XCD-aware numbering) ------------------------------------
  int64_t L = blockIdx.x;
  if (a.xcd_remap) L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t bt = L / a.n_tiles;
  const int64_t rem = L - bt * a.n_tiles;
  const int64_t ct = rem / a.n_row_tiles;
  const int64_t rt = rem - ct * a.n_row_tiles;
  const int64_t row0 = rt * BM;
  const int64_t col0 = ct * BN;

  const uint8_t* __restrict__ vals = reinterpret_cast<const uint8_t*>(a.values + bt * a.stride_values);
  const uint8_t* __restrict__ meta = a.meta + bt * a.stride_meta;
  const uint16_t* __restrict__ Bm = a.B + bt * a.stride_B;
  uint16_t* __restrict__ Y = a.Y + bt * a.stride_Y;
  const int64_t Kc = a.Kc;
  const int64_t nst = (Kc + KS - 1) / KS;
  const int64_t nfull = Kc / KS;   // stages whose sources need no clamping
  const int64_t mrow = Kc >> 3;    // metadata bytes per row; a values row is Kc bytes
  const int64_t ldb2 = a.ldb * 2;

  if constexpr (GATHER) {   // this V-block's column-loc bytes after the ring, zero-padded
    const uint8_t* cl = a.colloc + (row0 / a.V) * Kc;
    for (int64_t i = (int64_t)tid * 16; i < Kc + 2 * KS; i += Cfg::kThreads * 16)
      *reinterpret_cast<u4*>(smem + Cfg::kRing + i) = i < Kc ? *reinterpret_cast<const u4*>(cl + i) : u4{0u, 0u, 0u, 0u};
    __syncthreads();
  }

  // ---- per-lane DMA source offsets (stage-invariant) -------------------------------------
  const uint32_t o0 = (uint32_t)(wave * nB * 1024 + lane * 16);
  const int bx0 = wide::b_row_of<BN>(o0);   // chunk j covers tile row bx0 + j*kRowsPerDma
  uint32_t boff[nB];
#pragma unroll
  for (int j = 0; j < nB; ++j) {
    const uint32_t o = o0 + (uint32_t)(j * 1024);
    const int x = wide::b_row_of<BN>(o);
    int64_t c = col0 + wide::b_col_of<BN>(o);
    c = c < a.C ? c : 0;
    boff[j] = GATHER ? (uint32_t)(((int64_t)(x >> 2) * a.M * a.ldb + c) * 2) : (uint32_t)(((int64_t)x * a.ldb + c) * 2);
  }
  // A chunk (16 bytes = 16 positions) and index word sources. Canonical storage: row r's
  // chunk c at r Kc + 16 c, word w at r mrow + 2 w. Row-group interleaved storage (row0 is
  // a multiple of 32): chunk c of row r at 32 Kc (r / 32) + 512 c + 16 (r % 32), word w at
  // 32 mrow (r / 32) + 64 w + 2 (r % 32), so a stage's copies read whole lines.
  uint32_t aoff[nA], moff[nA];
#pragma unroll
  for (int j = 0; j < nA; ++j) {
    const int bi = wave * nA + j;
    int64_t r = wide::a_dma_row<KS>(bi, lane);
    r = row0 + r < a.R ? r : a.R - 1 - row0;
    const int64_t ch = wide::a_dma_chunk<KS>(bi, lane);
    aoff[j] = a.a_tiled ? (uint32_t)((r >> 5) * 32 * Kc + ch * 512 + (r & 31) * 16) : (uint32_t)(r * Kc + ch * 16);
    int64_t rm = wide::m_dma_row<KS>(bi, lane);
    rm = row0 + rm < a.R ? rm : a.R - 1 - row0;
    const int64_t wd = wide::m_dma_word<KS>(lane);
    moff[j] = a.a_tiled ? (uint32_t)((rm >> 5) * 32 * mrow + wd * 64 + (rm & 31) * 2) : (uint32_t)(rm * mrow + wd * 2);
  }
  // bytes between consecutive stages' A chunks and index words (the same run of rows)
  const int64_t a_stage = a.a_tiled ? (int64_t)KS * 32 : (int64_t)KS;
  const int64_t m_stage = a.a_tiled ? (int64_t)KS * 4 : (int64_t)(KS / 8);

  // column-loc bytes of the B rows a stage gathers: read from LDS one stage ahead of the
  // DMA that needs them, so the issue path never waits on LDS
  int gcl[nB];
  auto fetch_colloc = [&](int64_t s) {
    if (GATHER && s < nst) {
#pragma unroll
      for (int j = 0; j < nB; ++j) gcl[j] = smem[Cfg::kRing + s * KS + bx0 + j * kRowsPerDma];
    }
  };
  auto issue = [&](int64_t s, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t sb = lds0 + (uint32_t)(slot * Cfg::kStage);
    if (s < nfull) {
      const uint16_t* bs = Bm + (GATHER ? s * (KS / 4) * a.M * a.ldb : s * KS * a.ldb);
#pragma unroll
      for (int j = 0; j < nB; ++j) {
        const uint32_t v = GATHER ? boff[j] + (uint32_t)gcl[j] * (uint32_t)ldb2 : boff[j];
        dma_s<16>(bs, v, sb + (uint32_t)((wave * nB + j) * 1024));
      }
      const uint8_t* vs = vals + row0 * Kc + s * a_stage;
      const uint8_t* ms = meta + row0 * mrow + s * m_stage;
#pragma unroll
      for (int j = 0; j < nA; ++j) {
        dma_s<16>(vs, aoff[j], sb + (uint32_t)(Cfg::kAOff + (wave * nA + j) * 1024));
        dma_s<2>(ms, moff[j], sb + (uint32_t)(Cfg::kMOff + (wave * nA + j) * 256));
      }
    } else {
      // last, partial stage: every source clamped into the operands
#pragma unroll
      for (int j = 0; j < nB; ++j) {
        const uint32_t o = o0 + (uint32_t)(j * 1024);
        int64_t kg = s * KS + wide::b_row_of<BN>(o);
        kg = kg < Kc ? kg : Kc - 1;
        int64_t c = col0 + wide::b_col_of<BN>(o);
        c = c < a.C ? c : 0;
        int64_t brow = kg;
        if constexpr (GATHER) {
          const int cl = smem[Cfg::kRing + kg];
          brow = (kg >> 2) * a.M + (cl < a.M ? cl : a.M - 1);   // column-loc entries are < M by contract
        }
        dma_v<16>(Bm + brow * a.ldb + c, sb + (uint32_t)((wave * nB + j) * 1024));
      }
#pragma unroll
      for (int j = 0; j < nA; ++j) {
        const int bi = wave * nA + j;
        int64_t r = row0 + wide::a_dma_row<KS>(bi, lane);
        r = r < a.R ? r : a.R - 1;
        int64_t p = s * KS + wide::a_dma_chunk<KS>(bi, lane) * 16;   // first position of the chunk
        p = p < Kc ? p : Kc - 16;
        const int64_t va = a.a_tiled ? (r >> 5) * 32 * Kc + (p >> 4) * 512 + (r & 31) * 16 : r * Kc + p;
        dma_v<16>(vals + va, sb + (uint32_t)(Cfg::kAOff + bi * 1024));
        int64_t rm = row0 + wide::m_dma_row<KS>(bi, lane);
        rm = rm < a.R ? rm : a.R - 1;
        int64_t wd = s * (KS / 16) + wide::m_dma_word<KS>(lane);   // index word of the row
        wd = wd < Kc / 16 ? wd : Kc / 16 - 1;
        const int64_t ma = a.a_tiled ? (rm >> 5) * 32 * mrow + wd * 64 + (rm & 31) * 2 : rm * mrow + wd * 2;
        dma_v<2>(meta + ma, sb + (uint32_t)(Cfg::kMOff + bi * 256));
      }
    }
  };

  f16v acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.f;

  // softmax mode: row maximum in log2 units and the running sum of this lane's share of
  // its row (lanes l and l + 32 hold the two halves of row l of each 32-row tile)
  constexpr float kLog2e = 1.4426950408889634f;
  float mx2[TM], rsum[TM];
  if constexpr (SMAX) {
    const float* __restrict__ rmx = a.rowmax + bt * a.stride_rowmax;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      int64_t r = row0 + (wm * TM + tm) * 32 + (lane & 31);
      r = r < a.R ? r : a.R - 1;
      mx2[tm] = rmx[r] * kLog2e;
      rsum[tm] = 0.f;
    }
  }

  // lane-constant LDS offsets of the operand reads: A operand of tile tm, step ks = row
  // (wm*TM + tm)*32 + lane%32, chunk 2 ks + lane/32; its index word likewise. The layout
  // makes tile tm + 1 a constant offset away (32 KS bytes of A, 8 KS of metadata), and the
  // index word of step ks + 1 too (8 bytes), so only the first tile's offsets are registers
  // and the rest fold into the read instructions (checked on the host with the layout).
  uint32_t a_lds[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    a_lds[ks] = wide::a_offset<KS>(wm * TM * 32 + (lane & 31), 2 * ks + (lane >> 5));
  const uint32_t m_lds = wide::m_offset<KS>(wm * TM * 32 + (lane & 31), lane >> 5);
  constexpr uint32_t kATile = wide::a_tile_delta<KS>();
  constexpr uint32_t kMTile = wide::m_tile_delta<KS>();
  // transpose reads: rows x, x + 4, x + 16, x + 20 of a step share the cell swizzle, so
  // they are one register plus constant row offsets
  uint32_t tr_lds[TN];
  {
    const int x = 8 * (lane >> 5) + ((lane & 15) >> 2);                       // row in a step
    const int cb = wn * TN * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);    // column
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) tr_lds[tn] = wide::b_offset<BN>(x, cb + tn * 32);
  }

  // Operands of one 32-position step, read from the ring; the step's products are issued
  // one step later, so that the reads of step t + 1 (across a stage barrier too) are in
  // flight while the matrix core works on step t.
  struct Frag {
    h8 af[TM];
    uint32_t ix[TM];
    h16 bf[TN];
  };
  auto read_frag = [&](Frag& f, uint32_t sb, int ks) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      f.af[tm] = *reinterpret_cast<const h8*>(smem + a_lds[ks] + (sb + Cfg::kAOff + tm * kATile));
      f.ix[tm] = *reinterpret_cast<const uint32_t*>(smem + m_lds + (sb + Cfg::kMOff + tm * kMTile + ks * 8));
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const uint32_t so = sb + (uint32_t)(ks * 64 * BN);   // 32 rows of 2*BN bytes
      const h4 b0 = tr16_at(smem, tr_lds[tn] + so);
      const h4 b1 = tr16_at(smem, tr_lds[tn] + (so + 4 * 2 * BN));
      const h4 b2 = tr16_at(smem, tr_lds[tn] + (so + 16 * 2 * BN));
      const h4 b3 = tr16_at(smem, tr_lds[tn] + (so + 20 * 2 * BN));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f.bf[tn][e] = b0[e];
        f.bf[tn][4 + e] = b1[e];
        f.bf[tn][8 + e] = b2[e];
        f.bf[tn][12 + e] = b3[e];
      }
    }
  };
  auto mma = [&](Frag& f) {
    if constexpr (SMAX) {
      // scores -> 16-bit probabilities (packed pairs), and the fp32 sum of exactly the
      // 16-bit numbers the matrix core multiplies
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        u4 w = __builtin_bit_cast(u4, f.af[tm]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f2 x;
          x[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(E::lo(w[t]), kLog2e, -mx2[tm]));
          x[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(E::hi(w[t]), kLog2e, -mx2[tm]));
          w[t] = E::pack2(x);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) rsum[tm] = E::sum2(w[t], rsum[tm]);
        f.af[tm] = __builtin_bit_cast(h8, w);
      }
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = E::smfmac32(f.af[tm], f.bf[tn], acc[tm][tn], f.ix[tm]);
  };

  // The last stage of a ragged K' (a multiple of 16 positions) holds clamped DMA sources
  // past K': once it has landed, its A values there become 0 (-inf in the softmax mode,
  // whose exponential is 0) and its B rows there become 0, so that every stage runs the
  // same unchecked step loop and the extra positions contribute exact zeros.
  const int krem = (int)(Kc - nfull * KS);   // valid positions of the last stage, or 0
  auto clean_tail = [&](uint32_t sb) {
    constexpr int kChunks = KS / 16;
    const int c0 = krem / 16;
    const uint32_t fill = SMAX ? E::kNegInf2 : 0u;
    for (int e = tid; e < BM * kChunks; e += Cfg::kThreads) {
      const int R = e / kChunks;
      const int c = e - R * kChunks;
      if (c >= c0)
        *reinterpret_cast<u4*>(smem + sb + Cfg::kAOff + wide::a_offset<KS>(R, c)) = u4{fill, fill, fill, fill};
    }
    for (int e = krem * (BN / 8) + tid; e < KS * (BN / 8); e += Cfg::kThreads)   // rows >= krem
      *reinterpret_cast<u4*>(smem + sb + (uint32_t)e * 16u) = u4{0u, 0u, 0u, 0u};
  };

  // ---- the ring: stage s lives in slot s % NST. The loop is unrolled by NST (by 2 NST if
  // a pass of NST stages has an odd number of steps) so that slots and the two operand
  // buffers (global step g uses fr[g % 2]) are compile-time constants. ---------------------
  constexpr int UNR = PIPE && (NST * KSTEPS) % 2 ? 2 * NST : NST;
  Frag fr[2];
  bool pending = false;   // the previous step's operands are waiting for their products
  static_for<0, NST - 1>([&](auto p) {
    constexpr int P = decltype(p)::value;
    if (P < nst) {
      fetch_colloc(P);
      issue(P, cint<P>{});
    }
  });
  fetch_colloc(NST - 1);
  for (int64_t s0 = 0; s0 < nst; s0 += UNR) {
    static_for<0, UNR>([&](auto u) {
      constexpr int U = decltype(u)::value;
      constexpr int SLOT = U % NST;
      constexpr uint32_t sb = (uint32_t)(SLOT * Cfg::kStage);
      const int64_t s = s0 + U;
      if (s < nst) {
        // wait for this wave's DMA of stage s; the barrier publishes every wave's and
        // retires all reads of slot (s - 1) % NST, which is refilled with stage s + NST - 1
        if (s + NST - 2 < nst) wait_vmcnt<Cfg::kDma * (NST - 2)>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (s + NST - 1 < nst) {
          issue(s + NST - 1, cint<(SLOT + NST - 1) % NST>{});
          fetch_colloc(s + NST);
        }
        if (s == nfull) {   // only a ragged last stage gets here
          clean_tail(sb);
          lds_barrier();
        }
        static_for<0, KSTEPS>([&](auto k) {
          constexpr int KK = decltype(k)::value;
          if constexpr (PIPE) {
            constexpr int P = (U * KSTEPS + KK) % 2;
            read_frag(fr[P], sb, KK);
            if (pending) mma(fr[P ^ 1]);
            pending = true;
          } else {
            read_frag(fr[0], sb, KK);
            mma(fr[0]);
          }
        });
      }
    });
  }
  if (pending) {   // the last step: g = nst * KSTEPS - 1
    if ((nst * KSTEPS) & 1) mma(fr[0]);
    else mma(fr[1]);
  }

  // ---- epilogue: fp32 -> fp16 or bf16 (RNE), staged through LDS so that output rows leave as
  // whole 128-byte lines of 16-byte stores ([VENOM] Sec. 4.2, Fig. 8: wide output stores)
  __syncthreads();   // every wave is done with the ring (and the column-loc bytes)
  uint8_t* const otile = smem;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    // softmax mode: 1 / row sum for each of the lane's 16 output rows (row 8(i/4) + 4(l/32)
    // + i%4 of the tile, whose sum lanes r and r + 32 share)
    float inv[16];
    if constexpr (SMAX) {
      const float tot = rsum[tm] + __shfl_xor(rsum[tm], 32);
      const float rinv = 1.0f / tot;
#pragma unroll
      for (int i = 0; i < 16; ++i) inv[i] = __shfl(rinv, 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3));
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int ct = (wn * TN + tn) * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rt = (wm * TM + tm) * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float y = SMAX ? acc[tm][tn][i] * inv[i] : acc[tm][tn][i];
        *reinterpret_cast<uint16_t*>(otile + rt * Cfg::kOutPitch + ct * 2) = E::narrow(y);
      }
      // scheduling fence: convert and store tile by tile (hoisting every conversion above
      // the first store would need a second register copy of the accumulators)
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();
  constexpr int kChunksPerRow = BN / 8;   // 16-byte chunks of a tile row; C % 8 == 0, so a
                                          // chunk is wholly inside or outside the output
  for (int e = tid; e < BM * kChunksPerRow; e += Cfg::kThreads) {
    const int r = e / kChunksPerRow;
    const int ch = e - r * kChunksPerRow;
    const int64_t row = row0 + r;
    const int64_t col = col0 + ch * 8;
    if (row < a.R && col < a.C) {
      const u4 v = *reinterpret_cast<const u4*>(otile + r * Cfg::kOutPitch + ch * 16);
      uint16_t* dst = Y + row * a.ldy + col;
      if (a.y_vec) {
        *reinterpret_cast<u4*>(dst) = v;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dst[2 * w] = (uint16_t)(v[w] & 0xFFFFu);
          dst[2 * w + 1] = (uint16_t)(v[w] >> 16);
        }
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, int KSTEPS, int NST, bool GATHER, bool SMAX = false,
          bool PIPE = true, bool BF = false>
hipError_t launch_wide(WideArgs a, hipStream_t stream) {
  using Cfg = WideCfg<WM, WN, TM, TN, KSTEPS, NST, GATHER>;
  a.n_row_tiles = (a.R + Cfg::BM - 1) / Cfg::BM;
  const int64_t n_col_tiles = (a.C + Cfg::BN - 1) / Cfg::BN;
  a.n_tiles = a.n_row_tiles * n_col_tiles;
  const int64_t total = a.n_tiles * a.batch;
  if (total == 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.xcd_remap = (total % 8) == 0;
  const size_t ring = (size_t)Cfg::kRing + (GATHER ? (size_t)(a.Kc + 2 * Cfg::KS) : 0);
  const size_t lds = ring > (size_t)Cfg::kOut ? ring : (size_t)Cfg::kOut;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = k_spmm_wide<WM, WN, TM, TN, KSTEPS, NST, GATHER, SMAX, PIPE, BF>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, 160 * 1024)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(Cfg::kThreads), lds, stream, a);
  return hipGetLastError();
}

constexpr int64_t kMaxGatherKc = 16384;   // column-loc of one V-block staged in LDS

bool y_rows_aligned(const void* Y, int64_t ldy, int64_t batch, int64_t stride_Y) {
  return ((uintptr_t)Y & 15) == 0 && ldy % 8 == 0 && (batch <= 1 || stride_Y % 8 == 0);
}

}  // namespace

bool spmm_wide_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                        int64_t batch, int64_t stride_B) {
  return C > 32 && spmm_wide_supported(R, Kc, V, M, B, C, ldb, batch, stride_B);
}

bool spmm_wide_supported(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                         int64_t batch, int64_t stride_B) {
  // Kc == 0 is an empty contraction: no stage runs and the epilogue writes zeros
  if (R <= 0 || Kc < 0 || C <= 0 || C % 8 != 0 || ldb % 8 != 0) return false;
  if (((uintptr_t)B & 15) != 0) return false;
  if (batch > 1 && stride_B % 8 != 0) return false;
  if (V > 0 && (V % 32 != 0 || Kc > kMaxGatherKc)) return false;
  // per-lane DMA offsets are 32-bit: one tile's A rows, one stage's B rows
  constexpr int64_t kLim = (int64_t)1 << 31;
  if (128 * Kc >= kLim) return false;
  const int64_t b_stage_rows = V > 0 ? 32 * (int64_t)M : 256;   // largest stage of any tile shape (128 positions)
  if ((b_stage_rows * ldb + C) * 2 >= kLim) return false;
  return true;
}

hipError_t launch_spmm_wide(const void* values, const void* meta, const void* colloc, int64_t R,
                            int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                            void* Y, int64_t ldy, int64_t batch, int64_t stride_values,
                            int64_t stride_meta, int64_t stride_B, int64_t stride_Y,
                            hipStream_t stream, bool a_tiled) {
  if (a_tiled && (V <= 0 || V % 32 != 0 || batch > 1)) return hipErrorInvalidValue;
  WideArgs a{};
  a.a_tiled = a_tiled ? 1 : 0;
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.colloc = (const uint8_t*)colloc;
  a.R = R; a.Kc = Kc; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = batch < 1 ? 1 : batch;
  a.stride_values = stride_values; a.stride_meta = stride_meta;
  a.stride_B = stride_B; a.stride_Y = stride_Y;
  a.V = V; a.M = M;
  a.y_vec = y_rows_aligned(Y, ldy, a.batch, stride_Y);
  // 128 x 256 tiles where they still give every CU two workgroups; 128 x 128 otherwise
  const bool wide_grid = a.batch * ((R + 127) / 128) * ((C + 255) / 256) >= 512;
  const char* op = V > 0 ? (a_tiled ? "spmm_vnm_tiled" : "spmm_vnm") : "spmm_nm";
  const int64_t K = V > 0 ? Kc / 4 * M : Kc;
  if (V > 0) {
    // the large-tile kernel runs one workgroup per CU: only where its grid fills the chip
    const Variant f = forced_variant();
    if (a.batch == 1 && f != Variant::kWide && spmm_vnm_big_eligible(R, Kc, V, M, B, C, ldb) &&
        (f == Variant::kLarge || (R / 128) * ((C + 511) / 512) >= 256)) {
      log_variant(op, R, K, C, "large 128x512");
      return launch_spmm_vnm_big(values, meta, colloc, R, Kc, V, M, B, C, ldb, Y, ldy, a_tiled, stream);
    }
    // its 64 x 256 form wherever that grid has at least 128 workgroups: measured 23.6
    // against 26.4 us (wide 64 x 128) on 11008 x 4096 . 4096 x 256 with V = 64, and 7-20 %
    // faster than the wide tiles on the 1024-row V = 64 and V = 128 products of the sweep
    if (a.batch == 1 && f != Variant::kWide && spmm_vnm_big64_eligible(R, Kc, V, M, B, C, ldb) &&
        (f == Variant::kLarge || (R / 64) * ((C + 255) / 256) >= 128)) {
      log_variant(op, R, K, C, "large 64x256");
      return launch_spmm_vnm_big64(values, meta, colloc, R, Kc, V, M, B, C, ldb, Y, ldy, a_tiled, stream);
    }
    if (V % 128 == 0) {
      if (C > 128 && wide_grid) {
        log_variant(op, R, K, C, "wide 128x256");
        return launch_wide<1, 4, 4, 2, 1, 3, true, false, false>(a, stream);
      }
      log_variant(op, R, K, C, "wide 128x128");
      return launch_wide<1, 4, 4, 1, 2, 3, true>(a, stream);
    }
    if (V % 64 == 0) {
      log_variant(op, R, K, C, "wide 64x128");
      return launch_wide<1, 4, 2, 1, 2, 3, true>(a, stream);
    }
    log_variant(op, R, K, C, "wide 32x128");   // 128-position stages
    return launch_wide<1, 4, 1, 1, 4, 2, true>(a, stream);
  }
  if (C <= 64) {
    log_variant(op, R, K, C, "wide 128x64");   // 128-position stages
    return launch_wide<4, 1, 1, 2, 4, 2, false>(a, stream);
  }
  if (C <= 128 || !wide_grid) {
    log_variant(op, R, K, C, "wide 128x128");
    return launch_wide<1, 4, 4, 1, 2, 3, false>(a, stream);
  }
  log_variant(op, R, K, C, "wide 128x256");
  return launch_wide<1, 4, 4, 2, 1, 3, false, false, false>(a, stream);
}

hipError_t launch_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K,
                               const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                               int64_t batch, int64_t stride_values, int64_t stride_meta,
                               int64_t stride_B, int64_t stride_Y, hipStream_t stream) {
  if (!spmm_wide_supported(R, K, 0, 4, B, C, ldb, batch, stride_B)) return hipErrorInvalidValue;
  WideArgs a{};
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.R = R; a.Kc = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = batch < 1 ? 1 : batch;
  a.stride_values = stride_values; a.stride_meta = stride_meta;
  a.stride_B = stride_B; a.stride_Y = stride_Y;
  a.V = 0; a.M = 4;
  a.y_vec = y_rows_aligned(Y, ldy, a.batch, stride_Y);
  const bool wide_grid = a.batch * ((R + 127) / 128) * ((C + 255) / 256) >= 512;
  if (C <= 64) return launch_wide<4, 1, 1, 2, 4, 2, false, false, true, true>(a, stream);
  if (C <= 128 || !wide_grid) return launch_wide<1, 4, 4, 1, 2, 3, false, false, true, true>(a, stream);
  return launch_wide<1, 4, 4, 2, 1, 3, false, false, false, true>(a, stream);
}

}  // namespace snm

namespace snm {

hipError_t launch_spmm_nm_softmax(const void* values, const void* meta, const float* row_max,
                                  int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb,
                                  void* Y, int64_t ldy, int64_t batch, int64_t stride_values,
                                  int64_t stride_meta, int64_t stride_row_max, int64_t stride_B,
                                  int64_t stride_Y, bool bf16, hipStream_t stream) {
  if (!spmm_wide_supported(R, K, 0, 4, B, C, ldb, batch, stride_B)) return hipErrorInvalidValue;
  WideArgs a{};
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.rowmax = row_max;
  a.R = R; a.Kc = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = batch < 1 ? 1 : batch;
  a.stride_values = stride_values; a.stride_meta = stride_meta;
  a.stride_B = stride_B; a.stride_Y = stride_Y; a.stride_rowmax = stride_row_max;
  a.V = 0; a.M = 4;
  a.y_vec = y_rows_aligned(Y, ldy, a.batch, stride_Y);
  // one wave column (WN = 1) so each score is exponentiated once per column tile
  if (bf16) {
    if (C <= 64) return launch_wide<4, 1, 1, 2, 4, 2, false, true, true, true>(a, stream);
    return launch_wide<4, 1, 1, 4, 2, 3, false, true, true, true>(a, stream);
  }
  if (C <= 64) return launch_wide<4, 1, 1, 2, 4, 2, false, true>(a, stream);    // 128 x 64
  return launch_wide<4, 1, 1, 4, 2, 3, false, true>(a, stream);                 // 128 x 128 (strips)
}

}  // namespace snm
