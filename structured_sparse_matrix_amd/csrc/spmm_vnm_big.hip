// V:2:M structured-sparse x dense product for large problems ("VENOM ...", SC'23, Sec. 4 and
// Fig. 4: per block of V rows, the K/M*4 rows of B named by column-loc are gathered and the
// product becomes 2:4 over K' = 4K/M), on the sparse matrix core of gfx950.
//
// One workgroup = one V-block of 128 rows x 512 output columns, one workgroup per CU. The
// B rows a V-block gathers are shared only by its 128 rows, so the gathered B stream is
// 512 bytes per 32x32x32 sparse product whatever the tiling; the values and index words add
// 64 bytes per product at 512 columns (128 at 256). The workgroup is as wide as the
// accumulator registers allow: 128 x 512 fp32 = 256 KiB.
//
// Eight waves (two per SIMD) each own all 128 rows x 64 columns: 4 x 2 tiles of
// v_smfmac_f32_32x32x32_f16 whose 128 fp32 accumulators live in the AGPR file (every
// instruction that touches them is bound to it), leaving the ordinary registers for two
// operand buffers and the copy bookkeeping. The body is written for four waves as well (one
// wave per SIMD, 128 x 128 each, 256 accumulators); that form measured within a few percent
// and is not built. Eight waves are used because global -> LDS copies are limited per issuing wave: on one
// MI355X a streaming copy into LDS from L2 reaches about 41 B/clk per CU with four waves
// and 63 B/clk with eight, and a stage moves 37 KiB.
//
// Per 32-position stage: the 32 gathered B rows x 512 columns (32 KiB), the 128 rows'
// values (4 KiB) and index words (zero-extended to dwords, 1 KiB), all copied global -> LDS
// by the DMA path into a 4-deep ring (148 KiB). Each wave copies its share, waits for its
// own copies of the stage about to be read (s_waitcnt vmcnt), and one barrier per stage
// publishes them and frees the oldest slot. The operands of stage s are read while the
// products of stage s - 1 run. The stage loop runs in rounds of four stages so that ring
// slots and operand buffers are compile-time constants; the first and last rounds are
// peeled, so the steady-state round carries no branch.
//
// What bounds it (V:2:16, 8192 x 8192 . 8192 x 4096, per-stage timestamps and ablations of
// a copy of the kernel): the copies. Copies alone take about as long as the products and
// operand reads alone (each about 60-70 us for that shape), and a wave that issues a copy
// waits for the CU's address unit, so the two overlap only in part.
//
// LDS layouts (B tile cell swizzle, A and index blocks) and the DMA/operand lane maps are
// those of wide_layout.hpp with BN = 512, KS = 32. The output tile is staged through LDS
// and written as whole 128-byte lines.
//
// Shapes: V % 128 == 0 (R a multiple of 128), K' = 4K/M a multiple of 32 (whole stages; a
// ragged last round is padded with stages that are copied but not multiplied) with at least
// two rounds (K' >= 256), K' <= 12224 (column-loc of the V-block staged after the ring), C >= 256
// and C % 8 == 0 (a ragged last column tile is clamped on load and masked on store),
// row-major B with ldb % 8 == 0 and 16-byte rows. The values and m-indices may be in the
// canonical or the row-group interleaved storage.
#include "elem.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"
#include "wide_layout.hpp"

#include <type_traits>

namespace snm {
namespace {

namespace big {
constexpr int BM = 128, BN = 512, KS = 32, NST = 4, TM = 4;
constexpr int kBBytes = KS * BN * 2;          // one stage of gathered B rows (32 KiB)
constexpr int kBlocks = BM / 32;              // 1 KiB values blocks = 256 B index blocks
constexpr int kAOff = kBBytes;
constexpr int kMOff = kAOff + kBlocks * 1024;
constexpr int kStage = kMOff + kBlocks * 256;
constexpr int kRing = NST * kStage;
constexpr int kOutPitch = 2 * BN + 64;        // fp16 output rows; the pad spreads rows over banks
constexpr int kOut = BM * kOutPitch;
constexpr int kLdsLimit = 160 * 1024;
constexpr int64_t kMaxKc = kLdsLimit - kRing - 2 * KS;
static_assert(kOut <= kLdsLimit && kRing <= kLdsLimit, "LDS");

// WAVES waves share the 512 columns: each owns all 128 rows x TN 32-column tiles, copies nB
// of a stage's 32 gathered B rows plus (four waves) one values and one index block, or
// (eight waves) one values block (waves 0-3) or one index block (waves 4-7).
template <int WAVES>
struct Cfg {
  static constexpr int kWaves = WAVES, kThreads = 64 * WAVES;
  static constexpr int TN = 16 / WAVES;
  static constexpr int nB = kBBytes / 1024 / WAVES;
  static constexpr int kDma = nB + (WAVES == 4 ? 2 : 1);
  static constexpr int kPairs = TM * TN / 2;     // statements of two products per stage
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
  static_assert(kDma * (NST - 2) < 64, "vmcnt holds at most 63 outstanding operations");
  static_assert(kPairs >= 4 && kDma - 2 <= kPairs, "the stage schedule");
};
}  // namespace big

struct BigArgs {
  const uint8_t* values;   // fp16 bits
  const uint8_t* meta;     // m-indices
  const uint16_t* B;       // row-major, ldb
  uint16_t* Y;
  const uint8_t* colloc;   // (R/V) x Kc bytes
  int64_t R, Kc, C, ldb, ldy;
  int64_t n_row_tiles;
  int V, M;
  int a_tiled;
  int y_vec;
  int xcd_remap;   // the workgroup count is a multiple of 8
};

template <int I>
using cint = std::integral_constant<int, I>;
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(cint<I>{});
    static_for<I + 1, N>(f);
  }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ h4 tr16_at(uint8_t* smem, uint32_t byte_off) {
  typedef __fp16 fp4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) fp4 lds_fp4;
  lds_fp4* p = (lds_fp4*)((lds_u8*)smem + byte_off);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
}

template <int WAVES>
__device__ __forceinline__ void spmm_vnm_big_body(const BigArgs& a) {
  using namespace big;
  using C = Cfg<WAVES>;
  constexpr int THREADS = C::kThreads, TN = C::TN, nB = C::nB, kDma = C::kDma, kPairs = C::kPairs;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register

  // ---- tile (XCD-aware: the workgroups resident on one XCD share a column strip of B) ----
  int64_t L = blockIdx.x;
  if (a.xcd_remap) L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t ct = L / a.n_row_tiles;
  const int64_t rt = L - ct * a.n_row_tiles;
  const int64_t row0 = rt * BM;
  const int64_t col0 = ct * BN;
  const int64_t Kc = a.Kc;
  const int64_t nst = Kc / KS;                  // stages, >= 2 NST
  // the ring runs in rounds of NST stages: a ragged last round is padded with stages whose
  // copies repeat stage nst - 1 (so every wait keeps its count and every address stays in
  // the arrays) and whose products are skipped
  const int64_t nstp = (nst + NST - 1) / NST * NST;
  auto src = [&](int64_t s) { return s < nst ? s : nst - 1; };
  const int64_t mrow = Kc >> 3;                 // index bytes per row; a values row is Kc bytes

  // column-loc bytes of this V-block after the ring
  {
    const uint8_t* cl = a.colloc + (row0 / a.V) * Kc;
    for (int64_t i = (int64_t)tid * 16; i < Kc; i += THREADS * 16)
      *reinterpret_cast<u4*>(smem + kRing + i) = *reinterpret_cast<const u4*>(cl + i);
    __syncthreads();
  }

  // ---- per-lane DMA sources (stage-invariant) ----------------------------------------
  // B: DMA j of this wave fills tile row x = nB*wave + j (one 1 KiB row of 512 columns)
  uint32_t boff[nB];
  const int xrow0 = wave * nB;
#pragma unroll
  for (int j = 0; j < nB; ++j) {
    const uint32_t o = (uint32_t)((xrow0 + j) * 1024 + lane * 16);
    const int x = wide::b_row_of<BN>(o);
    int64_t c = col0 + wide::b_col_of<BN>(o);
    c = c < a.C ? c : 0;   // a ragged last column tile: loaded from column 0, never stored
    boff[j] = (uint32_t)(((int64_t)(x >> 2) * a.M * a.ldb + c) * 2);
  }
  // values block and index block of this wave: block `wave` of both (four waves); block
  // `wave` of the values (waves 0-3) or block `wave - 4` of the index words (waves 4-7)
  const int ablk = WAVES == 4 ? wave : (wave & 3);
  uint32_t aoff, moff;
  {
    const int r = wide::a_dma_row<KS>(ablk, lane);
    const int ch = wide::a_dma_chunk<KS>(ablk, lane);
    aoff = a.a_tiled ? (uint32_t)((int64_t)(r >> 5) * 32 * Kc + ch * 512 + (r & 31) * 16) : (uint32_t)((int64_t)r * Kc + ch * 16);
    const int rm = wide::m_dma_row<KS>(ablk, lane);
    const int wd = wide::m_dma_word<KS>(lane);
    moff = a.a_tiled ? (uint32_t)((int64_t)(rm >> 5) * 32 * mrow + wd * 64 + (rm & 31) * 2) : (uint32_t)((int64_t)rm * mrow + wd * 2);
  }
  const int64_t a_stage = a.a_tiled ? (int64_t)KS * 32 : (int64_t)KS;
  const int64_t m_stage = a.a_tiled ? (int64_t)KS * 4 : (int64_t)(KS / 8);
  const uint8_t* vals = a.values + row0 * Kc;
  const uint8_t* meta = a.meta + row0 * mrow;
  const uint32_t ldb2 = (uint32_t)(a.ldb * 2);

  // column-loc bytes of the nB rows this wave gathers for the next stage it copies, four
  // to a word (xrow0 is a multiple of 4). The word is read late in a stage and only used
  // after the next barrier, which waits for every LDS read anyway: unpacking it earlier
  // would make the wave wait for all of its operand reads in flight (LDS reads complete in
  // order) in the middle of a stage.
  static_assert(nB % 4 == 0, "whole words of column-loc");
  uint32_t gw[nB / 4];
  auto fetch_colloc = [&](int64_t s) {
#pragma unroll
    for (int w = 0; w < nB / 4; ++w) gw[w] = *reinterpret_cast<const uint32_t*>(smem + kRing + src(s) * KS + xrow0 + 4 * w);
  };
  auto pin_colloc = [&]() {
#pragma unroll
    for (int w = 0; w < nB / 4; ++w) asm volatile("" : "+v"(gw[w]));
  };
  // copy J of stage s into ring slot SLOT: J < nB is gathered B row xrow0 + J of the stage,
  // then this wave's values and/or index block. One instruction each, so that a stage's
  // copies can be spread between its matrix instructions.
  auto copy = [&](int64_t s, auto slot_c, auto j_c) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int j = decltype(j_c)::value;
    const uint32_t sb = lds0 + (uint32_t)(slot * kStage);
    if constexpr (j < nB) {
      const uint16_t* bs = a.B + src(s) * (KS / 4) * a.M * a.ldb;
      const uint32_t g = (gw[j / 4] >> (8 * (j % 4))) & 0xFFu;
      dma_s<16>(bs, boff[j] + g * ldb2, sb + (uint32_t)((xrow0 + j) * 1024));
    } else if constexpr (WAVES == 4) {
      if constexpr (j == nB) dma_s<16>(vals + src(s) * a_stage, aoff, sb + (uint32_t)(kAOff + ablk * 1024));
      else dma_s<2>(meta + src(s) * m_stage, moff, sb + (uint32_t)(kMOff + ablk * 256));
    } else {
      if (wave < 4) dma_s<16>(vals + src(s) * a_stage, aoff, sb + (uint32_t)(kAOff + ablk * 1024));
      else dma_s<2>(meta + src(s) * m_stage, moff, sb + (uint32_t)(kMOff + ablk * 256));
    }
  };
  auto copy_all = [&](int64_t s, auto slot_c) {
    static_for<0, kDma>([&](auto j) { copy(s, slot_c, j); });
  };

  // ---- accumulators: 4 x 4 tiles, every instruction on them bound to the AGPR file ----
  // The matrix instructions are inline assembly (the compiler's own forms split the 256
  // accumulators between register files and copy them around every instruction), so the
  // compiler does not insert their wait states: every statement below opens with
  // s_nop 4, which covers a vector-ALU write of an operand just before it (the hardware
  // needs 2), and all of them are volatile, so they keep program order among themselves
  // and against the padding before the epilogue.
  f16v acc[TM][TN];
  {
    const h8 z = {};
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "=a"(acc[tm][tn]) : "v"(z));
  }

  // lane-constant LDS offsets of the operand reads (wide_layout.hpp): A tile tm at + tm KiB,
  // its index words at + 256 tm; the B operand of column tile tn is four transpose reads of
  // rows x, x + 4, x + 16, x + 20 of the tile (one cell swizzle)
  const uint32_t a_lds = wide::a_offset<KS>(lane & 31, lane >> 5);
  const uint32_t m_lds = wide::m_offset<KS>(lane & 31, lane >> 5);
  constexpr uint32_t kATile = wide::a_tile_delta<KS>();
  constexpr uint32_t kMTile = wide::m_tile_delta<KS>();
  uint32_t tr_lds[TN];
  {
    const int x = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int cb = wave * TN * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) tr_lds[tn] = wide::b_offset<BN>(x, cb + tn * 32);
  }

  struct Frag {
    h8 af[TM];
    uint32_t ix[TM];
    h16 bf[TN];
  };
  // operands of one stage, read in four parts: part t = the A operand and index word of row
  // tile t and (t < TN) the B operand of column tile t
  auto read_part = [&](Frag& f, uint32_t sb, auto t_c) {
    constexpr int t = decltype(t_c)::value;
    f.af[t] = *reinterpret_cast<const h8*>(smem + a_lds + (sb + kAOff + t * kATile));
    f.ix[t] = *reinterpret_cast<const uint32_t*>(smem + m_lds + (sb + kMOff + t * kMTile));
    if constexpr (t < TN) {
    const h4 b0 = tr16_at(smem, tr_lds[t] + sb);
    const h4 b1 = tr16_at(smem, tr_lds[t] + (sb + 4 * 2 * BN));
    const h4 b2 = tr16_at(smem, tr_lds[t] + (sb + 16 * 2 * BN));
    const h4 b3 = tr16_at(smem, tr_lds[t] + (sb + 20 * 2 * BN));
    f.bf[t] = __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                      __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7),
                                      0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
  };
  // products (row tile TM_, column tiles TN0, TN0 + 1) of an operand set: one statement
  auto mma_pair = [&](const Frag& f, auto tm_c, auto tn_c) {
    constexpr int tm = decltype(tm_c)::value;
    constexpr int tn = decltype(tn_c)::value;
    f16v* const ar = &acc[tm][tn];   // named outside the statement: a generic lambda captures it
    asm volatile(
        "s_nop 4\n\t"
        "v_smfmac_f32_32x32x32_f16 %0, %2, %3, %5\n\t"
        "v_smfmac_f32_32x32x32_f16 %1, %2, %4, %5"
        : "+a"(ar[0]), "+a"(ar[1])
        : "v"(f.af[tm]), "v"(f.bf[tn]), "v"(f.bf[tn + 1]), "v"(f.ix[tm]));
  };

  Frag fr[2];
  // One stage: the products of the previous stage go out in pairs (64 cycles of matrix work
  // each) with a quarter of this stage's operand reads and one copy between pairs, two
  // copies first. (Measured on the V:2:16 workload against all copies first, one copy per
  // pair, and opposite orders for the two waves of a SIMD: this order was the fastest, by a
  // few percent.) ISSUE: copy stage s + NST - 1 into slot (s - 1) % NST; MMA: the previous
  // stage's operands are complete.
  auto stage = [&](int64_t s, auto u_c, auto issue_c, auto mma_c) {
    constexpr int U = decltype(u_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value != 0;
    constexpr bool MMA = decltype(mma_c)::value != 0;
    constexpr uint32_t sb = (uint32_t)(U * kStage);
    constexpr int NX = (U + NST - 1) % NST;
    Frag& cur = fr[U % 2];
    const Frag& prev = fr[(U + 1) % 2];
    const int64_t sx = s + NST - 1;
    if constexpr (ISSUE) {
      pin_colloc();   // after this stage's barrier: the read has completed
      copy(sx, cint<NX>{}, cint<0>{});
      copy(sx, cint<NX>{}, cint<1>{});
    }
    static_for<0, kPairs>([&](auto q) {
      constexpr int Q = decltype(q)::value;   // product pair: row tile Q / (TN / 2)
      constexpr int kRd = kPairs / 4;         // pairs per read part
      if constexpr (MMA) {
        if (s - 1 < nst) mma_pair(prev, cint<Q / (TN / 2)>{}, cint<2 * (Q % (TN / 2))>{});
      }
      if constexpr (Q % kRd == 0) read_part(cur, sb, cint<Q / kRd>{});
      if constexpr (ISSUE && Q + 2 < kDma) copy(sx, cint<NX>{}, cint<Q + 2>{});
    });
    // the column-loc of the stage the next stage copies, after this stage's last copy
    if constexpr (ISSUE) fetch_colloc(s + NST);
  };

  // ---- the ring: stage s in slot s % NST, operands of stage s in fr[s % 2] ---------------
  // At stage s: wait for this wave's copies of stage s, barrier (publishes every wave's and
  // retires every read of stage s - 1), then, interleaved: copy stage s + NST - 1 into slot
  // (s - 1) % NST, read the operands of stage s, issue the products of stage s - 1.
  static_for<0, NST - 1>([&](auto p) {
    constexpr int P = decltype(p)::value;
    fetch_colloc(P);
    copy_all((int64_t)P, cint<P>{});
  });
  fetch_colloc(NST - 1);
  const int64_t rounds = nstp / NST;
  // first round (no products before stage 0); the fetch of column-loc for stage s + NST
  // stays inside column-loc because nst >= 2 NST
  static_for<0, NST>([&](auto u) {
    constexpr int U = decltype(u)::value;
    wait_vmcnt<kDma * (NST - 2)>();
    lds_barrier();
    stage((int64_t)U, cint<U>{}, cint<1>{}, cint<(U > 0)>{});
  });
  // steady rounds: every stage copies stage s + NST - 1 (< nstp)
  for (int64_t r = 1; r < rounds - 1; ++r) {
    static_for<0, NST>([&](auto u) {
      constexpr int U = decltype(u)::value;
      wait_vmcnt<kDma * (NST - 2)>();
      lds_barrier();
      stage(r * NST + U, cint<U>{}, cint<1>{}, cint<1>{});
    });
  }
  // last round: only its first stage still copies (stage nstp - 1), and it fetches no
  // column-loc past the V-block's
  static_for<0, NST>([&](auto u) {
    constexpr int U = decltype(u)::value;
    const int64_t s = (rounds - 1) * NST + U;
    constexpr int kAfter = (NST - 2) < (NST - 1 - U) ? (NST - 2) : (NST - 1 - U);
    wait_vmcnt<kDma * kAfter>();
    lds_barrier();
    if constexpr (U == 0) {
      pin_colloc();
      copy_all(s + NST - 1, cint<(U + NST - 1) % NST>{});
    }
    stage(s, cint<U>{}, cint<0>{}, cint<1>{});
  });
  if (nstp == nst) {   // products of the last stage, unless it is padding
    static_for<0, kPairs>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      mma_pair(fr[(NST - 1) % 2], cint<Q / (TN / 2)>{}, cint<2 * (Q % (TN / 2))>{});
    });
  }
  // The epilogue reads the accumulators with ordinary instructions: give the last products
  // 32 wait states first (a 16-pass product needs 18), and route every accumulator through
  // an empty statement after them so that no read is scheduled earlier.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) asm volatile("" : "+a"(acc[tm][tn]));

  // ---- epilogue: fp32 -> fp16 (RNE) through an LDS tile, whole 128-byte lines out --------
  __syncthreads();   // every wave is done with the ring and column-loc
  uint8_t* const otile = smem;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int ctl = (wave * TN + tn) * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rtl = tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        *reinterpret_cast<uint16_t*>(otile + rtl * kOutPitch + ctl * 2) = f16_bits(to_f16(acc[tm][tn][i]));
      }
      asm volatile("" ::: "memory");   // convert and store tile by tile
    }
  }
  __syncthreads();
  constexpr int kChunksPerRow = BN / 8;
  for (int e = tid; e < BM * kChunksPerRow; e += THREADS) {
    const int r = e / kChunksPerRow;
    const int ch = e - r * kChunksPerRow;
    const int64_t row = row0 + r;
    const int64_t col = col0 + ch * 8;
    if (row < a.R && col < a.C) {
      const u4 v = *reinterpret_cast<const u4*>(otile + r * kOutPitch + ch * 16);
      uint16_t* dst = a.Y + row * a.ldy + col;
      if (a.y_vec) {
        // streaming stores: the output is not read again here, and it would otherwise
        // displace the gathered B rows other workgroups still read from L2
        __builtin_nontemporal_store(v, reinterpret_cast<u4*>(dst));
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

// the eight-wave instance as a plain kernel: one workgroup per CU, two waves per SIMD
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) k_spmm_vnm_big8(BigArgs a) {
  spmm_vnm_big_body<8>(a);
}

template <int WAVES>
hipError_t launch_big(const BigArgs& a, int64_t tiles, hipStream_t stream) {
  static_assert(WAVES == 8, "the instance built");
  auto kern = k_spmm_vnm_big8;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, big::kLdsLimit)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(64 * WAVES), big::kLdsLimit, stream, a);
  return hipGetLastError();
}

}  // namespace

bool spmm_vnm_big_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb) {
  using namespace big;
  if (V <= 0 || V % BM != 0 || R <= 0 || R % BM != 0) return false;
  if (Kc % KS != 0 || Kc < 2 * KS * NST || Kc > kMaxKc) return false;
  if (C < BN / 2 || C % 8 != 0 || ldb % 8 != 0 || ((uintptr_t)B & 15) != 0) return false;
  // 32-bit DMA offsets: a tile's rows of values, one stage's gathered B rows
  constexpr int64_t kLim = (int64_t)1 << 31;
  if ((int64_t)BM * Kc >= kLim || ((int64_t)(KS / 4) * M * ldb + C) * 2 >= kLim) return false;
  return (R / BM) * ((C + BN - 1) / BN) <= 0x7FFFFFFF;
}

hipError_t launch_spmm_vnm_big(const void* values, const void* meta, const void* colloc, int64_t R,
                               int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                               int64_t ldy, bool a_tiled, hipStream_t stream) {
  using namespace big;
  if (!spmm_vnm_big_eligible(R, Kc, V, M, B, C, ldb)) return hipErrorInvalidValue;
  BigArgs a{};
  a.values = (const uint8_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.colloc = (const uint8_t*)colloc;
  a.R = R; a.Kc = Kc; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.n_row_tiles = R / BM;
  a.V = V; a.M = M;
  a.a_tiled = a_tiled ? 1 : 0;
  a.y_vec = ((uintptr_t)Y & 15) == 0 && ldy % 8 == 0;
  const int64_t tiles = a.n_row_tiles * ((C + BN - 1) / BN);
  a.xcd_remap = tiles % 8 == 0;
  return launch_big<8>(a, tiles, stream);
}

}  // namespace snm
