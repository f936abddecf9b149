// V:2:M structured-sparse x dense product with V-blocks of 64 rows ("VENOM ...", SC'23, Sec. 4
// and Fig. 4: per block of V rows, the K/M*4 rows of B named by column-loc are gathered and
// the product becomes 2:4 over K' = 4K/M), on the sparse matrix core of gfx950. This is the
// large-tile kernel's form for V % 64 == 0 (spmm_vnm_big.hip holds the 128 x 512 one).
//
// One workgroup = 64 rows (one V-block, or half of one) x 256 output columns, eight waves
// (two per SIMD), one workgroup per CU. Each wave owns all 64 rows x its 32 columns: two
// tiles of v_smfmac_f32_32x32x32_f16 with fp32 accumulators, so a B operand read from LDS
// serves both row tiles. Per 64-position stage the ring holds the 64 gathered B rows x 256
// columns (32 KiB), the tile's values (4 KiB) and its index words zero-extended to dwords
// (1 KiB), 37 KiB in all, copied global -> LDS by the DMA path into a 4-deep ring (148 KiB).
// Each wave copies 8 of the B rows (four instructions of two rows) and one values block
// (waves 0-3) or one index block (waves 4-7), waits for its own copies of the stage about
// to be read (s_waitcnt vmcnt), and one barrier per stage publishes them and frees the
// oldest slot. A stage's products run on the previous stage's operands, with this stage's
// operand reads and one copy between products. The stage loop runs in rounds of four
// stages so that ring slots and operand buffers are compile-time constants; the first and
// last rounds are peeled.
//
// Compared with the 64 x 128 tiles of the wide kernel (two workgroups per CU), every
// workgroup gathers its V-block's B rows once for all 256 columns instead of twice, and
// the four-stage ring keeps three stages of copies in flight.
//
// LDS layouts (B tile cell swizzle, A and index blocks) and the DMA/operand lane maps are
// those of wide_layout.hpp with BN = 256, KS = 64. The output tile is staged through LDS
// and written as whole 128-byte lines.
//
// Shapes: V % 64 == 0 (R a multiple of 64), K' = 4K/M a multiple of 64 (whole stages; a ragged
// last round is padded with stages that are copied but not multiplied) with at least two
// rounds (K' >= 512), K' <= 12288 (column-loc staged after the ring), C >= 128 and
// C % 8 == 0 (a ragged last column tile is clamped on load and masked on store), row-major
// B with ldb % 8 == 0 and 16-byte rows. Values and m-indices canonical or row-group
// interleaved.
#include "elem.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"
#include "wide_layout.hpp"

#include <type_traits>

namespace snm {
namespace {

namespace big64 {
constexpr int BM = 64, BN = 256, KS = 64, NST = 4, WAVES = 8, THREADS = 64 * WAVES;
constexpr int KSTEPS = KS / 32;                 // 32-position products per stage
constexpr int TM = BM / 32;                     // row tiles per wave
constexpr int kBBytes = KS * BN * 2;            // one stage of gathered B rows (32 KiB)
constexpr int kBlocks = (BM / 32) * KSTEPS;     // 1 KiB values blocks = 256 B index blocks
constexpr int kAOff = kBBytes;
constexpr int kMOff = kAOff + kBlocks * 1024;
constexpr int kStage = kMOff + kBlocks * 256;
constexpr int kRing = NST * kStage;
constexpr int kOutPitch = 2 * BN + 64;          // fp16 output rows; the pad spreads rows over banks
constexpr int kOut = BM * kOutPitch;
constexpr int kLdsLimit = 160 * 1024;
constexpr int64_t kMaxKc = kLdsLimit - kRing;
constexpr int nB = kBBytes / 1024 / WAVES;      // B copies per wave per stage, two rows each
constexpr int kDma = nB + 1;                    // and one values or index block
static_assert(kBlocks == WAVES / 2, "waves 0-3 copy the values blocks, waves 4-7 the index blocks");
static_assert(wide::a_rows_per_block<KS>() * kBlocks == BM, "values blocks");
static_assert(wide::m_rows_per_block<KS>() * kBlocks == BM, "index blocks");
static_assert(kDma * (NST - 2) < 64, "vmcnt holds at most 63 outstanding operations");
static_assert(kRing <= kLdsLimit && kOut <= kLdsLimit, "LDS");
}  // namespace big64

struct Big64Args {
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
using cint64 = std::integral_constant<int, I>;
template <int I, int N, typename F>
__device__ __forceinline__ void static_for64(F&& f) {
  if constexpr (I < N) {
    f(cint64<I>{});
    static_for64<I + 1, N>(f);
  }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_64;
__device__ __forceinline__ h4 tr16_at64(uint8_t* smem, uint32_t byte_off) {
  typedef __fp16 fp4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) fp4 lds_fp4;
  lds_fp4* p = (lds_fp4*)((lds_u8_64*)smem + byte_off);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) k_spmm_vnm_big64(Big64Args a) {
  using namespace big64;
  using E = Elem<false>;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register

  // tile of this workgroup (XCD-aware: the workgroups resident on one XCD share a run of
  // column strips of B in its L2)
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

  // column-loc bytes of this tile's V-block after the ring
  {
    const uint8_t* cl = a.colloc + (row0 / a.V) * Kc;
    for (int64_t i = (int64_t)tid * 16; i < Kc; i += THREADS * 16)
      *reinterpret_cast<u4*>(smem + kRing + i) = *reinterpret_cast<const u4*>(cl + i);
    __syncthreads();
  }

  // ---- per-lane DMA sources (stage-invariant) ----------------------------------------
  // B: copy j of this wave fills bytes (nB*wave + j) KiB of the B tile, two tile rows of
  // 256 columns; each lane's row x and first column follow from the cell swizzle
  uint32_t boff[nB];
  int bx[nB];
#pragma unroll
  for (int j = 0; j < nB; ++j) {
    const uint32_t o = (uint32_t)((wave * nB + j) * 1024 + lane * 16);
    const int x = wide::b_row_of<BN>(o);
    int64_t c = col0 + wide::b_col_of<BN>(o);
    c = c < a.C ? c : 0;   // a ragged last column tile: loaded from column 0, never stored
    bx[j] = x;
    boff[j] = (uint32_t)(((int64_t)(x >> 2) * a.M * a.ldb + c) * 2);
  }
  // values block `wave` (waves 0-3) or index block `wave - 4` (waves 4-7)
  const int ablk = wave & 3;
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

  // column-loc byte of each lane's B rows for the next stage this wave copies. Read late in
  // a stage, used after the next barrier (which waits for every LDS read anyway): the empty
  // statement after the barrier keeps the compiler from using it earlier, which would make
  // the wave wait for all of its operand reads in flight in the middle of a stage.
  uint32_t gcl[nB];
  auto fetch_colloc = [&](int64_t s) {
#pragma unroll
    for (int j = 0; j < nB; ++j) gcl[j] = smem[kRing + src(s) * KS + bx[j]];
  };
  auto pin_colloc = [&]() {
#pragma unroll
    for (int j = 0; j < nB; ++j) asm volatile("" : "+v"(gcl[j]));
  };
  // copy J of stage s into ring slot SLOT: J < nB is two gathered B rows, then this wave's
  // values or index block
  auto copy = [&](int64_t s, auto slot_c, auto j_c) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int j = decltype(j_c)::value;
    const uint32_t sb = lds0 + (uint32_t)(slot * kStage);
    if constexpr (j < nB) {
      const uint16_t* bs = a.B + src(s) * (KS / 4) * a.M * a.ldb;
      dma_s<16>(bs, boff[j] + gcl[j] * ldb2, sb + (uint32_t)((wave * nB + j) * 1024));
    } else {
      if (wave < 4) dma_s<16>(vals + src(s) * a_stage, aoff, sb + (uint32_t)(kAOff + ablk * 1024));
      else dma_s<2>(meta + src(s) * m_stage, moff, sb + (uint32_t)(kMOff + ablk * 256));
    }
  };
  auto copy_all = [&](int64_t s, auto slot_c) {
    static_for64<0, kDma>([&](auto j) { copy(s, slot_c, j); });
  };

  f16v acc[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) acc[tm] = f16v{};

  // lane-constant LDS offsets of the operand reads: A tile tm at + tm * 32 KS bytes, its
  // index words at + 8 KS tm (+ 8 per step); the B operand of step ks is four transpose reads
  // of rows 32 ks + {x, x + 4, x + 16, x + 20} (one cell swizzle)
  uint32_t a_lds[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) a_lds[ks] = wide::a_offset<KS>(lane & 31, 2 * ks + (lane >> 5));
  const uint32_t m_lds = wide::m_offset<KS>(lane & 31, lane >> 5);
  constexpr uint32_t kATile = wide::a_tile_delta<KS>();
  constexpr uint32_t kMTile = wide::m_tile_delta<KS>();
  uint32_t tr_lds;
  {
    const int x = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int cb = wave * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    tr_lds = wide::b_offset<BN>(x, cb);
  }

  struct Frag {
    h8 af[KSTEPS][TM];
    uint32_t ix[KSTEPS][TM];
    h16 bf[KSTEPS];
  };
  auto read_a = [&](Frag& f, uint32_t sb, auto ks_c, auto tm_c) {
    constexpr int ks = decltype(ks_c)::value;
    constexpr int tm = decltype(tm_c)::value;
    f.af[ks][tm] = *reinterpret_cast<const h8*>(smem + a_lds[ks] + (sb + kAOff + tm * kATile));
    f.ix[ks][tm] = *reinterpret_cast<const uint32_t*>(smem + m_lds + (sb + kMOff + tm * kMTile + ks * 8));
  };
  auto read_b = [&](Frag& f, uint32_t sb, auto ks_c) {
    constexpr int ks = decltype(ks_c)::value;
    const uint32_t so = sb + (uint32_t)(ks * 32 * 2 * BN);
    const h4 b0 = tr16_at64(smem, tr_lds + so);
    const h4 b1 = tr16_at64(smem, tr_lds + (so + 4 * 2 * BN));
    const h4 b2 = tr16_at64(smem, tr_lds + (so + 16 * 2 * BN));
    const h4 b3 = tr16_at64(smem, tr_lds + (so + 20 * 2 * BN));
    f.bf[ks] = __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                       __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7),
                                       0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  };
  auto mma = [&](const Frag& f, auto ks_c, auto tm_c) {
    constexpr int ks = decltype(ks_c)::value;
    constexpr int tm = decltype(tm_c)::value;
    acc[tm] = E::smfmac32(f.af[ks][tm], f.bf[ks], acc[tm], f.ix[ks][tm]);
  };

  Frag fr[2];
  // One stage: the four products of the previous stage's operands (step ks, row tile tm in
  // order q = 2 ks + tm), each followed by the matching part of this stage's operand reads
  // and one copy of stage s + NST - 1 into slot (s - 1) % NST, two copies first.
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
      copy(sx, cint64<NX>{}, cint64<0>{});
      copy(sx, cint64<NX>{}, cint64<1>{});
    }
    static_for64<0, KSTEPS * TM>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      constexpr int KS_ = Q / TM, TM_ = Q % TM;
      if constexpr (MMA) {
        if (s - 1 < nst) mma(prev, cint64<KS_>{}, cint64<TM_>{});
      }
      read_a(cur, sb, cint64<KS_>{}, cint64<TM_>{});
      if constexpr (TM_ == 0) read_b(cur, sb, cint64<KS_>{});
      if constexpr (ISSUE && Q + 2 < kDma) copy(sx, cint64<NX>{}, cint64<Q + 2>{});
    });
    // the column-loc of the stage the next stage copies, after this stage's last copy
    if constexpr (ISSUE) fetch_colloc(s + NST);
  };

  // ---- the ring: stage s in slot s % NST, operands of stage s in fr[s % 2] ---------------
  static_for64<0, NST - 1>([&](auto p) {
    constexpr int P = decltype(p)::value;
    fetch_colloc(P);
    copy_all((int64_t)P, cint64<P>{});
  });
  fetch_colloc(NST - 1);
  const int64_t rounds = nstp / NST;
  // first round (no products before stage 0)
  static_for64<0, NST>([&](auto u) {
    constexpr int U = decltype(u)::value;
    wait_vmcnt<kDma * (NST - 2)>();
    lds_barrier();
    stage((int64_t)U, cint64<U>{}, cint64<1>{}, cint64<(U > 0)>{});
  });
  // steady rounds: every stage copies stage s + NST - 1 (< nstp)
  for (int64_t r = 1; r < rounds - 1; ++r) {
    static_for64<0, NST>([&](auto u) {
      constexpr int U = decltype(u)::value;
      wait_vmcnt<kDma * (NST - 2)>();
      lds_barrier();
      stage(r * NST + U, cint64<U>{}, cint64<1>{}, cint64<1>{});
    });
  }
  // last round: only its first stage still copies (stage nstp - 1), and it fetches no
  // column-loc past the V-block's
  static_for64<0, NST>([&](auto u) {
    constexpr int U = decltype(u)::value;
    const int64_t s = (rounds - 1) * NST + U;
    constexpr int kAfter = (NST - 2) < (NST - 1 - U) ? (NST - 2) : (NST - 1 - U);
    wait_vmcnt<kDma * kAfter>();
    lds_barrier();
    if constexpr (U == 0) {
      pin_colloc();
      copy_all(s + NST - 1, cint64<(U + NST - 1) % NST>{});
    }
    stage(s, cint64<U>{}, cint64<0>{}, cint64<1>{});
  });
  if (nstp == nst) {   // products of the last stage, unless it is padding
    static_for64<0, KSTEPS * TM>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      mma(fr[(NST - 1) % 2], cint64<Q / TM>{}, cint64<Q % TM>{});
    });
  }

  // ---- epilogue: fp32 -> fp16 (RNE) through an LDS tile, whole 128-byte lines out --------
  __syncthreads();   // every wave is done with the ring and column-loc
  uint8_t* const otile = smem;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int ctl = wave * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rtl = tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      *reinterpret_cast<uint16_t*>(otile + rtl * kOutPitch + ctl * 2) = f16_bits(to_f16(acc[tm][i]));
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

}  // namespace

bool spmm_vnm_big64_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb) {
  using namespace big64;
  if (V <= 0 || V % BM != 0 || R <= 0 || R % BM != 0) return false;
  if (Kc % KS != 0 || Kc < 2 * KS * NST || Kc > kMaxKc) return false;
  if (C < BN / 2 || C % 8 != 0 || ldb % 8 != 0 || ((uintptr_t)B & 15) != 0) return false;
  // 32-bit DMA offsets: a tile's rows of values, one stage's gathered B rows
  constexpr int64_t kLim = (int64_t)1 << 31;
  if ((int64_t)BM * Kc >= kLim || ((int64_t)(KS / 4) * M * ldb + C) * 2 >= kLim) return false;
  return (R / BM) * ((C + BN - 1) / BN) <= 0x7FFFFFFF;
}

hipError_t launch_spmm_vnm_big64(const void* values, const void* meta, const void* colloc, int64_t R,
                                 int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                                 int64_t ldy, bool a_tiled, hipStream_t stream) {
  using namespace big64;
  if (!spmm_vnm_big64_eligible(R, Kc, V, M, B, C, ldb)) return hipErrorInvalidValue;
  Big64Args a{};
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
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)k_spmm_vnm_big64, kLdsLimit)) return e;
  hipLaunchKernelGGL(k_spmm_vnm_big64, dim3((unsigned)tiles), dim3(THREADS), kLdsLimit, stream, a);
  return hipGetLastError();
}

}  // namespace snm
