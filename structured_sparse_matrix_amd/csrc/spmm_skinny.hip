// 2:4 SpMM for skinny dense operands (C <= 32 columns): the decode regime, where the
// product is bound by streaming the compressed weights from HBM ("2:4 sparsity on
// sparse tensor cores", lecture notes: "Speedup: a staircase toward 2x" -- small GEMMs
// are bound by memory traffic and fixed costs).
//
// Design for MI355X (gfx950), from rocprof timings and counters of earlier variants:
//   * one workgroup per 16-row tile of A; its NW waves (up to 16) split the reduction
//     into slices of S = 64*KSUB positions; K is walked in phases of P = NW*S.
//   * every cache line is requested by exactly one wave: concurrent misses of several
//     waves to one line are not merged and were measured to multiply HBM traffic (six
//     times for scattered 2-byte metadata reads). So
//       - A values: with the canonical layout one load covers 16 rows x 64 contiguous
//         bytes; with the operand-major layout (snm_spmm_nm_tiled) every operand is one
//         contiguous 1 KiB block, which streams about a quarter faster;
//       - canonical metadata is loaded cooperatively (coalesced) into LDS; operand-major
//         metadata is one contiguous 128-byte block per operand, loaded directly;
//       - column-major B (decode activations X[C][K] as stored): each lane loads its
//         operand half (eight consecutive k of one column) directly; the four lanes of
//         a column together read whole 128-byte lines. Row-major B: the phase's B tile
//         is loaded cooperatively into LDS as [k][CP] and read with ds_read_b64_tr_b16.
//   * LDS staging (row-major B, canonical metadata) is requested before A, so the
//     barrier waits for L2, not for the HBM stream.
//   * the per-wave fp32 partial sums are added through LDS once; Y is written with
//     consecutive threads on consecutive columns.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"
#include "variant.hpp"

#include <type_traits>

namespace snm {

struct SkinnyArgs {
  const uint16_t* values;
  const uint8_t* meta;
  const uint16_t* B;
  uint16_t* Y;
  int64_t R, Kc, C, ldb, ldy;
  int64_t batch, stride_values, stride_meta, stride_B, stride_Y;
  int b_vec;   // B rows (row-major) or B columns (column-major) are 16-byte aligned
};

template <int CP, int KSUB>
struct SkinnyCfg {
  static constexpr int S = 64 * KSUB;                        // positions per wave slice
  static constexpr int CT = CP / 16;                         // 16-column MFMA tiles
  // row-major B tile of one phase: NW*S rows x CP columns = NW*S*CP/8 chunks of 16 bytes
  // over 64*NW threads -> S*CP/512 chunks per thread.
  static constexpr int kBChunks = S * CP / 512;
  // canonical metadata tile of one phase: 16 rows x NW*S/16 halfwords over 64*NW threads
  static constexpr int kMetaHalves = S / 64;
};

// Row-major [k][CP] tile with 32-byte cells XOR-placed so that one transpose read
// (rows {0..3, 8..11, 16..19, 24..27} + const) hits each of the 8 cells of a 256-byte
// line at most twice.
template <int CP>
__device__ __forceinline__ uint32_t rm_offset(int x, int c) {
  const uint32_t inner = (uint32_t)(c & 15) * 2u;
  if constexpr (CP == 16) {
    const int L = x >> 3;
    const int u = (x & 7) ^ ((L & 1) << 2);
    return (uint32_t)L * 256u + (uint32_t)u * 32u + inner;
  } else {
    static_assert(CP == 32, "skinny tiles are 16 or 32 columns wide");
    const int L = x >> 2;
    const int u = (((x & 3) << 1) | (c >> 4)) ^ ((L >> 1) & 1);
    return (uint32_t)L * 256u + (uint32_t)u * 32u + inner;
  }
}

// ATILED: A (values, meta) in the operand-major layout; BCOL: B column-major;
// BVEC: B lines are 16-byte aligned.
template <int CP, int KSUB, bool ATILED, bool BCOL, bool BVEC>
__global__ void __launch_bounds__(1024)
k_spmm_skinny(SkinnyArgs a) {
  using Cfg = SkinnyCfg<CP, KSUB>;
  constexpr int S = Cfg::S, CT = Cfg::CT;
  constexpr bool kStageB = !BCOL;          // row-major B goes through LDS
  constexpr bool kStageMeta = !ATILED;     // canonical metadata goes through LDS
  constexpr bool kBarrier = kStageB || kStageMeta;
  static_assert(!kStageB || S * CP * 2 <= 16384, "phase B tile must fit in 160 KiB with 16 waves");
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int NW = blockDim.x >> 6;
  const int nthreads = blockDim.x;
  const int q = lane >> 4;
  const int li = lane & 15;
  const int64_t rt = blockIdx.x;
  const int64_t row0 = rt * 16;
  const int P = NW * S;                                     // positions per phase
  const int nphases = (int)((a.Kc + P - 1) / P);
  const int64_t KC = (a.Kc + 63) / 64;                      // 64-position operand chunks
  const int64_t vals_row = a.Kc >> 1;
  const int64_t meta_row = a.Kc >> 3;
  const bool row_ok = row0 + li < a.R;
  // LDS: [B tile (row-major B only) | canonical metadata tile (16 rows, pitch P/8 + 4 B)]
  const uint32_t btile_bytes = kStageB ? (uint32_t)P * CP * 2u : 0u;
  const uint32_t mpitch = (uint32_t)P / 8u + 4u;
  const uint32_t mtile = btile_bytes;

  // Cooperative staging geometry: chunk i of this thread is a fixed base plus a
  // workgroup-uniform stride (CP/8 and P/16 divide the thread count).
  const int bline0 = tid / (CP / 8);                        // B row within the phase
  const int bcol0 = (tid - bline0 * (CP / 8)) * 8;
  const int bstep = nthreads / (CP / 8);
  const uint32_t boff0 = rm_offset<CP>(bline0, bcol0);
  const uint32_t bofs_step = (uint32_t)bstep * CP * 2u;
  const int mdiv = P / 16;
  const int mrow0 = tid / mdiv;
  const int mhw = tid - mrow0 * mdiv;
  const int mstep = nthreads / mdiv;
  const uint32_t moff0 = mtile + (uint32_t)mrow0 * mpitch + (uint32_t)mhw * 2u;

  for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
    const uint16_t* __restrict__ vals = a.values + b * a.stride_values;
    const uint8_t* __restrict__ meta = a.meta + b * a.stride_meta;
    const uint16_t* __restrict__ Bm = a.B + b * a.stride_B;
    uint16_t* __restrict__ Y = a.Y + b * a.stride_Y;

    f4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};

    for (int ph = 0; ph < nphases; ++ph) {
      const int64_t pbase = (int64_t)ph * P;
      // ---- cooperative staging requests (L2), issued before the HBM stream ------------
      u4 bst[kStageB ? Cfg::kBChunks : 1];
      if constexpr (kStageB) {
        const int col = bcol0;
        const uint16_t* src0 = Bm + (pbase + bline0) * a.ldb + col;
        const int64_t sstep = (int64_t)bstep * a.ldb;
#pragma unroll
        for (int i = 0; i < Cfg::kBChunks; ++i) {
          u4 v = {0u, 0u, 0u, 0u};
          const uint16_t* src = src0 + i * sstep;
          if (pbase + bline0 + i * bstep < a.Kc) {
            if (BVEC && col + 8 <= a.C) {
              v = *reinterpret_cast<const u4*>(src);
            } else if (col < a.C) {
              uint32_t e[8];
#pragma unroll
              for (int t = 0; t < 8; ++t) e[t] = (col + t < a.C) ? src[t] : 0u;
              v[0] = e[0] | (e[1] << 16);
              v[1] = e[2] | (e[3] << 16);
              v[2] = e[4] | (e[5] << 16);
              v[3] = e[6] | (e[7] << 16);
            }
          }
          bst[i] = v;
        }
      }
      uint32_t mst[kStageMeta ? Cfg::kMetaHalves : 1];
      if constexpr (kStageMeta) {
        const int64_t k = pbase + mhw * 16;
        const uint8_t* src0 = meta + (row0 + mrow0) * meta_row + (k >> 3);
        const int64_t sstep = (int64_t)mstep * meta_row;
#pragma unroll
        for (int i = 0; i < Cfg::kMetaHalves; ++i) {
          uint32_t v = 0;
          if (row0 + mrow0 + i * mstep < a.R && k < a.Kc) v = *reinterpret_cast<const uint16_t*>(src0 + i * sstep);
          mst[i] = v;
        }
      }
      // ---- this wave's A operands: operand t of quarter q = positions w*S + 64t + 16q + [0,16)
      h8 av[KSUB];
      uint32_t ai[KSUB];
#pragma unroll
      for (int t = 0; t < KSUB; ++t) {
        const int64_t kd = pbase + w * S + 64 * t + 16 * q;
        h8 v = {};
        uint32_t id = 0;
        if constexpr (ATILED) {
          const int64_t blk = rt * KC + (kd >> 6);   // the tiled arrays are padded: rows and chunks exist
          if (kd < a.Kc) {
            v = *reinterpret_cast<const h8*>(vals + blk * 512 + lane * 8);
            id = *reinterpret_cast<const uint16_t*>(meta + (blk * 64 + lane) * 2);
          }
        } else {
          if (row_ok && kd < a.Kc) v = *reinterpret_cast<const h8*>(vals + (row0 + li) * vals_row + (kd >> 1));
        }
        av[t] = v;
        ai[t] = id;
      }
      // ---- column-major B: operand halves straight from memory -------------------------
      h16 bdir[BCOL ? KSUB : 1][BCOL ? CT : 1];
      if constexpr (BCOL) {
#pragma unroll
        for (int t = 0; t < KSUB; ++t) {
          const int64_t k1 = pbase + w * S + 64 * t + 8 * q;   // rows k1 + e, k1 + 32 + e - 8
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int64_t col = 16 * ct + li;
            const uint16_t* colp = Bm + col * a.ldb;
            h8 lo = {}, hi = {};
            // K is a multiple of 16 and k1 of 8: each 8-row half is wholly inside or outside
            if (col < a.C) {
              if constexpr (BVEC) {
                if (k1 < a.Kc) lo = *reinterpret_cast<const h8*>(colp + k1);
                if (k1 + 32 < a.Kc) hi = *reinterpret_cast<const h8*>(colp + k1 + 32);
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  if (k1 < a.Kc) lo[e] = bits_f16(colp[k1 + e]);
                  if (k1 + 32 < a.Kc) hi[e] = bits_f16(colp[k1 + 32 + e]);
                }
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) { bdir[t][ct][e] = lo[e]; bdir[t][ct][8 + e] = hi[e]; }
          }
        }
      }
      // ---- publish staged tiles ----------------------------------------------------------
      if constexpr (kStageB) {
#pragma unroll
        for (int i = 0; i < Cfg::kBChunks; ++i) *reinterpret_cast<u4*>(smem + boff0 + i * bofs_step) = bst[i];
      }
      if constexpr (kStageMeta) {
#pragma unroll
        for (int i = 0; i < Cfg::kMetaHalves; ++i)
          *reinterpret_cast<uint16_t*>(smem + moff0 + i * mstep * mpitch) = (uint16_t)mst[i];
      }
      if constexpr (kBarrier) __syncthreads();
      // ---- sparse MFMAs over the slice ---------------------------------------------------
      const int xs = w * S;
      const int r1_0 = xs + 8 * q + (li >> 2);
      const uint32_t tr0 = rm_offset<CP>(r1_0, 4 * (li & 3));
      const uint32_t tr4 = rm_offset<CP>(r1_0 + 4, 4 * (li & 3));
      constexpr uint32_t kRow64 = 64u * CP * 2u;       // +64 rows
      constexpr uint32_t kRow32 = 32u * CP * 2u;       // +32 rows
      const uint32_t ct_step = CP == 32 ? rm_offset<CP>(r1_0, 16 + 4 * (li & 3)) - tr0 : 0u;
#pragma unroll
      for (int t = 0; t < KSUB; ++t) {
        uint32_t idx = ai[t];
        if constexpr (kStageMeta)
          idx = *reinterpret_cast<const uint16_t*>(
              smem + mtile + (uint32_t)li * mpitch + (uint32_t)((xs + 64 * t + 16 * q) >> 3));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          h16 bf;
          if constexpr (BCOL) {
            bf = bdir[t][ct];
          } else {
            // transpose reads: the swizzle turns +64 rows and +32 rows into constant byte
            // offsets and +4 rows / +16 columns into per-lane constants
            const uint32_t o0 = lds + tr0 + ct * ct_step + t * kRow64;
            const uint32_t o4 = lds + tr4 + ct * ct_step + t * kRow64;
            const h4 b0 = lds_read_tr16(o0);
            const h4 b1 = lds_read_tr16(o4);
            const h4 b2 = lds_read_tr16(o0 + kRow32);
            const h4 b3 = lds_read_tr16(o4 + kRow32);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bf[e] = b0[e]; bf[4 + e] = b1[e]; bf[8 + e] = b2[e]; bf[12 + e] = b3[e];
            }
          }
          acc[ct] = smfmac16<0>(av[t], bf, acc[ct], idx);
        }
      }
      if constexpr (kBarrier) __syncthreads();
    }

    // ---- sum the NW partial tiles and store Y ----------------------------------------------
    f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) red[(w * CT + ct) * 64 + lane] = acc[ct];
    __syncthreads();
    for (int e = tid; e < 16 * CP; e += nthreads) {
      const int r = e / CP;
      const int c = e - r * CP;
      const int ct = c >> 4;
      const int ln = ((r >> 2) << 4) | (c & 15);
      const float* rp = reinterpret_cast<const float*>(red);
      float s = 0.f;
      for (int ww = 0; ww < NW; ++ww) s += rp[((ww * CT + ct) * 64 + ln) * 4 + (r & 3)];
      const int64_t orow = row0 + r;
      if (orow < a.R && c < a.C) Y[orow * a.ldy + c] = f16_bits(to_f16(s));
    }
    __syncthreads();
  }
}

template <int CP, int KSUB, bool ATILED, bool BCOL, bool BVEC>
static hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream) {
  using Cfg = SkinnyCfg<CP, KSUB>;
  const int64_t nslices = (a.Kc + Cfg::S - 1) / Cfg::S;
  int nw = (int)(nslices < 16 ? nslices : 16);
  if (nw < 1) nw = 1;
  const size_t P = (size_t)nw * Cfg::S;
  const size_t btile = BCOL ? 0 : P * CP * 2;
  const size_t mtile = ATILED ? 0 : 16 * (P / 8 + 4);
  const size_t red = (size_t)nw * Cfg::CT * 64 * 16;
  const size_t lds = btile + mtile > red ? btile + mtile : red;
  auto kern = k_spmm_skinny<CP, KSUB, ATILED, BCOL, BVEC>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, 160 * 1024)) return e;
  const unsigned gx = (unsigned)((a.R + 15) / 16);
  const unsigned gy = (unsigned)(a.batch < 65535 ? a.batch : 65535);
  hipLaunchKernelGGL(kern, dim3(gx, gy), dim3(64 * nw), lds, stream, a);
  return hipGetLastError();
}

// Phases of up to 4096 positions (S = 256); row-major B with 32 columns uses phases of
// 2048 (S = 128) so that its LDS tile fits.
template <bool ATILED>
static hipError_t dispatch_skinny(const SkinnyArgs& a, int b_layout, hipStream_t stream) {
  const bool narrow = a.C <= 16;
  if (b_layout == 1) {
    if (a.b_vec)
      return narrow ? launch_skinny<16, 4, ATILED, true, true>(a, stream) : launch_skinny<32, 4, ATILED, true, true>(a, stream);
    return narrow ? launch_skinny<16, 4, ATILED, true, false>(a, stream) : launch_skinny<32, 4, ATILED, true, false>(a, stream);
  }
  if (a.b_vec)
    return narrow ? launch_skinny<16, 4, ATILED, false, true>(a, stream) : launch_skinny<32, 2, ATILED, false, true>(a, stream);
  return narrow ? launch_skinny<16, 4, ATILED, false, false>(a, stream) : launch_skinny<32, 2, ATILED, false, false>(a, stream);
}

static SkinnyArgs skinny_args(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                              int64_t C, int64_t ldb, void* Y, int64_t ldy, int64_t batch,
                              int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                              int64_t stride_Y) {
  SkinnyArgs a{};
  a.values = (const uint16_t*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.R = R; a.Kc = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.batch = batch;
  a.stride_values = stride_values; a.stride_meta = stride_meta;
  a.stride_B = stride_B; a.stride_Y = stride_Y;
  a.b_vec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0) && (batch <= 1 || stride_B % 8 == 0);
  return a;
}


// ---------------------------------------------------------------------------------------
// Column-major B through an LDS ring (operand-major A, one product): the decode regime's
// other stream. Every workgroup needs all of B (C x K, 256 KiB at C = 32, K = 4096). Loaded
// straight into the operand registers, each lane takes 16 bytes of one column, so one load
// instruction touches sixteen 128-byte lines, half of each, and B arrives at about a third
// of the rate at which whole lines can be copied into LDS. Here B goes global -> LDS by DMA,
// one whole 1 KiB column slice per instruction, into a ring of NBUF phases of 512 positions;
// each wave reads its operands back with two 16-byte LDS reads per column tile. A (the HBM
// stream) is requested in full at the start, as in the register kernel above.
//   * eight waves; phase p covers positions [512 p, 512 p + 512), wave w the operand chunk
//     8 p + w (64 positions); the phase count NPH = K / 512 is a template parameter, so that
//     every wait below is an exact count; each workgroup walks the phases from its own
//     starting phase (the fp32 sums of a row are still in one fixed order per launch shape);
//   * ring slot: CP column slices of 1 KiB, each padded by 16 bytes so that the sixteen
//     columns one read touches start in sixteen different 16-byte bank groups;
//   * copies: wave w copies columns w*D .. w*D + D - 1 of the phase (D = CP / 8); columns
//     past C are copied from column C - 1 (they feed only output columns that are not
//     stored), except that a wave whose columns all lie past C copies nothing (its waits
//     then only cover its own loads of A, which the compiler waits for anyway);
//   * issue order: the copies of the first NBUF phases (every slot is free), then A, then one
//     phase of copies per barrier. Loads and copies retire in issue order, so phase p < NBUF
//     waits for its own copies and A of the phases it needs, not for all of A; the copies of
//     phase p + NBUF - 1 go out at barrier p >= 1 (every read of phase p - 1, whose slot it
//     takes, has retired there) while the rest of A is still arriving;
//   * one barrier per phase: wait for this wave's copies of phase p, barrier (publishes
//     phase p), copy, read and multiply phase p.
namespace sring {
constexpr int NW = 8, THREADS = 64 * NW;
// KS: 64-position operands per wave per phase. Operand-major A: 1 (a phase of 512 positions,
// four ring slots). Canonical A: 2, so that one wave reads both halves of every 128-byte line
// of its 16 rows (two adjacent chunks) -- concurrent misses of two waves to one line are not
// merged -- with phases of 1024 positions in two slots (the same bytes in flight).
template <int CP, int KS>
struct Cfg {
  static constexpr int PK = 64 * NW * KS;          // positions per phase
  static constexpr int NBUF = KS == 1 ? 4 : 2;     // ring slots
  static constexpr int kMaxPhases = 8192 / PK;     // A of every phase is held in registers
  static constexpr int kPitch = PK * 2 + 16;       // one padded column slice of a phase
  static constexpr int CT = CP / 16;
  static constexpr int D = CP / NW * KS;           // copies (1 KiB each) per wave per phase
  static constexpr int kSlot = CP * kPitch;
  static constexpr int kLds = NBUF * kSlot;
  static_assert(NW * CT * 64 * 16 <= kLds, "the partial-sum tile fits in the ring");
  // at most NBUF + 1 phases of copies and all of A are outstanding at once
  static_assert((NBUF + 1) * D + 2 * KS * kMaxPhases < 64, "vmcnt holds at most 63 outstanding operations");
  // phases copied before A is requested, and whether barrier q issues the copies of q + NBUF - 1
  static constexpr int prologue(int nph) { return nph < NBUF ? nph : NBUF; }
  static constexpr bool issues_at(int q, int nph) { return q >= 1 && q + NBUF - 1 < nph; }
  // vector-memory operations a copying wave issues after phase p's copies and before its
  // wait at phase p
  static constexpr int younger(int p, int nph) {
    int n = 0;
    if (p < prologue(nph)) {
      n += D * (prologue(nph) - 1 - p) + 2 * KS * nph;
      for (int q = 1; q < p; ++q) n += issues_at(q, nph) ? D : 0;
    } else {
      for (int q = p - NBUF + 2; q < p; ++q) n += issues_at(q, nph) ? D : 0;
    }
    return n;
  }
};
template <bool ATILED>
constexpr int ks_of() { return ATILED ? 1 : 2; }
}  // namespace sring

template <int I, int N, typename F>
__device__ __forceinline__ void ring_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    ring_for<I + 1, N>(f);
  }
}

template <int CP, int NPH, bool ATILED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
k_spmm_skinny_ring(SkinnyArgs a) {
  using namespace sring;
  constexpr int KS = ks_of<ATILED>();
  using Cf = Cfg<CP, KS>;
  constexpr int CT = Cf::CT, D = Cf::D, PK = Cf::PK, NBUF = Cf::NBUF, PRO = Cf::prologue(NPH);
  constexpr int kPitch = Cf::kPitch;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t lds0 = lds_addr(smem);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int li = lane & 15;
  const int64_t rt = blockIdx.x;
  const int64_t row0 = rt * 16;
  const int64_t KC = (int64_t)NPH * (PK / 64);   // 64-position chunks per row
  // Phase order rotated per workgroup: consecutive workgroups go to different XCDs, so the
  // 32 or so of one XCD (every eighth) start at different phases and together request all
  // of B at once; the later phases of each then find their lines in that XCD's L2. Ring
  // position p (registers, slot) holds memory phase phys(p).
  const int rot = (int)((blockIdx.x >> 3) % NPH);
  auto phys = [&](int p) { const int v = p + rot; return v >= NPH ? v - NPH : v; };

  // ---- B copies: this wave's CP / NW columns (none when they all lie past C) --------------
  constexpr int NCOL = CP / NW;
  const bool copies = (int64_t)w * NCOL < a.C;
  uint32_t voff[NCOL];
  uint32_t lcol[NCOL];
#pragma unroll
  for (int j = 0; j < NCOL; ++j) {
    const int col = w * NCOL + j;
    const int64_t src = col < a.C ? col : a.C - 1;
    voff[j] = (uint32_t)((src * a.ldb) * 2 + lane * 16);
    lcol[j] = (uint32_t)(col * kPitch);
  }
  auto copy_phase = [&](int p, int slot) {
    if (!copies) return;
#pragma unroll
    for (int j = 0; j < NCOL; ++j)
#pragma unroll
      for (int h = 0; h < KS; ++h)
        dma_s<16>(a.B + (int64_t)phys(p) * PK + 512 * h, voff[j],
                  lds0 + (uint32_t)(slot * Cf::kSlot) + lcol[j] + (uint32_t)(1024 * h));
  };
#pragma unroll
  for (int p = 0; p < PRO; ++p) copy_phase(p, p);

  // ---- A: every phase's operands (chunk KS (NW p + w) + t) -------------------------------------
  h8 av[NPH][KS];
  uint32_t ai[NPH][KS];
  // canonical rows past R read row R - 1 (their outputs are not stored), so that every wave
  // issues the same loads
  const int64_t crow = row0 + li < a.R ? row0 + li : a.R - 1;
#pragma unroll
  for (int p = 0; p < NPH; ++p)
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int64_t chunk = (int64_t)KS * (NW * phys(p) + w) + t;
      if constexpr (ATILED) {
        const int64_t blk = rt * KC + chunk;
        av[p][t] = *reinterpret_cast<const h8*>(a.values + blk * 512 + lane * 8);
        ai[p][t] = *reinterpret_cast<const uint16_t*>(a.meta + (blk * 64 + lane) * 2);
      } else {
        av[p][t] = *reinterpret_cast<const h8*>(a.values + crow * (a.Kc >> 1) + chunk * 32 + 8 * q);
        ai[p][t] = *reinterpret_cast<const uint16_t*>(a.meta + crow * (a.Kc >> 3) + chunk * 8 + 2 * q);
      }
    }

  f4 acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
  // LDS byte offset of this lane's first operand half in a slot: column li of tile 0,
  // positions 64 (KS w + t) + 8 q (the second half is 32 positions on, 64 bytes)
  const uint32_t rd0 = (uint32_t)(li * kPitch + (64 * KS * w + 8 * q) * 2);

  ring_for<0, NPH>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    wait_vmcnt<Cf::younger(p, NPH)>();
    lds_barrier();
    if constexpr (Cf::issues_at(p, NPH)) copy_phase(p + NBUF - 1, (p + NBUF - 1) % NBUF);
    constexpr uint32_t so = (uint32_t)((p % NBUF) * Cf::kSlot);
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint32_t o = so + rd0 + (uint32_t)(ct * 16 * kPitch + 128 * t);
        const h8 lo = *reinterpret_cast<const h8*>(smem + o);
        const h8 hi = *reinterpret_cast<const h8*>(smem + o + 64);
        const h16 bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        acc[ct] = smfmac16<0>(av[p][t], bf, acc[ct], ai[p][t]);
      }
  });

  // ---- sum the NW partial tiles and store Y --------------------------------------------------
  lds_barrier();   // every wave is done with the ring
  f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) red[(w * CT + ct) * 64 + lane] = acc[ct];
  __syncthreads();
  for (int e = tid; e < 16 * CP; e += THREADS) {
    const int r = e / CP;
    const int c = e - r * CP;
    const int ct = c >> 4;
    const int ln = ((r >> 2) << 4) | (c & 15);
    const float* rp = reinterpret_cast<const float*>(red);
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += rp[((ww * CT + ct) * 64 + ln) * 4 + (r & 3)];
    const int64_t orow = row0 + r;
    if (orow < a.R && c < a.C) a.Y[orow * a.ldy + c] = f16_bits(to_f16(s));
  }
}

// The ring kernel's shape rules: column-major B with 16-byte column slices (ldb % 8, a
// 16-byte aligned base), whole phases (K % 512 for operand-major A, K % 1024 for canonical A),
// every phase's A in registers (K <= 8192), C <= 32, one product, and 32-bit copy offsets.
static bool skinny_ring_eligible(int64_t K, const void* B, int64_t C, int64_t ldb, bool a_tiled) {
  const int64_t pk = a_tiled ? sring::Cfg<16, 1>::PK : sring::Cfg<16, 2>::PK;
  if (C < 1 || C > 32 || K < pk || K % pk != 0 || K > 8192) return false;
  if (ldb % 8 != 0 || ((uintptr_t)B & 15) != 0) return false;
  return (C * ldb + K) * 2 < ((int64_t)1 << 31);
}

bool skinny_ring_selected(int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, bool a_tiled) {
  return b_layout == 1 && forced_variant() != Variant::kDirect && skinny_ring_eligible(K, B, C, ldb, a_tiled);
}

template <int CP, bool ATILED, int NPH>
static hipError_t launch_skinny_ring(const SkinnyArgs& a, int nph, hipStream_t stream) {
  using Cf = sring::Cfg<CP, sring::ks_of<ATILED>()>;
  if constexpr (NPH < Cf::kMaxPhases) {
    if (nph != NPH) return launch_skinny_ring<CP, ATILED, NPH + 1>(a, nph, stream);
  }
  auto kern = k_spmm_skinny_ring<CP, NPH, ATILED>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, Cf::kLds)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)((a.R + 15) / 16)), dim3(sring::THREADS), Cf::kLds, stream, a);
  return hipGetLastError();
}

template <bool ATILED>
static hipError_t dispatch_skinny_ring(const SkinnyArgs& a, hipStream_t stream) {
  const int nph = (int)(a.Kc / sring::Cfg<16, sring::ks_of<ATILED>()>::PK);
  return a.C <= 16 ? launch_skinny_ring<16, ATILED, 1>(a, nph, stream)
                   : launch_skinny_ring<32, ATILED, 1>(a, nph, stream);
}

hipError_t launch_spmm_nm_skinny(const void* values, const void* meta, int64_t R, int64_t K,
                                 const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                 int64_t ldy, int64_t batch, int64_t stride_values,
                                 int64_t stride_meta, int64_t stride_B, int64_t stride_Y,
                                 hipStream_t stream) {
  const SkinnyArgs a = skinny_args(values, meta, R, K, B, C, ldb, Y, ldy, batch, stride_values,
                                   stride_meta, stride_B, stride_Y);
  if (batch == 1 && skinny_ring_selected(K, B, C, ldb, b_layout, false)) return dispatch_skinny_ring<false>(a, stream);
  return dispatch_skinny<false>(a, b_layout, stream);
}

hipError_t launch_spmm_nm_tiled_skinny(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                       const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                       int64_t ldy, hipStream_t stream) {
  const SkinnyArgs a = skinny_args(values_t, meta_t, R, K, B, C, ldb, Y, ldy, 1, 0, 0, 0, 0);
  if (skinny_ring_selected(K, B, C, ldb, b_layout, true)) return dispatch_skinny_ring<true>(a, stream);
  return dispatch_skinny<true>(a, b_layout, stream);
}

}  // namespace snm
