// Dynamic 2:4 attention kernels ("Dynamic N:M fine-grained structured sparse attention
// mechanism on GPUs", PPoPP'23, Sec. 3.2 and Listing 1; Sec. 4.2 and 4.3).
//
// k_sddmm_prune: S = fp16((Q K^T) * scale) computed on the dense matrix cores and pruned
// to 2:4 along the key axis in the epilogue, so only values + metadata reach memory.
// The product is formed transposed, S^T = K Q^T, because the 32x32 MFMA result then
// hands every lane four consecutive keys of one query -- one whole 2:4 group -- with no
// data movement (this plays the role of the page's column interleave of B). Both
// operands are rows of Q and K read as stored (d contiguous).
//
// k_softmax_rows: row softmax over the kept values only, in place.
//
// Both kernels take fp16 or bf16 (template BF): the page prunes 16-bit scores of either
// type 2:4 (Sec. 4.2); the selection works on bit patterns and is the same for both.
#include "elem.hpp"
#include "launch.hpp"

namespace snm {

// Workgroup: 8 waves (two per SIMD); each wave owns QT tiles of 32 queries and walks all
// keys in tiles of 32. The product is formed transposed (S^T = K Q^T, dense 32x32x16 MFMA)
// so each lane holds four consecutive keys of one query per group. Per tile and lane:
// scale in fp32, round to fp16 (packed RNE conversion), select 2 of 4, and stage the kept
// pairs and the metadata nibbles in the wave's LDS buffers.
//   * values leave every 4 key tiles (128 keys = one 128-byte line per query row), and
//     metadata every 32 key tiles (1024 keys = one 128-byte line per row): only whole
//     lines are written, so the L2 never evicts partly written lines (measured: 16-byte
//     metadata pieces cost as much as the 8x larger value stream). The stores are
//     non-temporal (streaming): the 1.1 GiB of output is not read back by this kernel,
//     and keeping it out of the caches' normal replacement measured 12 % faster.
//   * K tiles rotate through a 4-deep register ring loaded 3 tiles ahead. Vector loads and
//     stores retire in issue order on this architecture, so a load issued after a flush
//     cannot be waited for without waiting for the flush; the ring keeps every wait on a
//     load issued well before the last flush.
//   * the MFMA chain of query tile qt+1 is issued before the epilogue of tile qt.
template <int D, int QT>
struct SddmmCfg {
  static constexpr int kWaves = 8;
  static constexpr int KSTEPS = D / 16;
  static constexpr int KT = 4;                  // key tiles per values flush
  static constexpr int MT = 32;                 // key tiles per metadata flush
  static constexpr int VP = 144;                // staged value bytes per query row: 128 + pad
  static constexpr int MP = 144;                // staged metadata bytes per query row: 128 + pad
  static constexpr int kWaveV = QT * 32 * VP;
  static constexpr int kWaveM = QT * 32 * MP;
  static constexpr int kLds = kWaves * (kWaveV + kWaveM);
  static constexpr int kQueries = kWaves * 32 * QT;   // per workgroup
};

// DENSE: also write the pre-prune 16-bit S (the optional debug output).
// RMAX: also write, per query row, the largest kept score (the fused-softmax variant's
// statistic; a running maximum per lane, two lanes per row: packed fp16, or fp32 for bf16).
// BF: bf16 operands and scores instead of fp16.
template <int D, int QT, bool DENSE, bool RMAX, bool BF>
__global__ void __launch_bounds__(512)
k_sddmm_prune(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Km, int64_t batch,
              int64_t Lq, int64_t Lk, float scale, uint16_t* __restrict__ values,
              uint16_t* __restrict__ meta, uint16_t* __restrict__ S, float* __restrict__ rowmax,
              int xcd_remap) {
  using Cfg = SddmmCfg<D, QT>;
  using E = Elem<BF>;
  constexpr int KSTEPS = Cfg::KSTEPS, KT = Cfg::KT, MT = Cfg::MT, VP = Cfg::VP, MP = Cfg::MP;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;          // which 8-wide d slice / which 4-key subgroup
  const int l32 = lane & 31;
  uint8_t* const sv = smem + wave * Cfg::kWaveV;
  uint8_t* const sm = smem + Cfg::kWaves * Cfg::kWaveV + wave * Cfg::kWaveM;
  // Workgroup -> (query block, batch entry). With xcd_remap the grid is one-dimensional
  // (query blocks x batch, a multiple of 8) and numbered so that the workgroups resident on
  // one XCD take consecutive query blocks of the same batch entries: their key tiles are
  // then fetched into that XCD's L2 once instead of once per XCD.
  int64_t qblk = blockIdx.x, b0 = blockIdx.y, bstep = gridDim.y;
  if (xcd_remap) {
    const int64_t qblocks = (Lq + Cfg::kQueries - 1) / Cfg::kQueries;
    const int64_t L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    b0 = L / qblocks;
    qblk = L - b0 * qblocks;
    bstep = batch;
  }
  const int64_t q_wave = qblk * Cfg::kQueries + (int64_t)wave * 32 * QT;
  const int64_t nkt = Lk >> 5;         // key tiles (Lk % 32 == 0)

  for (int64_t b = b0; b < batch; b += bstep) {
    if (q_wave >= Lq) break;   // whole wave past the end (uniform per wave; no barriers)
    const uint16_t* Qb = Q + b * Lq * D;
    const uint16_t* Kb = Km + b * Lk * D;
    uint16_t* vals_b = values + b * Lq * (Lk >> 1);
    uint8_t* meta_b = reinterpret_cast<uint8_t*>(meta) + b * Lq * (Lk >> 3);
    uint16_t* S_b = DENSE ? S + b * Lq * Lk : nullptr;

    // Q^T operand: column = query, k = d. Lane holds d = 8*half + 16j + [0, 8).
    h8 qf[QT][KSTEPS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t qi = q_wave + qt * 32 + l32;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        h8 v = {};
        if (qi < Lq) v = *reinterpret_cast<const h8*>(Qb + qi * D + 16 * j + 8 * half);
        qf[qt][j] = v;
      }
    }

    // K ring: slot t % 4 holds key tile t; tile t + 3 is requested while tile t is used.
    // Requests past the last tile load the last tile again (nkt >= 1 where this runs), so
    // every path through a block issues the same loads and the waits the compiler derives
    // for each slot are exact instead of the worst case over skipped loads.
    h8 kr[4][KSTEPS];
    auto load_k = [&](int64_t t, h8 (&kf)[KSTEPS]) {
      const int64_t tc = t < nkt ? t : nkt - 1;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        kf[j] = *reinterpret_cast<const h8*>(Kb + (tc * 32 + l32) * D + 16 * j + 8 * half);
    };
    if (nkt > 0) {
      load_k(0, kr[0]);
      load_k(1, kr[1]);
      load_k(2, kr[2]);
    }
    hh2 rmx[QT];     // running max of the kept scores of each query tile's row (RMAX, fp16)
    float rmf[QT];   // the same for bf16
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      rmx[qt] = hh2{(_Float16)-__builtin_inff(), (_Float16)-__builtin_inff()};
      rmf[qt] = -__builtin_inff();
    }

    // the first K tiles and Q are in registers before the loop: the loop head then has no
    // load to wait for on either path into it
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int64_t t0 = 0; t0 < nkt; t0 += KT) {
      const int nk = (int)(nkt - t0 < KT ? nkt - t0 : KT);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (kt >= nk) break;
        const int64_t t = t0 + kt;
        const int64_t kk = t * 32;
        load_k(t + 3, kr[(kt + 3) % 4]);
        auto chain = [&](int qt) {
          f16v acc = {};
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j) acc = E::mfma32x32x16(kr[kt][j], qf[qt][j], acc);
          return acc;
        };
        const int mcol = (int)(t % MT);   // metadata word column of this tile
        f16v acc_next = chain(0);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const f16v acc = acc_next;
          if (qt + 1 < QT) acc_next = chain(qt + 1);
          // acc[i] = S[query l32][key kk + 8(i/4) + 4 half + i%4]
          const int64_t qi = q_wave + qt * 32 + l32;
          uint32_t mword = 0;   // nibble of group 2gi+half at bits 8gi + 4half
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const f2 x01 = {acc[4 * gi] * scale, acc[4 * gi + 1] * scale};
            const f2 x23 = {acc[4 * gi + 2] * scale, acc[4 * gi + 3] * scale};
            const uint32_t p01 = E::pack2(x01);
            const uint32_t p23 = E::pack2(x23);
            if (DENSE && qi < Lq) {
              const u2 pk = {p01, p23};
              *reinterpret_cast<u2*>(S_b + qi * Lk + kk + 8 * gi + 4 * half) = pk;
            }
            uint32_t kept;
            const uint32_t code = select_2of4_keys(p01, p23, kept);
            if constexpr (RMAX && !BF) rmx[qt] = __builtin_elementwise_max(rmx[qt], __builtin_bit_cast(hh2, kept));
            if constexpr (RMAX && BF) rmf[qt] = fmaxf(rmf[qt], fmaxf(E::lo(kept), E::hi(kept)));
            // kept pair of group (kk + 8gi + 4half)/4 -> value position kt*16 + 4gi + 2half
            *reinterpret_cast<uint32_t*>(sv + (qt * 32 + l32) * VP + (kt * 16 + 4 * gi + 2 * half) * 2) = kept;
            mword |= code << (8 * gi + 4 * half);
          }
          mword |= (uint32_t)__shfl_xor((int)mword, 32);
          if (!half) *reinterpret_cast<uint32_t*>(sm + (qt * 32 + l32) * MP + mcol * 4) = mword;
        }
      }
      // Every K tile requested so far (up to 3 tiles ahead) has arrived before the flush is
      // issued: waiting for a load issued after a store must wait for the store too (loads
      // and stores share one counter and may complete out of order), so a wait after the
      // flush would drain it. Waiting here instead leaves the next tiles nothing to wait for
      // until the flush is old. (vmcnt(0), other counters untouched)
      __builtin_amdgcn_s_waitcnt(0x0F70);
      // ---- values: the 4 staged tiles of every row as one 128-byte line. Every staged
      // chunk is read first (the reads stay inside the wave's buffer) and then stored, so
      // the LDS latency is paid once per flush, not once per store.
      {
        u4 vv[QT][4];
        const int ch = lane & 7;               // 16-byte chunk = 8 kept values
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[qt][i] = *reinterpret_cast<const u4*>(sv + (qt * 32 + 8 * i + (lane >> 3)) * VP + ch * 16);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t qi = q_wave + qt * 32 + 8 * i + (lane >> 3);
            if (ch < 2 * nk && qi < Lq)
              __builtin_nontemporal_store(vv[qt][i], reinterpret_cast<u4*>(vals_b + qi * (Lk >> 1) + t0 * 16 + ch * 8));
          }
        }
      }
      // ---- metadata: every 32 tiles (or at the end) the staged words of every row
      const int64_t tend = t0 + nk;   // tiles done
      if (tend % MT == 0 || tend == nkt) {
        const int64_t m0 = (tend - 1) / MT * MT;   // first tile of this metadata line
        const int nw = (int)(tend - m0);           // 4-byte words staged per row
        const int ch = lane & 7;               // 16-byte chunk = 4 words = 4 key tiles
        u4 mm[QT][4];                          // all staged chunks first, as for the values
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mm[qt][i] = *reinterpret_cast<const u4*>(sm + (qt * 32 + 8 * i + (lane >> 3)) * MP + ch * 16);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t qi = q_wave + qt * 32 + 8 * i + (lane >> 3);
            if (qi < Lq) {
              uint8_t* dst = meta_b + qi * (Lk >> 3) + m0 * 4 + ch * 16;
              if (4 * ch + 4 <= nw && (Lk & 127) == 0) {
                __builtin_nontemporal_store(mm[qt][i], reinterpret_cast<u4*>(dst));
              } else {
#pragma unroll
                for (int w = 0; w < 4; ++w)
                  if (4 * ch + w < nw) reinterpret_cast<uint32_t*>(dst)[w] = mm[qt][i][w];
              }
            }
          }
        }
      }
    }
    if constexpr (RMAX) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float m = BF ? rmf[qt] : fmaxf((float)rmx[qt][0], (float)rmx[qt][1]);
        m = fmaxf(m, __shfl_xor(m, 32));   // lanes l and l+32 hold the two halves of a row
        const int64_t qi = q_wave + qt * 32 + l32;
        if (!half && qi < Lq) rowmax[b * Lq + qi] = m;
      }
    }
  }
}

// Row softmax over kept values, one wave per row. Rows of up to 64*8*CH elements stay in
// registers (one read, one write); longer rows are streamed three times. BF: bf16 values.
// Six waves per SIMD (at most 85 registers; fp16 spills two): more rows in flight per CU,
// measured 420 -> 353 us on 64 x 4096 rows of 2048 fp16 values (eight waves spill ~45).
template <int CH, bool BF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6)))
k_softmax_rows(uint16_t* __restrict__ vals, int64_t rows, int64_t kept, int64_t ld, int vec) {
  using E = Elem<BF>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint16_t* v = vals + row * ld;
  float mx = -__builtin_inff();
  if (vec && kept <= 64 * 8 * CH) {
    h8 x[CH];   // 16-bit containers of either type
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 8;
      if (e < kept) {
        x[c] = __builtin_nontemporal_load(reinterpret_cast<const h8*>(v + e));
#pragma unroll
        for (int t = 0; t < 8; ++t) mx = fmaxf(mx, E::widen(f16_bits(x[c][t])));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
    float ex[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        ex[c][t] = e < kept ? __expf(E::widen(f16_bits(x[c][t])) - mx) : 0.f;
        sum += ex[c][t];
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 8;
      if (e < kept) {
        u4 o;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = E::pack2(f2{ex[c][2 * t] * inv, ex[c][2 * t + 1] * inv});
        __builtin_nontemporal_store(o, reinterpret_cast<u4*>(v + e));
      }
    }
    return;
  }
  for (int64_t e = lane; e < kept; e += 64) mx = fmaxf(mx, E::widen(v[e]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.f;
  for (int64_t e = lane; e < kept; e += 64) sum += __expf(E::widen(v[e]) - mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = 1.0f / sum;
  for (int64_t e = lane; e < kept; e += 64) v[e] = E::narrow(__expf(E::widen(v[e]) - mx) * inv);
}

template <int D, int QT, bool DENSE, bool RMAX, bool BF>
static hipError_t launch_sddmm_cfg1(const uint16_t* q, const uint16_t* k, int64_t batch, int64_t Lq,
                                   int64_t Lk, float scale, uint16_t* vv, uint16_t* mm, uint16_t* ss,
                                   float* rmax, hipStream_t stream) {
  using Cfg = SddmmCfg<D, QT>;
  const int64_t qblocks = (Lq + Cfg::kQueries - 1) / Cfg::kQueries;
  const int64_t total = qblocks * batch;
  const int remap = total % 8 == 0 && total <= 0x7FFFFFFF;
  const dim3 grid = remap ? dim3((unsigned)total) : dim3((unsigned)qblocks, (unsigned)(batch < 65535 ? batch : 65535));
  auto kern = k_sddmm_prune<D, QT, DENSE, RMAX, BF>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, Cfg::kLds)) return e;
  hipLaunchKernelGGL(kern, grid, dim3(64 * Cfg::kWaves), Cfg::kLds, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax,
                     remap);
  return hipGetLastError();
}
template <int D, int QT, bool BF>
static hipError_t launch_sddmm_cfg(const uint16_t* q, const uint16_t* k, int64_t batch, int64_t Lq,
                                   int64_t Lk, float scale, uint16_t* vv, uint16_t* mm, uint16_t* ss,
                                   float* rmax, hipStream_t stream) {
  if (ss && rmax) return launch_sddmm_cfg1<D, QT, true, true, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
  if (ss) return launch_sddmm_cfg1<D, QT, true, false, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, nullptr, stream);
  if (rmax) return launch_sddmm_cfg1<D, QT, false, true, BF>(q, k, batch, Lq, Lk, scale, vv, mm, nullptr, rmax, stream);
  return launch_sddmm_cfg1<D, QT, false, false, BF>(q, k, batch, Lq, Lk, scale, vv, mm, nullptr, nullptr, stream);
}

template <bool BF>
static hipError_t launch_sddmm_d(const uint16_t* q, const uint16_t* k, int64_t batch, int64_t Lq,
                                 int64_t Lk, int64_t d, float scale, uint16_t* vv, uint16_t* mm,
                                 uint16_t* ss, float* rmax, hipStream_t stream) {
  switch (d) {
    case 16: return launch_sddmm_cfg<16, 2, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
    case 32: return launch_sddmm_cfg<32, 2, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
    case 64: return launch_sddmm_cfg<64, 2, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
    default: return launch_sddmm_cfg<128, 1, BF>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
  }
}

hipError_t launch_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                 int64_t Lk, int64_t d, float scale, void* values, void* meta,
                                 void* S_dense, float* row_max, bool bf16, hipStream_t stream) {
  const uint16_t* q = (const uint16_t*)Q;
  const uint16_t* k = (const uint16_t*)Kmat;
  uint16_t* vv = (uint16_t*)values;
  uint16_t* mm = (uint16_t*)meta;
  uint16_t* ss = (uint16_t*)S_dense;
  if (bf16) return launch_sddmm_d<true>(q, k, batch, Lq, Lk, d, scale, vv, mm, ss, row_max, stream);
  return launch_sddmm_d<false>(q, k, batch, Lq, Lk, d, scale, vv, mm, ss, row_max, stream);
}

hipError_t launch_softmax_nm_rows(void* values, int64_t rows, int64_t kept, int64_t ld, bool bf16,
                                  hipStream_t stream) {
  const int vec = (kept % 8 == 0) && (ld % 8 == 0);
  const int64_t blocks = (rows + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL((k_softmax_rows<8, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint16_t*)values, rows, kept, ld, vec);
  else
    hipLaunchKernelGGL((k_softmax_rows<8, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint16_t*)values, rows, kept, ld, vec);
  return hipGetLastError();
}

}  // namespace snm
