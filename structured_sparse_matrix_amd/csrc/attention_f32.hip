// 1:2 dynamic attention on fp32 scores ("Dynamic N:M fine-grained structured sparse
// attention mechanism on GPUs", Sec. 1 and Fig. 1-3: the mechanism at 1:2; Sec. 4.2: 32-bit
// data is pruned one of every two 4-byte elements, and its 4-bit metadata codes are 0x4 for
// the first element of the pair and 0xe for the second, four codes per 16-bit word).
//
// This architecture has no sparse matrix instruction for 32-bit data (and no tf32 unit), so
// both products run on the dense fp32 matrix core (v_mfma_f32_32x32x2_f32, full fp32
// products): the SDDMM prunes in its epilogue as the 16-bit kernel does, and the product
// with V expands each kept value into its pair in registers. The 1:2 format halves the bytes
// of the score matrix; the flops are those of the dense products, so these kernels are bound
// by the fp32 matrix core rather than by HBM.
//
//   k_sddmm_1of2_f32   S = fp32((Q K^T) * scale), pruned 1:2 along the keys.
//   k_softmax_rows_f32 row softmax over the kept values, in place.
//   k_spmm_1of2_f32    Y = decode(P) * B, optionally with the softmax of the kept scores
//                      applied inside (the fused variant).
#include "device_common.hpp"
#include "launch.hpp"

namespace snm {

// v_mfma_f32_32x32x2_f32: D(32x32) += A(32x2) * B(2x32), one fp32 operand per lane.
//   A: row l % 32, k = l / 32.  B: column l % 32, k = l / 32.
//   D: column l % 32, element r holds row 8 (r / 4) + 4 (l / 32) + r % 4.
__device__ __forceinline__ f16v mfma32x32x2(float a, float b, const f16v& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 1:2 of a pair by magnitude: the second element is kept only if its magnitude (bits
// without the sign) is strictly larger, so on a tie the first stays.
__device__ __forceinline__ bool keep_second(float x0, float x1) {
  return (__builtin_bit_cast(uint32_t, x1) & 0x7FFFFFFFu) > (__builtin_bit_cast(uint32_t, x0) & 0x7FFFFFFFu);
}

// ---------------------------------------------------------------------------------------
// SDDMM-prune. Workgroup: 8 waves (two per SIMD), each owning 32 queries and walking all
// keys in tiles of 32. As in the 16-bit kernel the product is formed transposed
// (S^T = K Q^T), so a lane holds four consecutive keys of one query per 4 accumulators:
// two 1:2 pairs. The reduction index k of step j and lane half h is d = h D/2 + j, so a
// lane reads its query's and key's halves of d as contiguous 16-byte pieces.
//   * values leave every 2 key tiles (2 x 16 kept fp32 = one 128-byte line per query row),
//     metadata every 16 key tiles (16 x 8 bytes = one line per row), as non-temporal
//     (streaming) stores;
//   * the key tile t + 1 is loaded while tile t is multiplied (for D = 128, where two key
//     tiles do not fit in the register file beside the queries, tile t is loaded just
//     before use and the second wave of the SIMD covers the latency).
template <int D>
struct Sddmm12Cfg {
  static constexpr int kWaves = 8;
  static constexpr int KH = D / 2;        // MFMA steps per key tile
  static constexpr int RING = D <= 64 ? 2 : 1;   // key tiles held in registers
  static constexpr int KT = 2;            // key tiles per values flush
  static constexpr int MT = 16;           // key tiles per metadata flush
  static constexpr int VP = 144;          // staged value bytes per query row
  static constexpr int MP = 144;          // staged metadata bytes per query row
  static constexpr int kWaveV = 32 * VP;
  static constexpr int kWaveM = 32 * MP;
  static constexpr int kLds = kWaves * (kWaveV + kWaveM);
  static constexpr int kQueries = kWaves * 32;
};

template <int D, bool DENSE, bool RMAX>
__global__ void __launch_bounds__(512)
k_sddmm_1of2_f32(const float* __restrict__ Q, const float* __restrict__ Km, int64_t batch,
                 int64_t Lq, int64_t Lk, float scale, float* __restrict__ values,
                 uint8_t* __restrict__ meta, float* __restrict__ S, float* __restrict__ rowmax,
                 int xcd_remap) {
  using Cfg = Sddmm12Cfg<D>;
  constexpr int KH = Cfg::KH, KT = Cfg::KT, MT = Cfg::MT, VP = Cfg::VP, MP = Cfg::MP;
  constexpr int RING = Cfg::RING;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  uint8_t* const sv = smem + wave * Cfg::kWaveV;
  uint8_t* const sm = smem + Cfg::kWaves * Cfg::kWaveV + wave * Cfg::kWaveM;
  // workgroup -> (query block, batch entry); with xcd_remap the one-dimensional grid is
  // numbered so that one XCD's workgroups take consecutive query blocks of the same batch
  // entries and fetch each entry's key tiles into that XCD's L2 once
  int64_t qblk = blockIdx.x, b0 = blockIdx.y, bstep = gridDim.y;
  if (xcd_remap) {
    const int64_t qblocks = (Lq + Cfg::kQueries - 1) / Cfg::kQueries;
    const int64_t L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    b0 = L / qblocks;
    qblk = L - b0 * qblocks;
    bstep = batch;
  }
  const int64_t q_wave = qblk * Cfg::kQueries + (int64_t)wave * 32;
  const int64_t nkt = Lk >> 5;

  for (int64_t b = b0; b < batch; b += bstep) {
    if (q_wave >= Lq) break;   // uniform per wave; the kernel has no barriers
    const float* Qb = Q + b * Lq * D;
    const float* Kb = Km + b * Lk * D;
    float* vals_b = values + b * Lq * (Lk >> 1);
    uint8_t* meta_b = meta + b * Lq * (Lk >> 2);
    float* S_b = DENSE ? S + b * Lq * Lk : nullptr;
    const int64_t qi = q_wave + l32;

    f4 qf[KH / 4];   // Q^T operand: column = query, k = d = half*KH + j
#pragma unroll
    for (int j = 0; j < KH / 4; ++j) {
      f4 v = {};
      if (qi < Lq) v = *reinterpret_cast<const f4*>(Qb + qi * D + half * KH + 4 * j);
      qf[j] = v;
    }
    f4 kr[RING][KH / 4];
    auto load_k = [&](int64_t t, f4 (&kf)[KH / 4]) {
      if (t < nkt) {
#pragma unroll
        for (int j = 0; j < KH / 4; ++j)
          kf[j] = *reinterpret_cast<const f4*>(Kb + (t * 32 + l32) * D + half * KH + 4 * j);
      }
    };
    if (RING == 2) load_k(0, kr[0]);
    float rmf = -__builtin_inff();

    for (int64_t t0 = 0; t0 < nkt; t0 += KT) {
      const int nk = (int)(nkt - t0 < KT ? nkt - t0 : KT);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (kt >= nk) break;
        const int64_t t = t0 + kt;
        const int64_t kk = t * 32;
        if (RING == 2) load_k(t + 1, kr[(kt + 1) % RING]);   // t0 is even: tile t is in slot kt % 2
        else load_k(t, kr[0]);
        const int slot = kt % RING;
        f16v acc = {};
#pragma unroll
        for (int j = 0; j < KH / 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma32x32x2(kr[slot][j][e], qf[j][e], acc);
        // acc[i] * scale = S[query l32][key kk + 8(i/4) + 4 half + i%4]
        uint32_t mb = 0;   // byte gi: the codes of pairs (kk + 8gi + 4half)/2 + {0, 1}
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const float x0 = acc[4 * gi] * scale, x1 = acc[4 * gi + 1] * scale;
          const float x2 = acc[4 * gi + 2] * scale, x3 = acc[4 * gi + 3] * scale;
          if (DENSE && qi < Lq) *reinterpret_cast<f4*>(S_b + qi * Lk + kk + 8 * gi + 4 * half) = f4{x0, x1, x2, x3};
          const bool s01 = keep_second(x0, x1);
          const bool s23 = keep_second(x2, x3);
          const float v0 = s01 ? x1 : x0;
          const float v1 = s23 ? x3 : x2;
          if constexpr (RMAX) rmf = fmaxf(rmf, fmaxf(v0, v1));
          // kept values of the pairs -> positions kt*16 + 4gi + 2half + {0, 1} of the block
          *reinterpret_cast<f2*>(sv + l32 * VP + (kt * 16 + 4 * gi + 2 * half) * 4) = f2{v0, v1};
          mb |= ((s01 ? 0xEu : 0x4u) | ((s23 ? 0xEu : 0x4u) << 4)) << (8 * gi);
        }
        // the tile's 8 metadata bytes of this row: byte 2gi + half comes from half `half`
        const uint32_t other = (uint32_t)__shfl_xor((int)mb, 32);
        if (!half) {
          const uint32_t w0 = __builtin_amdgcn_perm(other, mb, 0x05010400u);
          const uint32_t w1 = __builtin_amdgcn_perm(other, mb, 0x07030602u);
          *reinterpret_cast<u2*>(sm + l32 * MP + (int)(t % MT) * 8) = u2{w0, w1};
        }
      }
      // ---- values: the staged tiles of every row as one 128-byte line
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + (lane >> 3);
        const int ch = lane & 7;   // 16-byte chunk = 4 kept values
        const int64_t q = q_wave + row;
        if (ch < 4 * nk && q < Lq)
          __builtin_nontemporal_store(*reinterpret_cast<const u4*>(sv + row * VP + ch * 16),
                                      reinterpret_cast<u4*>(vals_b + q * (Lk >> 1) + t0 * 16 + ch * 4));
      }
      // ---- metadata: every MT tiles (or at the end)
      const int64_t tend = t0 + nk;
      if (tend % MT == 0 || tend == nkt) {
        const int64_t m0 = (tend - 1) / MT * MT;
        const int nw = (int)(tend - m0);   // 8-byte tile entries staged per row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + (lane >> 3);
          const int ch = lane & 7;         // 16-byte chunk = 2 tiles
          const int64_t q = q_wave + row;
          if (q < Lq) {
            const uint8_t* src = sm + row * MP + ch * 16;
            uint8_t* dst = meta_b + q * (Lk >> 2) + m0 * 8 + ch * 16;
            if (2 * ch + 2 <= nw && (Lk & 63) == 0) {
              __builtin_nontemporal_store(*reinterpret_cast<const u4*>(src), reinterpret_cast<u4*>(dst));
            } else {
              for (int w = 2 * ch; w < 2 * ch + 2 && w < nw; ++w)
                reinterpret_cast<u2*>(dst)[w - 2 * ch] = reinterpret_cast<const u2*>(src)[w - 2 * ch];
            }
          }
        }
      }
    }
    if constexpr (RMAX) {
      const float m = fmaxf(rmf, __shfl_xor(rmf, 32));
      if (!half && qi < Lq) rowmax[b * Lq + qi] = m;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Row softmax over fp32 kept values, one wave per row; rows of up to 64*4*CH values stay
// in registers, longer rows are streamed three times.
template <int CH>
__global__ void __launch_bounds__(256)
k_softmax_rows_f32(float* __restrict__ vals, int64_t rows, int64_t kept, int64_t ld, int vec) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float* v = vals + row * ld;
  float mx = -__builtin_inff();
  if (vec && kept <= 64 * 4 * CH) {
    f4 x[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 4;
      if (e < kept) {
        x[c] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(v + e));
        mx = fmaxf(mx, fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3])));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[c][t] = e < kept ? __expf(x[c][t] - mx) : 0.f;
        sum += x[c][t];
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 4;
      if (e < kept) __builtin_nontemporal_store(x[c] * inv, reinterpret_cast<f4*>(v + e));
    }
    return;
  }
  for (int64_t e = lane; e < kept; e += 64) mx = fmaxf(mx, v[e]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.f;
  for (int64_t e = lane; e < kept; e += 64) sum += __expf(v[e] - mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = 1.0f / sum;
  for (int64_t e = lane; e < kept; e += 64) v[e] = __expf(v[e] - mx) * inv;
}

// ---------------------------------------------------------------------------------------
// Y = decode(P) * B for a 1:2 fp32 operand P (R x K) and row-major fp32 B (K x C).
// Workgroup: 4 waves x 32 rows = 128 rows, 64 output columns (two 32-column MFMA tiles per
// wave). Stages of 32 positions (16 pairs): B's 32 x 64 tile goes through LDS (double
// buffered, one barrier per stage); each lane reads its row's 16 kept values and 8 metadata
// bytes of the stage directly. For the pair p of a step, the lane of half h feeds
// A[row][2p + h] = the kept value if it sits at position h of the pair, else 0.
// SMAX: P holds scores; each kept value v enters as exp(v - row_max) (fp32), the lane keeps
// the fp32 sum of its row's exponentials, and the epilogue divides by it.
struct Spmm12Args {
  const float* values;
  const uint8_t* meta;
  const float* B;
  float* Y;
  const float* rowmax;
  int64_t R, K, C, ldb, ldy;
  int64_t stride_values, stride_meta, stride_B, stride_Y, stride_rowmax;
  int64_t n_row_tiles, n_col_tiles;
};

constexpr int kS12Pitch = 68;   // floats per staged B row (64 + 4: rows 2p, 2p + 1 apart in banks)

template <bool SMAX>
__global__ void __launch_bounds__(256)
k_spmm_1of2_f32(Spmm12Args a) {
  __shared__ __align__(16) float vb[2][32 * kS12Pitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t tiles = a.n_row_tiles * a.n_col_tiles;
  int64_t L = blockIdx.x;   // XCD-aware: one XCD's workgroups take consecutive tiles (same batch entries)
  if ((gridDim.x & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t bt = L / tiles;
  const int64_t rem = L - bt * tiles;
  const int64_t ct = rem / a.n_row_tiles;
  const int64_t rt = rem - ct * a.n_row_tiles;
  const int64_t row0 = rt * 128, col0 = ct * 64;

  const float* __restrict__ vals = a.values + bt * a.stride_values;
  const uint8_t* __restrict__ meta = a.meta + bt * a.stride_meta;
  const float* __restrict__ Bm = a.B + bt * a.stride_B;
  float* __restrict__ Y = a.Y + bt * a.stride_Y;
  const int64_t r = row0 + wave * 32 + l32;
  const int64_t rc = r < a.R ? r : a.R - 1;
  const float* arow = vals + rc * (a.K >> 1);
  const uint8_t* mrow = meta + rc * (a.K >> 2);
  const int64_t nst = a.K >> 5;

  constexpr float kLog2e = 1.4426950408889634f;
  float mx2 = 0.f, rsum = 0.f;
  if constexpr (SMAX) mx2 = a.rowmax[bt * a.stride_rowmax + rc] * kLog2e;

  // B stage: 32 rows x 64 columns = 512 chunks of 4 floats, two per thread
  f4 bst[2];
  auto load_b = [&](int64_t s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int br = c >> 4, bc = (c & 15) * 4;
      f4 v = {};
      if (col0 + bc < a.C) v = *reinterpret_cast<const f4*>(Bm + (s * 32 + br) * a.ldb + col0 + bc);
      bst[i] = v;
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<f4*>(&vb[buf][(c >> 4) * kS12Pitch + (c & 15) * 4]) = bst[i];
    }
  };
  f4 av[2][4];   // 16 kept values of the stage, two stages in flight
  u2 mv[2];      // their 16 codes (8 bytes)
  auto load_a = [&](int64_t s, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) av[buf][j] = *reinterpret_cast<const f4*>(arow + s * 16 + 4 * j);
    mv[buf] = *reinterpret_cast<const u2*>(mrow + s * 8);
  };

  f16v acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;

  if (nst > 0) {
    load_b(0);
    load_a(0, 0);
    store_b(0);
  }
  __syncthreads();
  for (int64_t s = 0; s < nst; ++s) {
    const int cur = (int)(s & 1);
    if (s + 1 < nst) {
      load_b(s + 1);
      load_a(s + 1, cur ^ 1);
    }
    const float* vbs = vb[cur];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t code = (mv[cur][p >> 3] >> (4 * (p & 7))) & 0xFu;
      const int slot = (int)((code >> 1) & 1u);   // 0x4 -> 0 (first), 0xe -> 1 (second)
      float v = av[cur][p >> 2][p & 3];
      if constexpr (SMAX) {
        v = __builtin_amdgcn_exp2f(__builtin_fmaf(v, kLog2e, -mx2));
        if (slot == h) rsum += v;
      }
      const float x = slot == h ? v : 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[c] = mfma32x32x2(x, vbs[(2 * p + h) * kS12Pitch + c * 32 + l32], acc[c]);
    }
    if (s + 1 < nst) store_b(cur ^ 1);
    __syncthreads();
  }

  float inv[16];
  if constexpr (SMAX) {
    const float rinv = 1.0f / (rsum + __shfl_xor(rsum, 32));
#pragma unroll
    for (int i = 0; i < 16; ++i) inv[i] = __shfl(rinv, 8 * (i >> 2) + 4 * h + (i & 3));
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t col = col0 + c * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t row = row0 + wave * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < a.R && col < a.C) Y[row * a.ldy + col] = SMAX ? acc[c][i] * inv[i] : acc[c][i];
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, bool DENSE, bool RMAX>
static hipError_t launch_sddmm12_cfg(const float* q, const float* k, int64_t batch, int64_t Lq,
                                     int64_t Lk, float scale, float* vv, uint8_t* mm, float* ss,
                                     float* rmax, hipStream_t stream) {
  using Cfg = Sddmm12Cfg<D>;
  const int64_t qblocks = (Lq + Cfg::kQueries - 1) / Cfg::kQueries;
  const int64_t total = qblocks * batch;
  const int remap = total % 8 == 0 && total <= 0x7FFFFFFF;
  const dim3 grid = remap ? dim3((unsigned)total) : dim3((unsigned)qblocks, (unsigned)(batch < 65535 ? batch : 65535));
  auto kern = k_sddmm_1of2_f32<D, DENSE, RMAX>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, Cfg::kLds)) return e;
  hipLaunchKernelGGL(kern, grid, dim3(64 * Cfg::kWaves), Cfg::kLds, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax,
                     remap);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_sddmm12_d(const float* q, const float* k, int64_t batch, int64_t Lq, int64_t Lk,
                                   float scale, float* vv, uint8_t* mm, float* ss, float* rmax,
                                   hipStream_t stream) {
  if (ss && rmax) return launch_sddmm12_cfg<D, true, true>(q, k, batch, Lq, Lk, scale, vv, mm, ss, rmax, stream);
  if (ss) return launch_sddmm12_cfg<D, true, false>(q, k, batch, Lq, Lk, scale, vv, mm, ss, nullptr, stream);
  if (rmax) return launch_sddmm12_cfg<D, false, true>(q, k, batch, Lq, Lk, scale, vv, mm, nullptr, rmax, stream);
  return launch_sddmm12_cfg<D, false, false>(q, k, batch, Lq, Lk, scale, vv, mm, nullptr, nullptr, stream);
}

hipError_t launch_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                       int64_t Lk, int64_t d, float scale, void* values, void* meta,
                                       void* S_dense, float* row_max, hipStream_t stream) {
  const float* q = (const float*)Q;
  const float* k = (const float*)Kmat;
  float* vv = (float*)values;
  uint8_t* mm = (uint8_t*)meta;
  float* ss = (float*)S_dense;
  switch (d) {
    case 16: return launch_sddmm12_d<16>(q, k, batch, Lq, Lk, scale, vv, mm, ss, row_max, stream);
    case 32: return launch_sddmm12_d<32>(q, k, batch, Lq, Lk, scale, vv, mm, ss, row_max, stream);
    case 64: return launch_sddmm12_d<64>(q, k, batch, Lq, Lk, scale, vv, mm, ss, row_max, stream);
    default: return launch_sddmm12_d<128>(q, k, batch, Lq, Lk, scale, vv, mm, ss, row_max, stream);
  }
}

hipError_t launch_softmax_rows_f32(void* values, int64_t rows, int64_t kept, int64_t ld,
                                   hipStream_t stream) {
  const int vec = (kept % 4 == 0) && (ld % 4 == 0);
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL((k_softmax_rows_f32<8>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (float*)values, rows, kept, ld, vec);
  return hipGetLastError();
}

hipError_t launch_spmm_1of2_f32(const void* values, const void* meta, const float* row_max, int64_t R,
                                int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                                int64_t batch, int64_t stride_values, int64_t stride_meta,
                                int64_t stride_row_max, int64_t stride_B, int64_t stride_Y,
                                hipStream_t stream) {
  Spmm12Args a{};
  a.values = (const float*)values;
  a.meta = (const uint8_t*)meta;
  a.B = (const float*)B;
  a.Y = (float*)Y;
  a.rowmax = row_max;
  a.R = R; a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.stride_values = stride_values; a.stride_meta = stride_meta; a.stride_B = stride_B;
  a.stride_Y = stride_Y; a.stride_rowmax = stride_row_max;
  a.n_row_tiles = (R + 127) / 128;
  a.n_col_tiles = (C + 63) / 64;
  const int64_t total = a.n_row_tiles * a.n_col_tiles * (batch < 1 ? 1 : batch);
  if (total == 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (row_max)
    hipLaunchKernelGGL(k_spmm_1of2_f32<true>, dim3((unsigned)total), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_spmm_1of2_f32<false>, dim3((unsigned)total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace snm
