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
#include "device_common.hpp"
#include "launch.hpp"

namespace snm {

__device__ __forceinline__ uint32_t select_2of4_attn(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                     uint32_t& v0, uint32_t& v1) {
  const uint32_t c0 = ((a0 & 0x7FFFu) << 2) | 3u;
  const uint32_t c1 = ((a1 & 0x7FFFu) << 2) | 2u;
  const uint32_t c2 = ((a2 & 0x7FFFu) << 2) | 1u;
  const uint32_t c3 = ((a3 & 0x7FFFu) << 2) | 0u;
  const uint32_t g01 = c0 > c1, g02 = c0 > c2, g03 = c0 > c3;
  const uint32_t g12 = c1 > c2, g13 = c1 > c3, g23 = c2 > c3;
  const uint32_t r0 = (1u - g01) + (1u - g02) + (1u - g03);
  const uint32_t r1 = g01 + (1u - g12) + (1u - g13);
  const uint32_t r2 = g02 + g12 + (1u - g23);
  const uint32_t r3 = g03 + g13 + g23;
  const uint32_t keep = (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) |
                        ((uint32_t)(r3 < 2) << 3);
  const uint32_t s0 = __builtin_ctz(keep);
  const uint32_t s1 = 31u - __builtin_clz(keep);
  v0 = s0 == 0 ? a0 : (s0 == 1 ? a1 : a2);
  v1 = s1 == 3 ? a3 : (s1 == 2 ? a2 : a1);
  return s0 | (s1 << 2);
}

// Workgroup: 4 waves x QT query tiles of 32 queries; the waves walk the same key tiles
// (32 keys each) so K rows are shared through L1.
template <int D, int QT>
__global__ void __launch_bounds__(256)
k_sddmm_prune(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Km, int64_t batch,
              int64_t Lq, int64_t Lk, float scale, uint16_t* __restrict__ values,
              uint16_t* __restrict__ meta, uint16_t* __restrict__ S) {
  constexpr int KSTEPS = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;          // which 8-wide d slice / which 4-key subgroup
  const int l32 = lane & 31;
  const int64_t q_wave = (int64_t)blockIdx.x * (4 * 32 * QT) + (int64_t)wave * 32 * QT;

  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const uint16_t* Qb = Q + b * Lq * D;
    const uint16_t* Kb = Km + b * Lk * D;
    uint16_t* vals_b = values + b * Lq * (Lk >> 1);
    uint16_t* meta_b = meta + b * Lq * (Lk >> 4);
    uint16_t* S_b = S ? S + b * Lq * Lk : nullptr;

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
    if (q_wave >= Lq) continue;   // whole wave past the end (uniform per wave)

    auto load_k = [&](int64_t k0, h8 (&kf)[KSTEPS]) {
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        kf[j] = *reinterpret_cast<const h8*>(Kb + (k0 + l32) * D + 16 * j + 8 * half);
    };
    h8 kcur[KSTEPS], knext[KSTEPS];
    load_k(0, kcur);
    for (int64_t k0 = 0; k0 < Lk; k0 += 32) {
      if (k0 + 32 < Lk) load_k(k0 + 32, knext);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f16v acc = {};
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) acc = mfma32x32x16(kcur[j], qf[qt][j], acc);
        // acc[i] = S[query l32][key k0 + 8(i/4) + 4 half + i%4]
        const int64_t qi = q_wave + qt * 32 + l32;
        uint32_t out[4];
        uint32_t codes = 0;   // code of this lane's group gi at bits [8 gi, 8 gi + 3]
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = f16_bits(to_f16(acc[4 * gi + e] * scale));
          if (S_b && qi < Lq) {
            u2 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            *reinterpret_cast<u2*>(S_b + qi * Lk + k0 + 8 * gi + 4 * half) = pk;
          }
          uint32_t v0, v1;
          const uint32_t code = select_2of4_attn(h[0], h[1], h[2], h[3], v0, v1);
          out[gi] = v0 | (v1 << 16);
          codes |= code << (8 * gi);
        }
        // Lanes l and l+32 hold the even and odd groups of the 8 groups of this query's
        // 32 keys. Swap so that lane l holds groups 0-3 and lane l+32 groups 4-7.
        const uint32_t send0 = half ? out[0] : out[2];
        const uint32_t send1 = half ? out[1] : out[3];
        const uint32_t recv0 = (uint32_t)__shfl_xor((int)send0, 32);
        const uint32_t recv1 = (uint32_t)__shfl_xor((int)send1, 32);
        const uint32_t pcodes = (uint32_t)__shfl_xor((int)codes, 32);
        u4 o;
        if (!half) { o[0] = out[0]; o[1] = recv0; o[2] = out[1]; o[3] = recv1; }
        else       { o[0] = recv0; o[1] = out[2]; o[2] = recv1; o[3] = out[3]; }
        const uint32_t ev = half ? pcodes : codes;
        const uint32_t od = half ? codes : pcodes;
        const uint32_t sh = half ? 16u : 0u;
        const uint32_t word = ((ev >> sh) & 0xF0Fu) | (((od >> sh) & 0xF0Fu) << 4);
        if (qi < Lq) {
          *reinterpret_cast<u4*>(vals_b + qi * (Lk >> 1) + (k0 >> 1) + 8 * half) = o;
          meta_b[qi * (Lk >> 4) + (k0 >> 4) + half] = (uint16_t)word;
        }
      }
      if (k0 + 32 < Lk) {
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) kcur[j] = knext[j];
      }
    }
  }
}

// Row softmax over kept values, one wave per row. Rows of up to 64*8*CH elements stay in
// registers (one read, one write); longer rows are streamed three times.
template <int CH>
__global__ void __launch_bounds__(256)
k_softmax_rows(uint16_t* __restrict__ vals, int64_t rows, int64_t kept, int64_t ld, int vec) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint16_t* v = vals + row * ld;
  float mx = -__builtin_inff();
  if (vec && kept <= 64 * 8 * CH) {
    h8 x[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t e = ((int64_t)c * 64 + lane) * 8;
      if (e < kept) {
        x[c] = *reinterpret_cast<const h8*>(v + e);
#pragma unroll
        for (int t = 0; t < 8; ++t) mx = fmaxf(mx, (float)x[c][t]);
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
        ex[c][t] = e < kept ? __expf((float)x[c][t] - mx) : 0.f;
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
        h8 o;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = to_f16(ex[c][t] * inv);
        *reinterpret_cast<h8*>(v + e) = o;
      }
    }
    return;
  }
  for (int64_t e = lane; e < kept; e += 64) mx = fmaxf(mx, (float)bits_f16(v[e]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.f;
  for (int64_t e = lane; e < kept; e += 64) sum += __expf((float)bits_f16(v[e]) - mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = 1.0f / sum;
  for (int64_t e = lane; e < kept; e += 64) v[e] = f16_bits(to_f16(__expf((float)bits_f16(v[e]) - mx) * inv));
}

hipError_t launch_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                 int64_t Lk, int64_t d, float scale, void* values, void* meta,
                                 void* S_dense, hipStream_t stream) {
  constexpr int QT = 2;
  const int64_t qblocks = (Lq + 4 * 32 * QT - 1) / (4 * 32 * QT);
  const dim3 grid((unsigned)qblocks, (unsigned)(batch < 65535 ? batch : 65535));
  const uint16_t* q = (const uint16_t*)Q;
  const uint16_t* k = (const uint16_t*)Kmat;
  uint16_t* vv = (uint16_t*)values;
  uint16_t* mm = (uint16_t*)meta;
  uint16_t* ss = (uint16_t*)S_dense;
  switch (d) {
    case 16: hipLaunchKernelGGL((k_sddmm_prune<16, QT>), grid, dim3(256), 0, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss); break;
    case 32: hipLaunchKernelGGL((k_sddmm_prune<32, QT>), grid, dim3(256), 0, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss); break;
    case 64: hipLaunchKernelGGL((k_sddmm_prune<64, QT>), grid, dim3(256), 0, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss); break;
    default: hipLaunchKernelGGL((k_sddmm_prune<128, QT>), grid, dim3(256), 0, stream, q, k, batch, Lq, Lk, scale, vv, mm, ss); break;
  }
  return hipGetLastError();
}

hipError_t launch_softmax_nm_rows(void* values, int64_t rows, int64_t kept, int64_t ld,
                                  hipStream_t stream) {
  const int vec = (kept % 8 == 0) && (ld % 8 == 0);
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL((k_softmax_rows<8>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (uint16_t*)values, rows, kept, ld, vec);
  return hipGetLastError();
}

}  // namespace snm
