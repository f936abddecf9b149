// Device-side building blocks for gfx950 (CDNA4): vector types, the sparse / dense
// matrix-core instructions with the lane layouts measured on MI355X, and the LDS
// transpose read. Every kernel of libsnm includes this header; nothing here is shared
// with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snm {

typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// v_smfmac_f32_16x16x64_f16: D(16x16, fp32) += A(16x64, 2:4 sparse along k) * B(64x16).
// Lane layout (lane l, quarter q = l / 16, i = l % 16):
//   A: row i; 8 stored values covering dense k = 16q + [0, 16) = four groups of four;
//      stored value j belongs to group j / 2 and its slot is bits [2j, 2j+1] of the
//      16-bit index word -- exactly one canonical 2:4 metadata word. `abid` picks the
//      low (0) or high (1) 16 bits of the 32-bit index register.
//   B: column i; element e < 8 holds k = 8q + e, element e >= 8 holds k = 32 + 8q + e - 8.
//   D: column i; element r holds row 4q + r.
// So A quarter p pairs with B quarters 2(p%2), 2(p%2)+1, elements 8(p/2)..8(p/2)+7.
// ---------------------------------------------------------------------------------------
template <int ABID>
__device__ __forceinline__ f4 smfmac16(const h8& a, const h16& b, const f4& c, uint32_t idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, (int)idx, 0, ABID);
}

// v_mfma_f32_32x32x16_f16: D(32x32) += A(32x16) * B(16x32).
//   A: row l % 32, k = 8 (l / 32) + [0, 8).  B: column l % 32, same k.
//   D: column l % 32, element r holds row 8 (r / 4) + 4 (l / 32) + r % 4.
__device__ __forceinline__ f16v mfma32x32x16(const h8& a, const h8& b, const f16v& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16. Within each group of 16 lanes, lane i receives element (i % 4) of
// the 8 bytes read by lane 4r + i / 4, for r = 0..3. With lane L pointing at
// &T[row0 + L / 4][c0 + 4 (L % 4)] of a row-major fp16 tile T, lane i therefore receives
// T[row0 + r][c0 + i] for r = 0..3: four consecutive rows of one column.
__device__ __forceinline__ h4 lds_read_tr16(uint32_t lds_byte_addr) {
  typedef __fp16 fp4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) fp4 lds_fp4;
  lds_fp4* p = (lds_fp4*)(uintptr_t)lds_byte_addr;
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
}

// Global -> LDS DMA of 16 bytes per active lane: lane l writes LDS bytes
// [lds_byte + 16 l, + 16) from its own 64-bit address (global_load_lds_dwordx4; lds_byte is
// wave-uniform and goes through M0). Inactive lanes neither read nor write. Completion is
// tracked with s_waitcnt vmcnt by the caller; from inline assembly so that the compiler's
// waitcnt pass does not make unrelated LDS reads wait for it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is set inside the statement
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_byte) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object (address space 3 offset).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ uint16_t f16_bits(_Float16 x) { return __builtin_bit_cast(uint16_t, x); }
__device__ __forceinline__ _Float16 bits_f16(uint16_t x) { return __builtin_bit_cast(_Float16, x); }

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default rounding mode).
__device__ __forceinline__ _Float16 to_f16(float x) { return (_Float16)x; }

// 2 of 4 by magnitude on composite keys: key_i = |h_i| << 16 | t_i, where |h| is the fp16
// pattern without its sign (orders like the magnitude; NaN > Inf > finite) and the tie
// field t = 0xFFFF, 0xFF00, 0x00FF, 0x0000 for slots 0..3 decreases with the slot, so a
// larger key means a larger magnitude or, on equal magnitudes, a lower slot -- the
// lower-slot-wins tie rule. Every key is one byte permute of the sign-cleared pair (the
// tie bytes are the permute's constant 0x00 / 0xFF bytes), and bits 8..7 of a key are
// 3 - slot. The two largest keys are the kept slots (a 6-operation max/min network instead
// of pairwise ranks). Inputs are the group's four fp16 patterns packed in pairs
// (p01 = h0 | h1 << 16, p23 = h2 | h3 << 16); the kept pair, ascending slot order, comes
// back packed the same way, gathered with one byte permute. Returns the group's code
// s0 | s1 << 2 (s0 < s1, the kept slots).
__device__ __forceinline__ uint32_t select_2of4_keys(uint32_t p01, uint32_t p23, uint32_t& kept) {
  const uint32_t a01 = p01 & 0x7FFF7FFFu, a23 = p23 & 0x7FFF7FFFu;
  // permute selectors: byte i of the result is byte sel_i of the pair (0..3), or 0x00
  // (0x0C) or 0xFF (0x0D)
  const uint32_t c0 = __builtin_amdgcn_perm(a01, a01, 0x01000D0Du);   // |h0| : FF FF
  const uint32_t c1 = __builtin_amdgcn_perm(a01, a01, 0x03020D0Cu);   // |h1| : FF 00
  const uint32_t c2 = __builtin_amdgcn_perm(a23, a23, 0x01000C0Du);   // |h2| : 00 FF
  const uint32_t c3 = a23 & 0xFFFF0000u;                              // |h3| : 00 00
  const uint32_t m01 = c0 > c1 ? c0 : c1, n01 = c0 > c1 ? c1 : c0;
  const uint32_t m23 = c2 > c3 ? c2 : c3, n23 = c2 > c3 ? c3 : c2;
  const uint32_t t1 = m01 > m23 ? m01 : m23;
  const uint32_t lo_m = m01 > m23 ? m23 : m01;
  const uint32_t hi_n = n01 > n23 ? n01 : n23;
  const uint32_t t2 = lo_m > hi_n ? lo_m : hi_n;
  const uint32_t x = (t1 >> 7) & 3u, y = (t2 >> 7) & 3u;   // 3 - slot of the two kept entries
  const uint32_t hi = x > y ? x : y, lo = x > y ? y : x;   // 3 - s0, 3 - s1
  // selector bytes 2 s0, 2 s0 + 1, 2 s1, 2 s1 + 1 of {p23 : p01}:
  // (s0 | s1 << 16) * 0x0202 + 0x01000100 with s = 3 - (3 - s)
  kept = __builtin_amdgcn_perm(p23, p01, 0x07060706u - (hi | (lo << 16)) * 0x0202u);
  return 15u - (hi | (lo << 2));
}

}  // namespace snm
