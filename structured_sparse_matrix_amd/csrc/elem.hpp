// The two 16-bit element types of the attention path, fp16 and bf16 ("Dynamic N:M
// fine-grained structured sparse attention mechanism on GPUs", Sec. 4.2: 16-bit data of
// either type is pruned 2:4). They share the sign-and-magnitude bit layout, so the 2:4
// selection on bit patterns, the packed values and the metadata are identical; they
// differ only in how a value widens to fp32, how an fp32 result rounds back (both round
// to nearest even), and which matrix-core instruction multiplies them. Kernels hold either
// type in the fp16 vector registers (h8, h16) as plain bit containers.
#pragma once

#include "device_common.hpp"

namespace snm {

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));

template <bool BF>
struct Elem;

template <>
struct Elem<false> {   // fp16
  static constexpr uint32_t kNegInf2 = 0xFC00FC00u;   // two -inf patterns
  __device__ static __forceinline__ float lo(uint32_t p) { return (float)__builtin_bit_cast(hh2, p)[0]; }
  __device__ static __forceinline__ float hi(uint32_t p) { return (float)__builtin_bit_cast(hh2, p)[1]; }
  __device__ static __forceinline__ float widen(uint16_t b) { return (float)bits_f16(b); }
  // two fp32 values -> packed pair, round to nearest even
  __device__ static __forceinline__ uint32_t pack2(f2 x) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, hh2));
  }
  __device__ static __forceinline__ uint16_t narrow(float x) { return f16_bits((_Float16)x); }
  __device__ static __forceinline__ f16v mfma32x32x16(const h8& a, const h8& b, const f16v& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f16v smfmac32(const h8& a, const h16& b, const f16v& c, uint32_t idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, (int)idx, 0, 0);
  }
  // acc + p.lo + p.hi in fp32 (v_dot2 against (1, 1))
  __device__ static __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(hh2, p), hh2{(_Float16)1.f, (_Float16)1.f}, acc, false);
  }
};

template <>
struct Elem<true> {    // bf16: the upper half of an fp32
  static constexpr uint32_t kNegInf2 = 0xFF80FF80u;
  __device__ static __forceinline__ float lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
  __device__ static __forceinline__ float hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }
  __device__ static __forceinline__ float widen(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
  // v_cvt_pk_bf16_f32: round to nearest even
  __device__ static __forceinline__ uint32_t pack2(f2 x) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2));
  }
  __device__ static __forceinline__ uint16_t narrow(float x) {
    return (uint16_t)(pack2(f2{x, x}) & 0xFFFFu);
  }
  __device__ static __forceinline__ f16v mfma32x32x16(const h8& a, const h8& b, const f16v& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f16v smfmac32(const h8& a, const h16& b, const f16v& c, uint32_t idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf16x16, b), c,
                                                     (int)idx, 0, 0);
  }
  __device__ static __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, p), bf2{(__bf16)1.f, (__bf16)1.f}, acc, false);
  }
};

}  // namespace snm
