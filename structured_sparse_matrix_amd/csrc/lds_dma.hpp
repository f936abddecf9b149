// Asynchronous global -> LDS copies (the gfx950 DMA path) and the explicit waits that go
// with them. Kernels that stage operands through LDS this way count their own outstanding
// vector-memory operations: every load, DMA and store of a wave retires in issue order and
// is counted by one vmcnt counter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snm {

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// All LDS reads of this wave are complete, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Global -> LDS DMA of 16 bytes (or 4 bytes, or 2 bytes zero-extended to a dword) per lane:
// lane l writes LDS bytes [lds_byte + 16 l, +16) (or [lds_byte + 4 l, +4)); lds_byte is
// wave-uniform and goes through M0. dma_s addresses a wave-uniform base (SGPR pair) plus a
// per-lane 32-bit byte offset, dma_v a per-lane 64-bit address. Issued from inline assembly
// on purpose: the compiler's waitcnt pass would otherwise make every later LDS read it
// cannot disambiguate (the transpose reads) wait for all DMA in flight, i.e. drain the
// prefetch ring each stage. Completion is tracked by hand with s_waitcnt vmcnt before the
// barrier that publishes a stage. No "memory" clobber: a DMA writes a ring slot no wave is
// reading, and the waits and barriers that order it are memory-clobbering statements.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is set inside the statement
template <int SIZE>
__device__ __forceinline__ void dma_s(const void* sbase_in, uint32_t voff, uint32_t lds_byte) {
  // the base is wave-uniform by construction; readfirstlane makes that explicit so the
  // operand always lands in an SGPR pair
  // (the builtin returns a signed int: widen through uint32_t, never sign-extend)
  const uint64_t bv = (uint64_t)(uintptr_t)sbase_in;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bv >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bv);
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  const void* sbase = (const void*)(uintptr_t)bu;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0) : "m0");
  else if constexpr (SIZE == 4)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0) : "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(sbase), "s"(m0) : "m0");
}
template <int SIZE>
__device__ __forceinline__ void dma_v(const void* src, uint32_t lds_byte) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" ::"v"(src), "s"(m0) : "m0");
}
#pragma clang diagnostic pop

}  // namespace snm
