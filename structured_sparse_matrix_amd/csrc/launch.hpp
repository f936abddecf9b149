// Host-side launchers of the device kernels (implemented in the .hip files). They assume
// arguments already passed validation and only enqueue work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace snm {

// Raises a kernel's dynamic-LDS limit on the current device, once per device: `done` is the
// launch site's record, bit d for device d (the entry points accept devices 0..63 only).
// hipFuncSetAttribute acts on the current device, so every device a kernel runs on gets its
// own call. Two threads that reach a device's first launch together both set the same
// value, which is harmless; the bit is published only after the call succeeded.
inline hipError_t ensure_lds_limit(std::atomic<uint64_t>& done, const void* kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = (uint64_t)1 << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

hipError_t launch_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, void* values,
                                  void* meta, hipStream_t stream);
hipError_t launch_prune_encode_nm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, void* values_t,
                                        void* meta_t, hipStream_t stream);
hipError_t launch_spmm_nm_tiled(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                int64_t ldy, hipStream_t stream);
// split reduction (plan from splitk_plan); B column-major; workspace as the plan sizes it
hipError_t launch_spmm_nm_tiled_splitk(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                       const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                                       void* workspace, hipStream_t stream);
// the same product with the library's own per-device scratch as the workspace
hipError_t launch_spmm_nm_tiled_splitk_noalloc(const void* values_t, const void* meta_t, int64_t R,
                                               int64_t K, const void* B, int64_t C, int64_t ldb,
                                               void* Y, int64_t ldy, hipStream_t stream);
// A decode product (one product, C <= 32) takes the LDS-ring kernel when B is column-major with
// 16-byte column slices, K % 512 == 0 (operand-major A) or K % 1024 == 0 (canonical A) and
// K <= 8192, unless SNM_FORCE_VARIANT=direct.
bool skinny_ring_selected(int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, bool a_tiled);
hipError_t launch_spmm_nm_tiled_skinny(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                       const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                       int64_t ldy, hipStream_t stream);
// tiled: the row-group interleaved storage of values and m-indices (R % 32 == 0)
hipError_t launch_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                                   void* values, void* midx, void* colloc, bool tiled,
                                   hipStream_t stream);
hipError_t launch_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                          int64_t C, int64_t ldb, int b_layout, void* Y, int64_t ldy, int64_t batch,
                          int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                          int64_t stride_Y, hipStream_t stream);
hipError_t launch_spmm_nm_skinny(const void* values, const void* meta, int64_t R, int64_t K,
                                 const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                                 int64_t ldy, int64_t batch, int64_t stride_values,
                                 int64_t stride_meta, int64_t stride_B, int64_t stride_Y,
                                 hipStream_t stream);
hipError_t launch_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R,
                           int64_t K, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                           int64_t ldy, hipStream_t stream);
// Wide-output SpMM (spmm_wide.hip): row-major B. V > 0 selects V:2:M with column-loc
// gathering (Kc = 4K/M); V == 0 is plain 2:4 (Kc = K), optionally batched.
// supported: the kernel can run the shape (C % 8 == 0, 16-byte B rows, 32-bit offsets);
// eligible: supported and C > 32, where it is the fastest kernel.
bool spmm_wide_supported(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                         int64_t batch, int64_t stride_B);
bool spmm_wide_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                        int64_t batch, int64_t stride_B);
hipError_t launch_spmm_wide(const void* values, const void* meta, const void* colloc, int64_t R,
                            int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb,
                            void* Y, int64_t ldy, int64_t batch, int64_t stride_values,
                            int64_t stride_meta, int64_t stride_B, int64_t stride_Y,
                            hipStream_t stream, bool a_tiled = false);
// Large V:2:M products (spmm_vnm_big.hip): V % 128 == 0, K' = 4K/M a multiple of 128 in
// [256, 12224], C >= 256, C % 8 == 0, 16-byte B rows. One workgroup per CU, 128 x 512 tiles.
bool spmm_vnm_big_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb);
hipError_t launch_spmm_vnm_big(const void* values, const void* meta, const void* colloc, int64_t R,
                               int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                               int64_t ldy, bool a_tiled, hipStream_t stream);
// the same product with 64-row tiles (spmm_vnm_big64.hip): V % 64 == 0
bool spmm_vnm_big64_eligible(int64_t R, int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb);
hipError_t launch_spmm_vnm_big64(const void* values, const void* meta, const void* colloc, int64_t R,
                                 int64_t Kc, int V, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                                 int64_t ldy, bool a_tiled, hipStream_t stream);
// V:2:M product with values and m-indices in the row-group interleaved storage (wide
// kernel only: V % 32 == 0 and the shape rules of spmm_wide_supported)
hipError_t launch_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc,
                                 int64_t R, int64_t K, int V, int M, const void* B, int64_t C,
                                 int64_t ldb, void* Y, int64_t ldy, hipStream_t stream);
// 2:4 SpMM that applies the softmax over each row's kept scores (wide kernel, softmax mode).
hipError_t launch_spmm_nm_softmax(const void* values, const void* meta, const float* row_max,
                                  int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb,
                                  void* Y, int64_t ldy, int64_t batch, int64_t stride_values,
                                  int64_t stride_meta, int64_t stride_row_max, int64_t stride_B,
                                  int64_t stride_Y, bool bf16, hipStream_t stream);
// 2:4 SpMM on bf16 values and B (wide kernel; its support set, row-major B).
hipError_t launch_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K,
                               const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                               int64_t batch, int64_t stride_values, int64_t stride_meta,
                               int64_t stride_B, int64_t stride_Y, hipStream_t stream);
hipError_t launch_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                 int64_t Lk, int64_t d, float scale, void* values, void* meta,
                                 void* S_dense, float* row_max, bool bf16, hipStream_t stream);
// Bitmap (Coruscant) format: encoder passes and the decode-shaped product (bitmap.hip).
hipError_t launch_bitmap_count(const void* A, int64_t R, int64_t K, int64_t lda, uint64_t* bitmaps,
                               uint32_t* offsets, hipStream_t stream);
hipError_t launch_bitmap_values(const void* A, int64_t R, int64_t K, int64_t lda,
                                const uint64_t* bitmaps, const uint32_t* offsets, void* values,
                                hipStream_t stream);
hipError_t launch_spmm_bitmap(const uint64_t* bitmaps, const uint32_t* offsets, const void* values,
                              int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb,
                              int b_layout, void* Y, int64_t ldy, hipStream_t stream);
// Measured ceilings (ceilings.hip): plain streams and matrix-instruction issue loops.
hipError_t launch_ceiling_read(const void* src, int64_t bytes, void* sink, hipStream_t stream);
hipError_t launch_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_ceiling_lds_fill(const void* src, int64_t window_bytes, int64_t workgroups, int64_t iters,
                                   float* out, hipStream_t stream);
hipError_t launch_ceiling_matrix(int sparse, int64_t workgroups, int64_t iters, float* out, hipStream_t stream);
hipError_t launch_softmax_nm_rows(void* values, int64_t rows, int64_t kept, int64_t ld, bool bf16,
                                  hipStream_t stream);
// 1:2 attention on fp32 scores (attention_f32.hip).
hipError_t launch_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                       int64_t Lk, int64_t d, float scale, void* values, void* meta,
                                       void* S_dense, float* row_max, hipStream_t stream);
hipError_t launch_softmax_rows_f32(void* values, int64_t rows, int64_t kept, int64_t ld,
                                   hipStream_t stream);
hipError_t launch_spmm_1of2_f32(const void* values, const void* meta, const float* row_max, int64_t R,
                                int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                                int64_t batch, int64_t stride_values, int64_t stride_meta,
                                int64_t stride_row_max, int64_t stride_B, int64_t stride_Y,
                                hipStream_t stream);

}  // namespace snm
