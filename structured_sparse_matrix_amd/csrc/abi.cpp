// extern "C" entry points of libsnm: validate on the host (validate.cpp), check once per
// device that it is a gfx950, then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "launch.hpp"
#include "snm.h"
#include "snm_ceilings.h"
#include "validate.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SNM_E_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SNM_E_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? SNM_OK : SNM_E_DEVICE;
}

snm_status launched(hipError_t e) { return e == hipSuccess ? SNM_OK : SNM_E_LAUNCH; }

// status codes of the host checks (plain ints) as the boundary's enum
snm_status st(int s) { return (snm_status)s; }

// the patterns implemented: n = 2 of m = 4 (N:M); n = 2 of m (V:N:M, m checked with v)
bool is_nm_2_4(int n, int m) { return n == 2 && m == 4; }

}  // namespace

extern "C" {

int snm_abi_version(void) { return 1; }

const char* snm_status_string(snm_status status) {
  switch (status) {
    case SNM_OK: return "ok";
    case SNM_E_NULL: return "a required pointer is NULL";
    case SNM_E_SHAPE: return "invalid size, leading dimension or stride";
    case SNM_E_ALIGN: return "pointer or leading dimension breaks the 16-byte alignment rule";
    case SNM_E_UNSUPPORTED: return "unsupported pattern parameters";
    case SNM_E_DEVICE: return "current HIP device is not gfx950";
    case SNM_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

snm_status snm_nm_sizes(int64_t R, int64_t K, int n, int m, int64_t* values_elems, int64_t* meta_bytes) {
  if (!is_nm_2_4(n, m)) return SNM_E_UNSUPPORTED;
  int s = snm::check_nm_sizes(R, K);
  if (s != SNM_OK) return st(s);
  if (!values_elems || !meta_bytes) return st(SNM_E_NULL);
  *values_elems = R * (K / 2);
  *meta_bytes = R * (K / 8);
  return st(SNM_OK);
}

snm_status snm_vnm_sizes(int64_t R, int64_t K, int V, int N, int M, int64_t* values_elems,
                         int64_t* midx_bytes, int64_t* colloc_bytes) {
  if (N != 2) return SNM_E_UNSUPPORTED;
  int s = snm::check_vnm_sizes(R, K, V, M);
  if (s != SNM_OK) return st(s);
  if (!values_elems || !midx_bytes || !colloc_bytes) return st(SNM_E_NULL);
  const int64_t G = K / M;
  *values_elems = R * 2 * G;
  *midx_bytes = R * (G / 2);
  *colloc_bytes = (R / V) * G * 4;
  return st(SNM_OK);
}

snm_status snm_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, int n, int m, void* values,
                               void* meta, void* stream) {
  if (!is_nm_2_4(n, m)) return SNM_E_UNSUPPORTED;
  int s = snm::check_prune_encode_nm(A, R, K, lda, values, meta);
  if (s != SNM_OK || R == 0 || K == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_prune_encode_nm(A, R, K, lda, values, meta, (hipStream_t)stream)));
}

snm_status snm_nm_tiled_sizes(int64_t R, int64_t K, int64_t* values_elems, int64_t* meta_bytes) {
  int s = snm::check_nm_sizes(R, K);
  if (s != SNM_OK) return st(s);
  if (!values_elems || !meta_bytes) return st(SNM_E_NULL);
  const int64_t blocks = ((R + 15) / 16) * ((K + 63) / 64);
  *values_elems = blocks * 512;
  *meta_bytes = blocks * 128;
  return st(SNM_OK);
}

snm_status snm_prune_encode_nm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, void* values_t,
                              void* meta_t, void* stream) {
  int s = snm::check_prune_encode_nm(A, R, K, lda, values_t, meta_t);
  if (s != SNM_OK || R == 0 || K == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_prune_encode_nm_tiled(A, R, K, lda, values_t, meta_t, (hipStream_t)stream)));
}

snm_status snm_spmm_nm_tiled(const void* values_t, const void* meta_t, int64_t R, int64_t K, const void* B,
                      int64_t C, int64_t ldb, int b_layout, void* Y, int64_t ldy, void* stream) {
  int s = snm::check_spmm_nm(values_t, meta_t, R, K, B, C, ldb, b_layout, Y, ldy, 1, 0, 0, 0, 0);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_tiled(values_t, meta_t, R, K, B, C, ldb, b_layout, Y, ldy,
                                            (hipStream_t)stream));
}

snm_status snm_spmm_nm_tiled_ws_bytes(int64_t R, int64_t K, int64_t C, int64_t* workspace_bytes) {
  int s = snm::check_nm_sizes(R, K);
  if (s != SNM_OK) return st(s);
  if (C < 0) return st(SNM_E_SHAPE);
  if (C > 32) return st(SNM_E_UNSUPPORTED);
  if (!workspace_bytes) return st(SNM_E_NULL);
  *workspace_bytes = (R == 0 || C == 0) ? 0 : snm::splitk_plan(R, K, C).workspace_bytes;
  return st(SNM_OK);
}

snm_status snm_spmm_nm_tiled_ws(const void* values_t, const void* meta_t, int64_t R, int64_t K, const void* B,
                         int64_t C, int64_t ldb, void* Y, int64_t ldy, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  int s = snm::check_spmm_nm_tiled_ws(values_t, meta_t, R, K, B, C, ldb, Y, ldy, workspace,
                                      workspace_bytes);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_tiled_splitk(values_t, meta_t, R, K, B, C, ldb, Y, ldy,
                                                   workspace, (hipStream_t)stream));
}

snm_status snm_spmm_nm_tiled_noalloc(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                              const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                              void* stream) {
  int s = snm::check_spmm_nm_tiled_noalloc(values_t, meta_t, R, K, B, C, ldb, Y, ldy);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_tiled_splitk_noalloc(values_t, meta_t, R, K, B, C, ldb, Y, ldy,
                                                           (hipStream_t)stream));
}

snm_status snm_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int N, int M,
                                void* values, void* midx, void* colloc, void* stream) {
  if (N != 2) return SNM_E_UNSUPPORTED;
  int s = snm::check_prune_encode_vnm(A, R, K, lda, V, M, values, midx, colloc);
  if (s != SNM_OK || R == 0 || K == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_prune_encode_vnm(A, R, K, lda, V, M, values, midx, colloc, false,
                                               (hipStream_t)stream));
}

snm_status snm_prune_encode_vnm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, int V, int N,
                                      int M, void* values_t, void* midx_t, void* colloc, void* stream) {
  if (N != 2) return SNM_E_UNSUPPORTED;
  int s = snm::check_prune_encode_vnm_tiled(A, R, K, lda, V, M, values_t, midx_t, colloc);
  if (s != SNM_OK || R == 0 || K == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_prune_encode_vnm(A, R, K, lda, V, M, values_t, midx_t, colloc, true,
                                               (hipStream_t)stream));
}

snm_status snm_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, int n, int m,
                       const void* B, int64_t C, int64_t ldb, int b_layout, void* Y, int64_t ldy,
                       int64_t batch, int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                       int64_t stride_Y, void* stream) {
  if (!is_nm_2_4(n, m)) return SNM_E_UNSUPPORTED;
  int s = snm::check_spmm_nm(values, meta, R, K, B, C, ldb, b_layout, Y, ldy, batch,
                             stride_values, stride_meta, stride_B, stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm(values, meta, R, K, B, C, ldb, b_layout, Y, ldy, batch,
                                      stride_values, stride_meta, stride_B, stride_Y,
                                      (hipStream_t)stream));
}

snm_status snm_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R, int64_t K,
                        int V, int N, int M, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                        void* stream) {
  if (N != 2) return SNM_E_UNSUPPORTED;
  int s = snm::check_spmm_vnm(values, midx, colloc, R, K, V, M, B, C, ldb, Y, ldy);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_vnm(values, midx, colloc, R, K, V, M, B, C, ldb, Y, ldy,
                                       (hipStream_t)stream));
}

snm_status snm_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc, int64_t R,
                              int64_t K, int V, int N, int M, const void* B, int64_t C, int64_t ldb,
                              void* Y, int64_t ldy, void* stream) {
  if (N != 2) return SNM_E_UNSUPPORTED;
  int s = snm::check_spmm_vnm_tiled(values_t, midx_t, colloc, R, K, V, M, B, C, ldb, Y, ldy);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_vnm_tiled(values_t, midx_t, colloc, R, K, V, M, B, C, ldb, Y,
                                             ldy, (hipStream_t)stream));
}

snm_status snm_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq, int64_t Lk,
                              int64_t d, float scale, int n, int m, void* values, void* meta,
                              void* S_dense, void* stream) {
  if (!is_nm_2_4(n, m)) return SNM_E_UNSUPPORTED;
  int s = snm::check_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, values, meta, S_dense);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, scale, values, meta,
                                             S_dense, nullptr, false, (hipStream_t)stream));
}

snm_status snm_sddmm_prune_nm_rowmax(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                              int64_t Lk, int64_t d, float scale, void* values, void* meta,
                              float* row_max, void* stream) {
  int s = snm::check_sddmm_prune_nm_rowmax(Q, Kmat, batch, Lq, Lk, d, values, meta, row_max);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, scale, values, meta,
                                             nullptr, row_max, false, (hipStream_t)stream));
}

snm_status snm_sddmm_prune_nm_bf16(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                            int64_t Lk, int64_t d, float scale, void* values, void* meta,
                            void* S_dense, float* row_max, void* stream) {
  int s = snm::check_sddmm_prune_nm_bf16(Q, Kmat, batch, Lq, Lk, d, values, meta, S_dense, row_max);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, scale, values, meta,
                                             S_dense, row_max, true, (hipStream_t)stream));
}

snm_status snm_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                     int64_t C, int64_t ldb, void* Y, int64_t ldy, int64_t batch,
                     int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                     int64_t stride_Y, void* stream) {
  int s = snm::check_spmm_nm_bf16(values, meta, R, K, B, C, ldb, Y, ldy, batch, stride_values,
                                  stride_meta, stride_B, stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_bf16(values, meta, R, K, B, C, ldb, Y, ldy, batch,
                                           stride_values, stride_meta, stride_B, stride_Y,
                                           (hipStream_t)stream));
}

snm_status snm_spmm_nm_softmax(const void* values, const void* meta, const float* row_max, int64_t R,
                        int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                        int64_t batch, int64_t stride_values, int64_t stride_meta,
                        int64_t stride_row_max, int64_t stride_B, int64_t stride_Y, void* stream) {
  int s = snm::check_spmm_nm_softmax(values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch,
                                     stride_values, stride_meta, stride_row_max, stride_B,
                                     stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_softmax(values, meta, row_max, R, K, B, C, ldb, Y, ldy,
                                              batch, stride_values, stride_meta, stride_row_max,
                                              stride_B, stride_Y, false, (hipStream_t)stream));
}

snm_status snm_spmm_nm_softmax_bf16(const void* values, const void* meta, const float* row_max,
                             int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb, void* Y,
                             int64_t ldy, int64_t batch, int64_t stride_values,
                             int64_t stride_meta, int64_t stride_row_max, int64_t stride_B,
                             int64_t stride_Y, void* stream) {
  int s = snm::check_spmm_nm_softmax(values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch,
                                     stride_values, stride_meta, stride_row_max, stride_B,
                                     stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_nm_softmax(values, meta, row_max, R, K, B, C, ldb, Y, ldy,
                                              batch, stride_values, stride_meta, stride_row_max,
                                              stride_B, stride_Y, true, (hipStream_t)stream));
}

snm_status snm_bitmap_sizes(int64_t R, int64_t K, int64_t* n_tiles, int64_t* n_offsets) {
  int s = snm::check_bitmap_sizes(R, K);
  if (s != SNM_OK) return st(s);
  if (!n_tiles || !n_offsets) return st(SNM_E_NULL);
  *n_tiles = R * (K / 64);
  *n_offsets = R * (K / 64) + 1;
  return st(SNM_OK);
}

snm_status snm_bitmap_count(const void* A, int64_t R, int64_t K, int64_t lda, void* bitmaps,
                     void* tile_offsets, void* stream) {
  int s = snm::check_bitmap_encode(A, R, K, lda, bitmaps, tile_offsets, nullptr, false);
  if (s != SNM_OK) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  // an empty matrix still gets its single offset (0)
  const int64_t Rl = (R == 0 || K == 0) ? 0 : R;
  return launched(snm::launch_bitmap_count(A, Rl, Rl ? K : 0, lda, (uint64_t*)bitmaps,
                                           (uint32_t*)tile_offsets, (hipStream_t)stream));
}

snm_status snm_bitmap_encode(const void* A, int64_t R, int64_t K, int64_t lda, const void* bitmaps,
                      const void* tile_offsets, void* values, void* stream) {
  int s = snm::check_bitmap_encode(A, R, K, lda, bitmaps, tile_offsets, values, true);
  if (s != SNM_OK || R == 0 || K == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_bitmap_values(A, R, K, lda, (const uint64_t*)bitmaps,
                                            (const uint32_t*)tile_offsets, values,
                                            (hipStream_t)stream));
}

snm_status snm_spmm_bitmap(const void* bitmaps, const void* tile_offsets, const void* values, int64_t R,
                    int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                    int64_t ldy, void* stream) {
  int s = snm::check_spmm_bitmap(bitmaps, tile_offsets, values, R, K, B, C, ldb, b_layout, Y, ldy);
  if (s != SNM_OK || R == 0 || C == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_bitmap((const uint64_t*)bitmaps, (const uint32_t*)tile_offsets,
                                          values, R, K, B, C, ldb, b_layout, Y, ldy,
                                          (hipStream_t)stream));
}

snm_status snm_softmax_nm_rows(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream) {
  int s = snm::check_softmax_nm_rows(values, rows, kept, ld);
  if (s != SNM_OK || rows == 0 || kept == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_softmax_nm_rows(values, rows, kept, ld, false, (hipStream_t)stream)));
}

snm_status snm_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                             int64_t Lk, int64_t d, float scale, void* values, void* meta,
                             void* S_dense, float* row_max, void* stream) {
  int s = snm::check_sddmm_prune_1of2_f32(Q, Kmat, batch, Lq, Lk, d, values, meta, S_dense, row_max);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_sddmm_prune_1of2_f32(Q, Kmat, batch, Lq, Lk, d, scale, values, meta,
                                                   S_dense, row_max, (hipStream_t)stream));
}

snm_status snm_softmax_nm_rows_f32(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream) {
  int s = snm::check_softmax_nm_rows(values, rows, kept, ld);
  if (s != SNM_OK || rows == 0 || kept == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_softmax_rows_f32(values, rows, kept, ld, (hipStream_t)stream)));
}

snm_status snm_spmm_1of2_f32(const void* values, const void* meta, const float* row_max, int64_t R,
                      int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                      int64_t batch, int64_t stride_values, int64_t stride_meta,
                      int64_t stride_row_max, int64_t stride_B, int64_t stride_Y, void* stream) {
  int s = snm::check_spmm_1of2_f32(values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch,
                                   stride_values, stride_meta, stride_row_max, stride_B, stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return launched(snm::launch_spmm_1of2_f32(values, meta, row_max, R, K, B, C, ldb, Y, ldy, batch,
                                            stride_values, stride_meta, stride_row_max, stride_B,
                                            stride_Y, (hipStream_t)stream));
}

snm_status snm_softmax_nm_rows_bf16(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream) {
  int s = snm::check_softmax_nm_rows(values, rows, kept, ld);
  if (s != SNM_OK || rows == 0 || kept == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_softmax_nm_rows(values, rows, kept, ld, true, (hipStream_t)stream)));
}

snm_status snm_ceiling_read(const void* src, int64_t bytes, void* sink, void* stream) {
  int s = snm::check_ceiling_stream(src, sink, bytes);
  if (s != SNM_OK || bytes == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_ceiling_read(src, bytes, sink, (hipStream_t)stream)));
}

snm_status snm_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  int s = snm::check_ceiling_stream(src, dst, bytes);
  if (s != SNM_OK || bytes == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_ceiling_copy(src, dst, bytes, (hipStream_t)stream)));
}

snm_status snm_ceiling_lds_fill(const void* src, int64_t window_bytes, int64_t workgroups, int64_t iters,
                                float* out, void* stream) {
  int s = snm::check_ceiling_lds_fill(src, window_bytes, workgroups, iters, out);
  if (s != SNM_OK || workgroups == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_ceiling_lds_fill(src, window_bytes, workgroups, iters, out, (hipStream_t)stream)));
}

snm_status snm_ceiling_matrix(int kind, int64_t workgroups, int64_t iters, float* out, void* stream) {
  int s = snm::check_ceiling_matrix(kind, workgroups, iters, out);
  if (s != SNM_OK || workgroups == 0) return st(s);
  if ((s = check_device()) != SNM_OK) return st(s);
  return st(launched(snm::launch_ceiling_matrix(kind, workgroups, iters, out, (hipStream_t)stream)));
}

}  // extern "C"
