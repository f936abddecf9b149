// Argument validation of every libsnm entry point. Pure host C++: no HIP call, so it is
// compiled into the library and also into a host-only test binary.
#pragma once

#include <stdint.h>

namespace snm {

int check_nm_sizes(int64_t R, int64_t K);
int check_vnm_sizes(int64_t R, int64_t K, int V, int M);
int check_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, const void* values,
                          const void* meta);
int check_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                           const void* values, const void* midx, const void* colloc);
int check_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                  int64_t C, int64_t ldb, int b_layout, const void* Y, int64_t ldy, int64_t batch,
                  int64_t stride_values, int64_t stride_meta, int64_t stride_B, int64_t stride_Y);
int check_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R, int64_t K,
                   int V, int M, const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy);
int check_prune_encode_vnm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                                 const void* values_t, const void* midx_t, const void* colloc);
int check_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc, int64_t R,
                         int64_t K, int V, int M, const void* B, int64_t C, int64_t ldb,
                         const void* Y, int64_t ldy);
int check_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq, int64_t Lk,
                         int64_t d, const void* values, const void* meta, const void* S_dense);
int check_sddmm_prune_nm_rowmax(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                int64_t Lk, int64_t d, const void* values, const void* meta,
                                const void* row_max);
int check_spmm_nm_softmax(const void* values, const void* meta, const void* row_max, int64_t R,
                          int64_t K, const void* B, int64_t C, int64_t ldb, const void* Y,
                          int64_t ldy, int64_t batch, int64_t stride_values, int64_t stride_meta,
                          int64_t stride_row_max, int64_t stride_B, int64_t stride_Y);
int check_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                       int64_t C, int64_t ldb, const void* Y, int64_t ldy, int64_t batch,
                       int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                       int64_t stride_Y);
int check_sddmm_prune_nm_bf16(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                              int64_t Lk, int64_t d, const void* values, const void* meta,
                              const void* S_dense, const void* row_max);
int check_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                               int64_t Lk, int64_t d, const void* values, const void* meta,
                               const void* S_dense, const void* row_max);
int check_spmm_1of2_f32(const void* values, const void* meta, const void* row_max, int64_t R,
                        int64_t K, const void* B, int64_t C, int64_t ldb, const void* Y,
                        int64_t ldy, int64_t batch, int64_t stride_values, int64_t stride_meta,
                        int64_t stride_row_max, int64_t stride_B, int64_t stride_Y);
int check_bitmap_sizes(int64_t R, int64_t K);
int check_bitmap_encode(const void* A, int64_t R, int64_t K, int64_t lda, const void* bitmaps,
                        const void* offsets, const void* values, bool need_values);
int check_spmm_bitmap(const void* bitmaps, const void* offsets, const void* values, int64_t R,
                      int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, const void* Y,
                      int64_t ldy);
int check_softmax_nm_rows(const void* values, int64_t rows, int64_t kept, int64_t ld);
int check_ceiling_stream(const void* src, const void* dst, int64_t bytes);
int check_ceiling_lds_fill(const void* src, int64_t window_bytes, int64_t workgroups, int64_t iters,
                           const void* out);
int check_ceiling_matrix(int kind, int64_t workgroups, int64_t iters, const void* out);

// Split-reduction plan of the operand-major 2:4 decode product (snm_spmm_nm_tiled_ws):
// row groups of 16*rt rows, `splits` workgroups per group along K, each covering
// chunks_per_split 64-position chunks; workspace = count_bytes of arrival counters, then
// splits x groups x (16*rt*cp) fp32 partial tiles. splits == 1: the product runs the
// unsplit decode kernel and needs no workspace.
struct SplitPlan {
  int cp, rt, splits, chunks_per_split;
  int64_t groups, count_bytes, workspace_bytes;
};
SplitPlan splitk_plan(int64_t R, int64_t K, int64_t C);
int check_spmm_nm_tiled_ws(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                           const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy,
                           const void* workspace, int64_t workspace_bytes);
// Size of the device-resident scratch of snm_spmm_nm_tiled_noalloc. A split plan keeps
// about 256 workgroups with at most 4 splits, so splits x groups < 512 partial tiles of at
// most 8 KiB, plus at most 1 KiB of counters: every plan fits.
constexpr int64_t kSplitScratchBytes = ((int64_t)4 << 20) + 4096;
int check_spmm_nm_tiled_noalloc(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy);

}  // namespace snm
