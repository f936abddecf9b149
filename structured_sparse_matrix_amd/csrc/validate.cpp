// Argument validation (host only, no HIP). Status values match snm_status in snm.h.
#include "validate.hpp"

#include <stdint.h>

#include <initializer_list>

#include "snm.h"

namespace snm {
namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned2(const void* p) { return ((uintptr_t)p & 1u) == 0; }
bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}
// Element counts above 2^47 are rejected so that every offset fits comfortably in int64.
constexpr int64_t kMaxElems = (int64_t)1 << 47;
bool fits(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (b == 0 || a <= kMaxElems / b); }

}  // namespace

int check_nm_sizes(int64_t R, int64_t K) {
  if (R < 0 || K < 0 || K % 16 != 0 || !fits(R, K)) return SNM_E_SHAPE;
  return SNM_OK;
}

int check_vnm_sizes(int64_t R, int64_t K, int V, int M) {
  if (V < 1 || V > 256 || M < 4 || M > 256) return SNM_E_UNSUPPORTED;
  if (R < 0 || K < 0 || !fits(R, K)) return SNM_E_SHAPE;
  if (R % V != 0 || K % M != 0 || (K / M) % 4 != 0) return SNM_E_SHAPE;
  return SNM_OK;
}

int check_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, const void* values,
                          const void* meta) {
  int s = check_nm_sizes(R, K);
  if (s != SNM_OK) return s;
  if (R == 0 || K == 0) return SNM_OK;
  if (!A || !values || !meta) return SNM_E_NULL;
  if (lda < K || !fits(R, lda)) return SNM_E_SHAPE;
  if (lda % 8 != 0 || !all_aligned({A, values, meta})) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                           const void* values, const void* midx, const void* colloc) {
  int s = check_vnm_sizes(R, K, V, M);
  if (s != SNM_OK) return s;
  if (R == 0 || K == 0) return SNM_OK;
  if (!A || !values || !midx || !colloc) return SNM_E_NULL;
  if (lda < K || !fits(R, lda)) return SNM_E_SHAPE;
  if (lda % 8 != 0 || !all_aligned({A, values, midx, colloc})) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                  int64_t C, int64_t ldb, int b_layout, const void* Y, int64_t ldy, int64_t batch,
                  int64_t stride_values, int64_t stride_meta, int64_t stride_B, int64_t stride_Y) {
  int s = check_nm_sizes(R, K);
  if (s != SNM_OK) return s;
  if (b_layout != 0 && b_layout != 1) return SNM_E_UNSUPPORTED;
  if (C < 0 || batch < 0 || !fits(K, C) || !fits(R, C)) return SNM_E_SHAPE;
  if (R == 0 || C == 0 || batch == 0) return SNM_OK;
  if (!Y || (K > 0 && (!values || !meta || !B))) return SNM_E_NULL;
  // row-major B: K rows of ldb >= C; column-major B: C columns of ldb >= K
  const int64_t b_lines = b_layout == 0 ? K : C;
  const int64_t b_min_ld = b_layout == 0 ? C : K;
  if (ldy < C || ldb < b_min_ld || !fits(b_lines, ldb) || !fits(R, ldy)) return SNM_E_SHAPE;
  if (batch > 1) {
    if (stride_values < R * (K / 2) || stride_meta < R * (K / 8) || stride_B < b_lines * ldb ||
        stride_Y < R * ldy || !fits(batch, stride_values) || !fits(batch, stride_B) ||
        !fits(batch, stride_Y) || !fits(batch, stride_meta))
      return SNM_E_SHAPE;
    // an empty reduction (K == 0) reads no A entry: its strides carry no alignment rule
    if (K > 0 && (stride_values % 8 != 0 || stride_meta % 16 != 0)) return SNM_E_ALIGN;
  }
  if (!all_aligned({values, meta}) || !aligned2(B) || !aligned2(Y)) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R, int64_t K,
                   int V, int M, const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy) {
  int s = check_vnm_sizes(R, K, V, M);
  if (s != SNM_OK) return s;
  if (V % 16 != 0) return SNM_E_UNSUPPORTED;
  if (C < 0 || !fits(K, C) || !fits(R, C)) return SNM_E_SHAPE;
  if (R == 0 || C == 0) return SNM_OK;
  if (!Y || (K > 0 && (!values || !midx || !colloc || !B))) return SNM_E_NULL;
  if (ldy < C || ldb < C || !fits(K, ldb) || !fits(R, ldy)) return SNM_E_SHAPE;
  if (!all_aligned({values, midx, colloc}) || !aligned2(B) || !aligned2(Y)) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_prune_encode_vnm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, int V, int M,
                                 const void* values_t, const void* midx_t, const void* colloc) {
  int s = check_vnm_sizes(R, K, V, M);
  if (s != SNM_OK) return s;
  if (V % 32 != 0) return SNM_E_UNSUPPORTED;   // whole groups of 32 rows
  return check_prune_encode_vnm(A, R, K, lda, V, M, values_t, midx_t, colloc);
}

int check_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc, int64_t R,
                         int64_t K, int V, int M, const void* B, int64_t C, int64_t ldb,
                         const void* Y, int64_t ldy) {
  int s = check_vnm_sizes(R, K, V, M);
  if (s != SNM_OK) return s;
  if (V % 32 != 0) return SNM_E_UNSUPPORTED;
  if ((s = check_spmm_vnm(values_t, midx_t, colloc, R, K, V, M, B, C, ldb, Y, ldy)) != SNM_OK) return s;
  if (R == 0 || C == 0) return SNM_OK;
  // the wide-tile kernel: 16-byte B rows, column-loc of a V-block staged in LDS, 32-bit
  // per-lane copy offsets (one tile's A rows, one stage's gathered B rows)
  const int64_t Kc = 4 * (K / M);
  if (C % 8 != 0 || ldb % 8 != 0 || Kc > 16384) return SNM_E_UNSUPPORTED;
  constexpr int64_t kLim = (int64_t)1 << 31;
  if (128 * Kc >= kLim || (32 * (int64_t)M * ldb + C) * 2 >= kLim) return SNM_E_UNSUPPORTED;
  if (K > 0 && !aligned16(B)) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq, int64_t Lk,
                         int64_t d, const void* values, const void* meta, const void* S_dense) {
  if (d != 16 && d != 32 && d != 64 && d != 128) return SNM_E_UNSUPPORTED;
  if (batch < 0 || Lq < 0 || Lk < 0 || Lk % 32 != 0 || !fits(batch, Lq) || !fits(batch * Lq, Lk) ||
      !fits(batch * Lk, d) || !fits(batch * Lq, d))
    return SNM_E_SHAPE;
  if (batch == 0 || Lq == 0 || Lk == 0) return SNM_OK;
  if (!Q || !Kmat || !values || !meta) return SNM_E_NULL;
  if (!all_aligned({Q, Kmat, values, meta, S_dense})) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_sddmm_prune_nm_rowmax(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                                int64_t Lk, int64_t d, const void* values, const void* meta,
                                const void* row_max) {
  int s = check_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, values, meta, nullptr);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return s;
  if (!row_max) return SNM_E_NULL;
  if (((uintptr_t)row_max & 3u) != 0) return SNM_E_ALIGN;
  return SNM_OK;
}

// Extra rules of the wide-output kernel (row-major B): 16-byte B rows and 32-bit per-lane
// offsets (128 rows of values, 256 rows of B).
static int check_wide_rules(int64_t K, const void* B, int64_t C, int64_t ldb, int64_t batch,
                            int64_t stride_B) {
  if (C % 8 != 0 || ldb % 8 != 0 || !aligned16(B) || (batch > 1 && stride_B % 8 != 0))
    return SNM_E_ALIGN;
  constexpr int64_t kLim = (int64_t)1 << 31;
  if (128 * K >= kLim || (256 * ldb + C) * 2 >= kLim) return SNM_E_SHAPE;
  return SNM_OK;
}

int check_spmm_nm_softmax(const void* values, const void* meta, const void* row_max, int64_t R,
                          int64_t K, const void* B, int64_t C, int64_t ldb, const void* Y,
                          int64_t ldy, int64_t batch, int64_t stride_values, int64_t stride_meta,
                          int64_t stride_row_max, int64_t stride_B, int64_t stride_Y) {
  int s = check_spmm_nm(values, meta, R, K, B, C, ldb, 0, Y, ldy, batch, stride_values,
                        stride_meta, stride_B, stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return s;
  if (K == 0) return SNM_E_SHAPE;   // a softmax over no entries is undefined
  if (!row_max) return SNM_E_NULL;
  if (batch > 1 && (stride_row_max < R || !fits(batch, stride_row_max))) return SNM_E_SHAPE;
  if (((uintptr_t)row_max & 3u) != 0) return SNM_E_ALIGN;
  return check_wide_rules(K, B, C, ldb, batch, stride_B);
}

int check_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                       int64_t C, int64_t ldb, const void* Y, int64_t ldy, int64_t batch,
                       int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                       int64_t stride_Y) {
  int s = check_spmm_nm(values, meta, R, K, B, C, ldb, 0, Y, ldy, batch, stride_values,
                        stride_meta, stride_B, stride_Y);
  if (s != SNM_OK || R == 0 || C == 0 || batch == 0) return s;
  return check_wide_rules(K, B, C, ldb, batch, stride_B);
}

int check_sddmm_prune_nm_bf16(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                              int64_t Lk, int64_t d, const void* values, const void* meta,
                              const void* S_dense, const void* row_max) {
  int s = check_sddmm_prune_nm(Q, Kmat, batch, Lq, Lk, d, values, meta, S_dense);
  if (s != SNM_OK || batch == 0 || Lq == 0 || Lk == 0) return s;
  if (((uintptr_t)row_max & 3u) != 0) return SNM_E_ALIGN;   // NULL: no row maxima
  return SNM_OK;
}

int check_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                               int64_t Lk, int64_t d, const void* values, const void* meta,
                               const void* S_dense, const void* row_max) {
  // the same shape and alignment rules as the 16-bit SDDMM
  return check_sddmm_prune_nm_bf16(Q, Kmat, batch, Lq, Lk, d, values, meta, S_dense, row_max);
}

int check_spmm_1of2_f32(const void* values, const void* meta, const void* row_max, int64_t R,
                        int64_t K, const void* B, int64_t C, int64_t ldb, const void* Y,
                        int64_t ldy, int64_t batch, int64_t stride_values, int64_t stride_meta,
                        int64_t stride_row_max, int64_t stride_B, int64_t stride_Y) {
  if (R < 0 || K < 0 || C < 0 || batch < 0 || K % 32 != 0 || !fits(R, K) || !fits(K, C) ||
      !fits(R, C))
    return SNM_E_SHAPE;
  if (R == 0 || C == 0 || batch == 0) return SNM_OK;
  if (row_max && K == 0) return SNM_E_SHAPE;   // a softmax over no entries is undefined
  if (!Y || (K > 0 && (!values || !meta || !B))) return SNM_E_NULL;
  if (ldy < C || ldb < C || !fits(K, ldb) || !fits(R, ldy)) return SNM_E_SHAPE;
  if (batch > 1) {
    if (stride_values < R * (K / 2) || stride_meta < R * (K / 4) || stride_B < K * ldb ||
        stride_Y < R * ldy || (row_max && stride_row_max < R) || !fits(batch, stride_values) ||
        !fits(batch, stride_meta) || !fits(batch, stride_B) || !fits(batch, stride_Y) ||
        !fits(batch, stride_row_max))
      return SNM_E_SHAPE;
    if (K > 0 && (stride_values % 4 != 0 || stride_meta % 8 != 0 || stride_B % 4 != 0)) return SNM_E_ALIGN;
  }
  if (!aligned16(values) || ((uintptr_t)meta & 7u) != 0 || !aligned16(B) || C % 4 != 0 ||
      ldb % 4 != 0 || ((uintptr_t)row_max & 3u) != 0 || ((uintptr_t)Y & 3u) != 0)
    return SNM_E_ALIGN;
  return SNM_OK;
}

int check_bitmap_sizes(int64_t R, int64_t K) {
  if (R < 0 || K < 0 || K % 64 != 0 || !fits(R, K)) return SNM_E_SHAPE;
  if (R * K >= ((int64_t)1 << 31)) return SNM_E_SHAPE;   // 32-bit tile offsets
  return SNM_OK;
}

int check_bitmap_encode(const void* A, int64_t R, int64_t K, int64_t lda, const void* bitmaps,
                        const void* offsets, const void* values, bool need_values) {
  int s = check_bitmap_sizes(R, K);
  if (s != SNM_OK) return s;
  if (!offsets) return SNM_E_NULL;
  if (((uintptr_t)offsets & 3u) != 0) return SNM_E_ALIGN;
  if (R == 0 || K == 0) return SNM_OK;
  // values may be NULL: an encoding with no non-zeros never touches it
  if (!A || !bitmaps) return SNM_E_NULL;
  if (lda < K || !fits(R, lda)) return SNM_E_SHAPE;
  if (lda % 8 != 0 || !aligned16(A) || ((uintptr_t)bitmaps & 7u) != 0) return SNM_E_ALIGN;
  if (need_values && !aligned2(values)) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_spmm_bitmap(const void* bitmaps, const void* offsets, const void* values, int64_t R,
                      int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, const void* Y,
                      int64_t ldy) {
  int s = check_bitmap_sizes(R, K);
  if (s != SNM_OK) return s;
  if (b_layout != 0 && b_layout != 1) return SNM_E_UNSUPPORTED;
  if (C < 0 || !fits(K, C) || !fits(R, C)) return SNM_E_SHAPE;
  if (C > 32) return SNM_E_UNSUPPORTED;
  // row-major B is read with 32-bit byte offsets from each 64-row tile's start
  if (b_layout == 0 && ldb > (int64_t(1) << 25)) return SNM_E_UNSUPPORTED;
  if (R == 0 || C == 0) return SNM_OK;
  if (!Y || (K > 0 && (!bitmaps || !offsets || !B))) return SNM_E_NULL;   // values may be NULL (no non-zeros)
  const int64_t b_lines = b_layout == 0 ? K : C;
  const int64_t b_min_ld = b_layout == 0 ? C : K;
  if (ldy < C || ldb < b_min_ld || !fits(b_lines, ldb) || !fits(R, ldy)) return SNM_E_SHAPE;
  if (!aligned16(values) || ((uintptr_t)bitmaps & 7u) != 0 || ((uintptr_t)offsets & 3u) != 0 ||
      !aligned2(B) || !aligned2(Y))
    return SNM_E_ALIGN;
  if (b_layout == 1 && (ldb % 8 != 0 || !aligned16(B))) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_softmax_nm_rows(const void* values, int64_t rows, int64_t kept, int64_t ld) {
  if (rows < 0 || kept < 0 || ld < kept || !fits(rows, ld)) return SNM_E_SHAPE;
  if (rows == 0 || kept == 0) return SNM_OK;
  if (!values) return SNM_E_NULL;
  if (!aligned16(values)) return SNM_E_ALIGN;
  return SNM_OK;
}

SplitPlan splitk_plan(int64_t R, int64_t K, int64_t C) {
  constexpr int64_t kWaves = 16;          // waves per workgroup of the split kernel
  constexpr int64_t kTargetGroups = 256;  // about one workgroup per CU
  SplitPlan p{};
  p.cp = C <= 16 ? 16 : 32;
  const int64_t rt16 = (R + 15) / 16;
  // 64 rows per dense-operand load where 64 groups or more fill the grid with at most 4
  // splits; else 32. More than 4 splits, or two workgroups per CU, measured slower: the
  // end chain of every split workgroup (stores, fence, counter) contends.
  p.rt = rt16 >= 256 ? 4 : 2;
  p.groups = (rt16 + p.rt - 1) / p.rt;
  const int64_t kc = (K + 63) / 64;
  // The split pays where the unsplit kernel (one workgroup per 16-row tile, all of K) would
  // stream a large dense operand per workgroup (K*C >= 163840: 320 KiB) or leave CUs idle
  // (fewer than 256 row tiles); elsewhere its extra round trips (partial stores, fence,
  // counter, re-read) cost more than they save (measured on MI355X at 4096 x 4096).
  const bool worth = K * C >= 163840 || rt16 < kTargetGroups;
  // enough splits for about one workgroup per CU, and at least one chunk per wave
  int64_t s = !worth ? 1 : p.groups > 0 ? (kTargetGroups + p.groups - 1) / p.groups : 1;
  if (s > 4) s = 4;
  if (s > kc / kWaves) s = kc / kWaves;
  if (s < 1) s = 1;
  p.splits = (int)s;
  p.chunks_per_split = (int)((kc + s - 1) / s);
  const int64_t tile = 16 * p.rt * p.cp;
  p.count_bytes = p.splits > 1 ? ((p.groups * 4 + 255) / 256) * 256 : 0;
  p.workspace_bytes = p.splits > 1 ? p.count_bytes + (int64_t)p.splits * p.groups * tile * 4 : 0;
  return p;
}

int check_spmm_nm_tiled_ws(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                           const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy,
                           const void* workspace, int64_t workspace_bytes) {
  int s = check_spmm_nm(values_t, meta_t, R, K, B, C, ldb, 1, Y, ldy, 1, 0, 0, 0, 0);
  if (s != SNM_OK) return s;
  if (C > 32) return SNM_E_UNSUPPORTED;
  if (workspace_bytes < 0) return SNM_E_SHAPE;
  if (R == 0 || C == 0) return SNM_OK;
  // grid: groups workgroups along x (< 2^31)
  if ((R + 15) / 16 > ((int64_t)1 << 31)) return SNM_E_SHAPE;
  const SplitPlan p = splitk_plan(R, K, C);
  if (p.workspace_bytes > 0) {
    if (workspace_bytes < p.workspace_bytes) return SNM_E_SHAPE;
    if (!workspace) return SNM_E_NULL;
    if (((uintptr_t)workspace & 15u) != 0) return SNM_E_ALIGN;
  }
  return SNM_OK;
}

int check_spmm_nm_tiled_noalloc(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                const void* B, int64_t C, int64_t ldb, const void* Y, int64_t ldy) {
  int s = check_spmm_nm(values_t, meta_t, R, K, B, C, ldb, 1, Y, ldy, 1, 0, 0, 0, 0);
  if (s != SNM_OK) return s;
  if (C > 32) return SNM_E_UNSUPPORTED;
  if (R == 0 || C == 0) return SNM_OK;
  if ((R + 15) / 16 > ((int64_t)1 << 31)) return SNM_E_SHAPE;
  // never taken for a plan of splitk_plan; kept so that a change of the plan cannot
  // overrun the fixed scratch
  if (splitk_plan(R, K, C).workspace_bytes > kSplitScratchBytes) return SNM_E_UNSUPPORTED;
  return SNM_OK;
}

int check_ceiling_stream(const void* src, const void* dst, int64_t bytes) {
  if (bytes < 0 || bytes % 16 != 0) return SNM_E_SHAPE;
  if (bytes == 0) return SNM_OK;
  if (!src || !dst) return SNM_E_NULL;
  if (((uintptr_t)src & 15u) != 0 || ((uintptr_t)dst & 15u) != 0) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_ceiling_lds_fill(const void* src, int64_t window_bytes, int64_t workgroups, int64_t iters,
                           const void* out) {
  if (window_bytes < 1024 || window_bytes > ((int64_t)1 << 40) || (window_bytes & (window_bytes - 1)) != 0)
    return SNM_E_SHAPE;
  if (workgroups < 0 || workgroups > 0x7FFFFFFF || iters < 0) return SNM_E_SHAPE;
  if (workgroups == 0) return SNM_OK;
  if (!src || !out) return SNM_E_NULL;
  if (((uintptr_t)src & 15u) != 0 || ((uintptr_t)out & 3u) != 0) return SNM_E_ALIGN;
  return SNM_OK;
}

int check_ceiling_matrix(int kind, int64_t workgroups, int64_t iters, const void* out) {
  if (kind != 0 && kind != 1) return SNM_E_UNSUPPORTED;
  if (workgroups < 0 || workgroups > 0x7FFFFFFF || iters < 0) return SNM_E_SHAPE;
  if (workgroups == 0) return SNM_OK;
  if (!out) return SNM_E_NULL;
  if (((uintptr_t)out & 3u) != 0) return SNM_E_ALIGN;
  return SNM_OK;
}

}  // namespace snm
