/*
 * snm.h -- C ABI of libsnm: N:M and V:N:M structured-sparse x dense products and
 * dynamic 2:4 attention on one AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types      Element buffers are IEEE binary16 (fp16). Metadata buffers are bytes.
 *            Everything is row-major. Leading dimensions (lda, ldb, ldy, ld) and
 *            batch strides are counted in elements of the buffer they describe.
 * Memory     Every pointer argument is DEVICE memory owned by the caller. The library
 *            never allocates, frees or synchronises. Work is enqueued on `stream`
 *            (a hipStream_t; NULL is the default stream) and the call returns at once.
 * Alignment  Compressed arrays (values, meta, midx, colloc), A, Q and Kmat must be
 *            16-byte aligned and A's leading dimension a multiple of 8 elements. Dense
 *            B and Y accept any leading dimension (2-byte aligned pointers); B rows
 *            that are 16-byte aligned are read 8 columns at a time.
 * Errors     All argument checks run on the host before any HIP call. A failed check
 *            returns its status with nothing enqueued. SNM_E_DEVICE means the current
 *            device is not gfx950. SNM_E_LAUNCH reports the HIP error of the launch
 *            itself; faults during execution surface at the caller's next
 *            synchronisation. Nothing throws across this interface.
 * Sizes      Empty problems (R, C or batch equal to 0) are valid and enqueue nothing.
 * Threads    The library holds no mutable state besides a per-device architecture
 *            check; calls from several host threads are safe.
 *
 * Canonical compressed layouts (identical on the host and the device; no reordering)
 * -------------------------------------------------------------------------------
 * 2:4 ("2:4 sparsity on sparse tensor cores", lecture notes: "The compressed format";
 *      "Dynamic N:M ... attention", PPoPP'23, Sec. 4.2 Fig. 6(b) and Sec. 4.3):
 *   values  fp16, R x K/2. Per group g of four consecutive elements along K, the two
 *           kept elements in ascending slot order at columns 2g, 2g+1.
 *   meta    uint8, R x K/8. Group code = s0 | s1 << 2 with slots s0 < s1 (one of
 *           0x4 0x8 0x9 0xc 0xd 0xe). Group g sits in bits [4(g%4), 4(g%4)+3] of the
 *           little-endian 16-bit word g/4; i.e. byte b holds group 2b (low nibble)
 *           and group 2b+1 (high nibble).
 *   Selection: the two largest magnitudes per group, magnitude = fp16 bits & 0x7FFF
 *           (NaN > Inf > finite; +0 and -0 tie); on equal magnitude the lower slot
 *           wins. Kept values are bit copies of the input.
 * V:2:M ("VENOM: A vectorized N:M format ...", SC'23, Sec. 3 and Fig. 2-4):
 *   values  fp16, R x 2K/M.   Two kept values per row per group of M columns.
 *   midx    uint8, R x K/(2M). 2-bit positions (0..3) into the four selected columns,
 *           packed exactly like the 2:4 meta.
 *   colloc  uint8, (R/V) x (K/M) x 4. The four selected columns of each V x M block,
 *           ascending, each in 0..M-1.
 *   Selection: per V x M block, the four columns with the largest sum of squares over
 *           the block's V rows (summed in float64, rows in ascending order; ties go to
 *           the lower column); then, per row, 2:4 over the four selected values.
 */
#ifndef SNM_H
#define SNM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SNM_OK = 0,
  SNM_E_NULL = 1,        /* a required pointer is NULL */
  SNM_E_SHAPE = 2,       /* a size, leading dimension or stride is invalid */
  SNM_E_ALIGN = 3,       /* a pointer or leading dimension breaks the alignment rule */
  SNM_E_UNSUPPORTED = 4, /* a pattern (V, M) or head_dim outside the supported set */
  SNM_E_DEVICE = 5,      /* the current HIP device is not gfx950, or no device */
  SNM_E_LAUNCH = 6       /* the kernel launch returned a HIP error */
} snm_status;

/* Version of this ABI and of the canonical layouts above. */
int snm_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* snm_status_string(snm_status status);

/* Pattern arguments. The calls named after a pattern take its parameters, as the pages
 * write them: (n, m) for N:M, (v, n, m) for V:N:M. This library implements n = 2 of m = 4
 * (N:M) and n = 2 of m in [4, 256] (V:N:M, the sparse matrix core's 2:4 after the column
 * selection); any other (n, m) returns SNM_E_UNSUPPORTED before anything else is checked.
 * Size queries report element counts of the values arrays (fp16) and byte counts of the
 * metadata arrays, as int64_t like every other size here. */

/* Sizes of the compressed 2:4 arrays of an R x K matrix: values elements (R*K/2) and
 * meta bytes (R*K/8). Requires R >= 0, K >= 0, K % 16 == 0. Host only. */
snm_status snm_nm_sizes(int64_t R, int64_t K, int n, int m, int64_t* values_elems, int64_t* meta_bytes);

/* Sizes of the V:2:M arrays of an R x K matrix. Requires R % V == 0, K % M == 0,
 * (K/M) % 4 == 0, V in {1,...,256}, 4 <= M <= 256. Host only. */
snm_status snm_vnm_sizes(int64_t R, int64_t K, int V, int N, int M, int64_t* values_elems,
                         int64_t* midx_bytes, int64_t* colloc_bytes);

/* 2:4 magnitude prune along K and compress (lecture notes, "The definition" and
 * "The compressed format"; worked 2 x 8 example).
 *   A       fp16 R x K, leading dimension lda >= K.
 *   values  fp16 R x K/2 (contiguous), meta uint8 R x K/8 (contiguous): written.
 * Requires K % 16 == 0. Output is bit-exactly the canonical layout above. */
snm_status snm_prune_encode_nm(const void* A, int64_t R, int64_t K, int64_t lda, int n, int m,
                               void* values, void* meta, void* stream);

/* V:2:M prune and compress (VENOM Sec. 3, Fig. 2 and Fig. 3).
 *   A       fp16 R x K, leading dimension lda >= K.
 *   values  fp16 R x 2K/M, midx uint8 R x K/(2M), colloc uint8 (R/V) x (K/M) x 4.
 * Requires the shape rules of snm_vnm_sizes. */
snm_status snm_prune_encode_vnm(const void* A, int64_t R, int64_t K, int64_t lda, int V, int N, int M,
                                void* values, void* midx, void* colloc, void* stream);

/* Y = decode(values, meta) * B, batched (lecture notes, "How the tensor core uses it";
 * the metadata selects, per kept value, the row of B it multiplies).
 *   values, meta  2:4 arrays of an R x K matrix (canonical layout), per batch entry at
 *                 values + b*stride_values (elements) and meta + b*stride_meta (bytes).
 *   B             fp16 K x C, entry b at B + b*stride_B. b_layout 0: row-major, element
 *                 (k, c) at B[k*ldb + c], ldb >= C. b_layout 1: column-major, element
 *                 (k, c) at B[c*ldb + k], ldb >= K (decode activations X[C][K] as stored).
 *   Y             fp16 R x C, row-major, leading dimension ldy >= C, entry b at Y + b*stride_Y.
 * Products accumulate in fp32; Y is rounded to fp16 (round to nearest even). Requires
 * K % 16 == 0, batch >= 1 (0 enqueues nothing). Strides are ignored when batch == 1. */
snm_status snm_spmm_nm(const void* values, const void* meta, int64_t R, int64_t K, int n, int m,
                const void* B, int64_t C, int64_t ldb, int b_layout, void* Y, int64_t ldy,
                int64_t batch, int64_t stride_values, int64_t stride_meta,
                int64_t stride_B, int64_t stride_Y, void* stream);

/* Operand-major ("tiled") storage of the same 2:4 data, laid out for the CDNA4 sparse
 * matrix instruction (the analogue of the fragment-ordered storage of VENOM Sec. 4.1.2,
 * Fig. 7): the matrix is cut into blocks of 16 rows x 64 positions along K; block
 * (rt, kc) is stored at index rt*ceil(K/64) + kc as
 *   values_t  64 lanes x 8 fp16 (1 KiB): lane l = 16q + i holds row 16rt + i, positions
 *             64kc + 16q + [0, 16) -- its four groups' kept values in canonical order;
 *   meta_t    64 lanes x uint16 (128 B): lane l's canonical metadata word for the same
 *             four groups.
 * Rows past R and positions past K are stored as zero values and zero metadata. The
 * content is a permutation (plus padding) of the canonical values and meta. */

/* Sizes of the operand-major arrays: values elements and meta bytes for an R x K matrix
 * (ceil(R/16)*ceil(K/64) blocks of 512 elements and 128 bytes). K % 16 == 0. Host only. */
snm_status snm_nm_tiled_sizes(int64_t R, int64_t K, int64_t* values_elems, int64_t* meta_bytes);

/* 2:4 prune and compress straight into the operand-major layout. Same selection as
 * snm_prune_encode_nm; A fp16 R x K (lda >= K, lda % 8 == 0); K % 16 == 0. */
snm_status snm_prune_encode_nm_tiled(const void* A, int64_t R, int64_t K, int64_t lda,
                              void* values_t, void* meta_t, void* stream);

/* Y = decode(values_t, meta_t) * B with A in the operand-major layout; B, b_layout, Y as
 * in snm_spmm_nm (no batching). fp32 accumulation, fp16 output (RNE). */
snm_status snm_spmm_nm_tiled(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                      const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                      int64_t ldy, void* stream);

/* Bytes of workspace that snm_spmm_nm_tiled_ws needs for an R x K matrix and C columns
 * (0 when it runs without a split reduction). K % 16 == 0; C <= 32 (else
 * SNM_E_UNSUPPORTED). Host only. */
snm_status snm_spmm_nm_tiled_ws_bytes(int64_t R, int64_t K, int64_t C, int64_t* workspace_bytes);

/* Y = decode(values_t, meta_t) * B for the decode regime, the same product as
 * snm_spmm_nm_tiled with B column-major (element (k, c) at B[c*ldb + k], ldb >= K, as
 * decode activations X[C][K] are stored) and C <= 32 (else SNM_E_UNSUPPORTED). The
 * reduction over K is split across workgroups where that pays (the lecture notes on 2:4
 * sparse tensor cores: small products are bound by memory traffic and fixed costs): each
 * dense operand load then serves 32 or 64 rows instead of 16. The split is chosen when
 * (K*C >= 163840 or ceil(R/16) < 256) and ceil(K/64) >= 32, with at most 4 splits;
 * elsewhere the call runs the kernel of snm_spmm_nm_tiled and the workspace size is 0.
 * The workspace never exceeds 4 MiB + 1 KiB, whatever the shape.
 *   workspace  device memory of at least snm_spmm_nm_tiled_ws_bytes(R, K, C) bytes,
 *              16-byte aligned, owned by the caller. It holds fp32 partial sums and
 *              arrival counters. It must be zero-filled before its first use; every
 *              call leaves every byte it wrote zero again, so one workspace serves any
 *              sequence of calls and shapes with no clearing in between. Calls that may
 *              run at the same time (other streams) need separate workspaces. May be NULL
 *              when the size is 0.
 * fp32 accumulation; the split partial sums are added in a fixed order, so the result
 * does not depend on scheduling. fp16 output (RNE). */
snm_status snm_spmm_nm_tiled_ws(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                         const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* snm_spmm_nm_tiled_ws for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * product, kernels and result bits as snm_spmm_nm_tiled_ws, with no workspace argument:
 * the split reduction's partial sums and counters live in a scratch array the library
 * holds on each device (4 MiB + 4 KiB, a static device array of the library, kept until
 * the process ends; every split plan fits it, a larger one would return
 * SNM_E_UNSUPPORTED). The call allocates and frees nothing. On its first use on a device
 * it looks the array up and enqueues one kernel on `stream` that zeroes it; every call
 * leaves the array zero again.
 * Concurrency: every call on one device shares that device's array, so calls that may
 * overlap on one device (other streams, other host threads) race and give wrong results;
 * serialise them, or use snm_spmm_nm_tiled_ws with a workspace per stream.
 * Arguments, layouts and requirements as snm_spmm_nm_tiled_ws without the workspace. */
snm_status snm_spmm_nm_tiled_noalloc(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                              const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                              void* stream);

/* Y = decode_vnm(values, midx, colloc) * B (VENOM Sec. 4 and Fig. 4: per block of V rows
 * the K/M*4 rows of B named by colloc are gathered, then 2:4 is applied with midx).
 *   values, midx, colloc  V:2:M arrays of an R x K matrix (canonical layout).
 *   B  fp16 K x C (ldb >= C);  Y  fp16 R x C (ldy >= C).
 * fp32 accumulation, fp16 output (RNE). Requires the shape rules of snm_vnm_sizes and
 * V a multiple of 16. */
snm_status snm_spmm_vnm(const void* values, const void* midx, const void* colloc, int64_t R,
                 int64_t K, int V, int N, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                 int64_t ldy, void* stream);

/* V:2:M prune and compress (as snm_prune_encode_vnm) into the row-group interleaved
 * storage of values and m-indices: the same arrays permuted so that the product's copies
 * read whole cache lines (the MI355X counterpart of VENOM Sec. 4.1.2 and Fig. 7, which
 * store the format in the order the kernel's fragments load it). With W = K/(4M) 16-byte
 * value chunks per row (chunk c = the 8 values of groups 4c .. 4c+3, whose m-indices form
 * the 16-bit word c of the canonical midx row):
 *   values_t  chunk c of row r at fp16 element ((r/32)*W + c)*256 + (r%32)*8;
 *   midx_t    word c of row r at 16-bit word ((r/32)*W + c)*32 + (r%32);
 *   colloc    canonical (unchanged).
 * Sizes as snm_vnm_sizes. Requires its shape rules and V % 32 == 0 (else
 * SNM_E_UNSUPPORTED); values_t, midx_t 16-byte aligned. */
snm_status snm_prune_encode_vnm_tiled(const void* A, int64_t R, int64_t K, int64_t lda, int V, int N,
                                      int M, void* values_t, void* midx_t, void* colloc, void* stream);

/* Y = decode_vnm(values_t, midx_t, colloc) * B with values and m-indices in the row-group
 * interleaved storage of snm_prune_encode_vnm_tiled; B, Y as in snm_spmm_vnm. fp32
 * accumulation, fp16 output (RNE). Runs the wide-tile kernel only: requires V % 32 == 0,
 * C % 8 == 0, ldb % 8 == 0, 4K/M <= 16384 and 32-bit copy offsets (128*4K/M < 2^31,
 * (32*M*ldb + C)*2 < 2^31), else SNM_E_UNSUPPORTED; B 16-byte aligned (else SNM_E_ALIGN). */
snm_status snm_spmm_vnm_tiled(const void* values_t, const void* midx_t, const void* colloc, int64_t R,
                       int64_t K, int V, int N, int M, const void* B, int64_t C, int64_t ldb, void* Y,
                       int64_t ldy, void* stream);

/* Dynamic 2:4 SDDMM ("Dynamic N:M ... attention", Sec. 3.2 and Listing 1; Sec. 4.2-4.3):
 * for each batch entry b, S = fp16_RNE((Q_b Kmat_b^T) * scale), then 2:4 prune and
 * compress each row of S along the key axis, fused in one kernel.
 *   Q       fp16 [batch, Lq, d] contiguous;  Kmat  fp16 [batch, Lk, d] contiguous.
 *   values  fp16 [batch, Lq, Lk/2];  meta uint8 [batch, Lq, Lk/8]  (canonical 2:4).
 *   S_dense optional fp16 [batch, Lq, Lk]: if not NULL it receives S before pruning.
 * The product accumulates in fp32 and is scaled in fp32 before the single rounding to
 * fp16. Requires Lk % 32 == 0 and d in {16, 32, 64, 128}. */
snm_status snm_sddmm_prune_nm(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                       int64_t Lk, int64_t d, float scale, int n, int m, void* values, void* meta,
                       void* S_dense, void* stream);

/* Fused-softmax variant of dynamic 2:4 attention ("Dynamic N:M ... attention", Sec. 3.2:
 * softmax acts on each row's kept entries only, and the SDDMM epilogue is the place that
 * sees a whole row of scores). Instead of a separate softmax pass over the compressed
 * scores, the SDDMM also reports each row's largest kept score and the SpMM turns the
 * scores into probabilities as it multiplies.
 *
 * snm_sddmm_prune_nm_rowmax: exactly snm_sddmm_prune_nm (no S_dense) and, in addition,
 *   row_max  fp32 [batch, Lq]: the largest kept (fp16) score of each row, widened exactly.
 * Requires what snm_sddmm_prune_nm requires; row_max 4-byte aligned. */
snm_status snm_sddmm_prune_nm_rowmax(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                              int64_t Lk, int64_t d, float scale, void* values, void* meta,
                              float* row_max, void* stream);

/* snm_spmm_nm_softmax: Y = P * B with P the row softmax of the kept scores (dropped entries
 * count as -inf), decoded through meta: per row, p = fp16_RNE(exp(v - row_max)) for each
 * kept score v (exp in fp32), the products accumulate in fp32, and the output row is
 * divided by the fp32 sum of its p values before rounding to fp16 (RNE).
 *   values, meta  2:4 scores as written by snm_sddmm_prune_nm (canonical layout), per batch
 *                 entry at values + b*stride_values and meta + b*stride_meta (bytes).
 *   row_max       fp32, R per batch entry at row_max + b*stride_row_max: a value >= every
 *                 kept score of the row (snm_sddmm_prune_nm_rowmax writes the maximum);
 *                 any such value gives the same P up to rounding.
 *   B, Y          as in snm_spmm_nm with b_layout 0 (row-major B).
 * Requires K % 16 == 0 and K > 0, C % 8 == 0, ldb % 8 == 0, B 16-byte aligned (and
 * stride_B % 8 == 0 when batch > 1), 128*K < 2^31 and (256*ldb + C)*2 < 2^31. */
snm_status snm_spmm_nm_softmax(const void* values, const void* meta, const float* row_max, int64_t R,
                        int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                        int64_t batch, int64_t stride_values, int64_t stride_meta,
                        int64_t stride_row_max, int64_t stride_B, int64_t stride_Y, void* stream);

/* Bitmap format for unstructured sparsity ("Coruscant: Co-Designing GPU Kernel and Sparse
 * Tensor Core ...", Sec. 3.1 and Fig. 7; Sec. 3.2 for the padding). An R x K fp16 matrix
 * (K % 64 == 0, R*K < 2^31) is cut into tiles of 64 consecutive positions along K of one
 * row, in row-major tile order (tile t = r*K/64 + k/64):
 *   bitmaps       uint64 [R*K/64]: bit i of tile t is set iff position i of the tile holds
 *                 a non-zero (fp16 magnitude bits not all zero: +0 and -0 are not stored);
 *   tile_offsets  uint32 [R*K/64 + 1]: element index in values of tile t's first non-zero
 *                 (the exclusive prefix sum of the padded counts); the last entry is the
 *                 number of values;
 *   values        fp16 [tile_offsets[R*K/64]]: each tile's non-zeros in ascending position
 *                 order, padded with +0 to a multiple of 8 (every tile starts 16-byte
 *                 aligned).
 * Sizes of the fixed arrays (host only). */
snm_status snm_bitmap_sizes(int64_t R, int64_t K, int64_t* n_tiles, int64_t* n_offsets);

/* Encoder, pass 1: bitmaps and tile_offsets of A (fp16 R x K row-major, lda >= K,
 * lda % 8 == 0, A 16-byte aligned; bitmaps 8-byte and tile_offsets 4-byte aligned). After
 * the stream reaches this call, tile_offsets[R*K/64] is the number of values to allocate. */
snm_status snm_bitmap_count(const void* A, int64_t R, int64_t K, int64_t lda, void* bitmaps,
                     void* tile_offsets, void* stream);

/* Encoder, pass 2: the packed values (fp16 [tile_offsets[R*K/64]]) from A and the arrays of
 * pass 1. values may be NULL when that count is 0 (it is then never touched). */
snm_status snm_bitmap_encode(const void* A, int64_t R, int64_t K, int64_t lda, const void* bitmaps,
                      const void* tile_offsets, void* values, void* stream);

/* Y = decode(bitmaps, tile_offsets, values) * B for a decode-shaped B with C <= 32 columns
 * (Coruscant Sec. 3.2: the product of a bitmap-compressed weight with few activations).
 * B, b_layout, Y as in snm_spmm_nm; column-major B (b_layout 1) needs ldb % 8 == 0 and a
 * 16-byte aligned B; row-major B (b_layout 0) is supported, slower, with ldb <= 2^25
 * (larger strides return SNM_E_UNSUPPORTED). values 16-byte aligned. fp32 accumulation,
 * fp16 output (RNE). C > 32 returns SNM_E_UNSUPPORTED. values may be NULL when the encoding
 * holds no non-zeros. */
snm_status snm_spmm_bitmap(const void* bitmaps, const void* tile_offsets, const void* values, int64_t R,
                    int64_t K, const void* B, int64_t C, int64_t ldb, int b_layout, void* Y,
                    int64_t ldy, void* stream);

/* In-place row softmax over the kept entries of compressed rows ("Dynamic N:M ...
 * attention", Sec. 3.2: softmax runs only on each row's kept entries; dropped
 * entries count as -inf). values: fp16 rows x kept, leading dimension ld >= kept.
 * p = exp(v - max) / sum exp(v - max) per row, in fp32, rounded to fp16 (RNE). */
snm_status snm_softmax_nm_rows(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream);

/* bf16 variant of dynamic 2:4 attention ("Dynamic N:M ... attention", Sec. 4.2: 16-bit
 * scores of either fp16 or bf16 are pruned 2 of 4 in every 8 bytes). Every element buffer
 * below holds bf16 instead of fp16; layouts, metadata, the selection rule (on the 16-bit
 * patterns: magnitude bits, lower slot wins ties) and all requirements are those of the
 * fp16 call of the same name. Every bf16 result is one round-to-nearest-even of an fp32
 * value; products and sums are in fp32.
 *
 * snm_sddmm_prune_nm_bf16: snm_sddmm_prune_nm on bf16 Q, Kmat, values (and S_dense);
 *   row_max optional (NULL: not written): as in snm_sddmm_prune_nm_rowmax. */
snm_status snm_sddmm_prune_nm_bf16(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                            int64_t Lk, int64_t d, float scale, void* values, void* meta,
                            void* S_dense, float* row_max, void* stream);

/* snm_softmax_nm_rows_bf16: snm_softmax_nm_rows on bf16 rows. */
snm_status snm_softmax_nm_rows_bf16(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream);

/* snm_spmm_nm_bf16: snm_spmm_nm with b_layout 0 on bf16 values, B and Y, batched the same
 * way. Requires, beyond the rules of snm_spmm_nm: C % 8 == 0, ldb % 8 == 0, B 16-byte
 * aligned (and stride_B % 8 == 0 when batch > 1), 128*K < 2^31 and (256*ldb + C)*2 < 2^31;
 * otherwise SNM_E_ALIGN or SNM_E_SHAPE. K == 0 writes zeros. */
snm_status snm_spmm_nm_bf16(const void* values, const void* meta, int64_t R, int64_t K, const void* B,
                     int64_t C, int64_t ldb, void* Y, int64_t ldy, int64_t batch,
                     int64_t stride_values, int64_t stride_meta, int64_t stride_B,
                     int64_t stride_Y, void* stream);

/* snm_spmm_nm_softmax_bf16: snm_spmm_nm_softmax on bf16 values, B and Y; the probabilities
 * are p = bf16_RNE(exp(v - row_max)). */
snm_status snm_spmm_nm_softmax_bf16(const void* values, const void* meta, const float* row_max,
                             int64_t R, int64_t K, const void* B, int64_t C, int64_t ldb, void* Y,
                             int64_t ldy, int64_t batch, int64_t stride_values,
                             int64_t stride_meta, int64_t stride_row_max, int64_t stride_B,
                             int64_t stride_Y, void* stream);

/* 1:2 dynamic attention on fp32 scores ("Dynamic N:M ... attention", Sec. 1 and Fig. 1-3:
 * the mechanism at 1:2; Sec. 4.2: 32-bit data keeps one of every two 4-byte elements).
 * Format of an R x K fp32 score matrix pruned 1:2 along K (K % 32 == 0):
 *   values  fp32 [R, K/2]: the kept element of each pair (2p, 2p + 1), a bit copy;
 *   meta    uint8 [R, K/4]: one 4-bit code per pair, 0x4 = the first element kept, 0xe = the
 *           second (the codes of 2:4 over the pair's 16-bit halves); pair 2b in the low and
 *           pair 2b + 1 in the high nibble of byte b.
 * Selection: the element with the larger magnitude (fp32 bits without the sign) is kept; on
 * a tie the first. The products run on the dense fp32 matrix core (full fp32 products,
 * fp32 accumulation): this architecture has no 32-bit sparse matrix instruction.
 *
 * snm_sddmm_prune_1of2_f32: S = fp32((Q_b Kmat_b^T) * scale) for each batch entry, pruned
 *   1:2 along the keys. Q fp32 [batch, Lq, d], Kmat fp32 [batch, Lk, d] contiguous;
 *   values fp32 [batch, Lq, Lk/2]; meta [batch, Lq, Lk/4]; S_dense optional fp32
 *   [batch, Lq, Lk] (pre-prune S); row_max optional fp32 [batch, Lq] (largest kept score).
 *   Requires Lk % 32 == 0, d in {16, 32, 64, 128}, 16-byte aligned arrays (row_max 4). */
snm_status snm_sddmm_prune_1of2_f32(const void* Q, const void* Kmat, int64_t batch, int64_t Lq,
                             int64_t Lk, int64_t d, float scale, void* values, void* meta,
                             void* S_dense, float* row_max, void* stream);

/* snm_softmax_nm_rows_f32: snm_softmax_nm_rows on fp32 rows (fp32 output, no rounding step
 * beyond fp32 arithmetic). */
snm_status snm_softmax_nm_rows_f32(void* values, int64_t rows, int64_t kept, int64_t ld, void* stream);

/* snm_spmm_1of2_f32: Y = decode(values, meta) * B for 1:2 fp32 operands, per batch entry at
 * values + b*stride_values, meta + b*stride_meta (bytes), B + b*stride_B, Y + b*stride_Y.
 *   B  fp32 K x C row-major (ldb >= C);  Y  fp32 R x C (ldy >= C).
 *   row_max  NULL: plain product. Otherwise values are scores and the row softmax over the
 *            kept entries is applied inside the product (fused variant): p = exp(v - row_max)
 *            in fp32, the output row divided by the fp32 sum of its p; row_max (R per batch
 *            entry at row_max + b*stride_row_max) must be >= every kept score of its row.
 * Requires K % 32 == 0 (K > 0 with row_max), C % 4 == 0, ldb % 4 == 0, values and B 16-byte,
 * meta 8-byte, Y and row_max 4-byte aligned; with batch > 1, stride_values % 4 == 0,
 * stride_meta % 8 == 0, stride_B % 4 == 0. K == 0 writes zeros. */
snm_status snm_spmm_1of2_f32(const void* values, const void* meta, const float* row_max, int64_t R,
                      int64_t K, const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                      int64_t batch, int64_t stride_values, int64_t stride_meta,
                      int64_t stride_row_max, int64_t stride_B, int64_t stride_Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SNM_H */
