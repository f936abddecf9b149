/*
 * snm_ceilings.h -- measurement kernels of libsnm: the rates one MI355X (gfx950) sustains
 * with no algorithm around them, against which the library's kernels are reported beside
 * the published peaks. They belong to the benchmark, not to the method: a streaming read,
 * a streaming copy, and issue loops of one matrix instruction.
 *
 * The lecture notes on 2:4 sparse tensor cores ("Speedup: a staircase toward 2x") explain
 * why a ceiling measured on the device matters here: small products are bound by memory
 * traffic and fixed costs, so the rate a plain stream of the same size reaches is the
 * honest bound for a decode-sized product, not the chip's headline bandwidth.
 *
 * Conventions as in snm.h: device pointers owned by the caller, work enqueued on `stream`
 * (a hipStream_t, NULL = default stream), host-side checks first, status codes of snm.h
 * (0 = SNM_OK). Nothing is allocated.
 */
#ifndef SNM_CEILINGS_H
#define SNM_CEILINGS_H

#include <stdint.h>

#include "snm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of src (16-byte aligned, bytes % 16 == 0) with 16-byte coalesced
 * loads, four in flight per lane. sink: 16 bytes of device memory, written only if the
 * XOR of the data equals a fixed 128-bit constant (it keeps the loads alive). */
snm_status snm_ceiling_read(const void* src, int64_t bytes, void* sink, void* stream);

/* Copies `bytes` bytes from src to dst (both 16-byte aligned, bytes % 16 == 0, not
 * overlapping) with 16-byte coalesced loads and stores. */
snm_status snm_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Global -> LDS copy loop (the DMA path through which the products stage their operands):
 * `workgroups` workgroups of 8 waves, one per CU, each wave copying 1 KiB per iteration
 * (16 bytes per lane, at most 16 copies in flight) for `iters` iterations from the first
 * window_bytes bytes of src into its own LDS ring. window_bytes: a power of two, at least
 * 1024 (a window of a few MiB stays in L2, so this measures how fast a CU fills its LDS from
 * L2); src holds window_bytes bytes, 16-byte aligned. out: one float per workgroup, 4-byte
 * aligned. Bytes moved per launch = workgroups * 8 * iters * 1024. */
snm_status snm_ceiling_lds_fill(const void* src, int64_t window_bytes, int64_t workgroups, int64_t iters,
                                float* out, void* stream);

/* Matrix-instruction issue loop: `workgroups` workgroups of 4 waves; every wave runs
 * `iters` iterations of 4 independent accumulator chains of one instruction on register
 * operands (no memory traffic), then writes one float per lane to out (workgroups * 256
 * floats, 4-byte aligned).
 *   kind 0: v_mfma_f32_32x32x16_f16,   2*32*32*16 = 32768 flops per instruction;
 *   kind 1: v_smfmac_f32_32x32x32_f16, 2*32*32*32 = 65536 flops per instruction (the
 *           dense equivalent of the 2:4 product, which is how the sparse peak counts).
 * Flops per launch = workgroups * 4 * iters * 4 * (flops per instruction). */
snm_status snm_ceiling_matrix(int kind, int64_t workgroups, int64_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SNM_CEILINGS_H */
