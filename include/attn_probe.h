/*
 * attn_probe.h - measurement helper of libattn.so (not part of the attention
 * computation): the rate at which the MI355X matrix cores run
 * v_mfma_f32_32x32x16_bf16 or v_mfma_f32_16x16x32_bf16 on given operands. bench.py uses it to state the
 * ceiling that the attention kernels' achieved MFMA throughput is compared
 * with, since the chip's clock under sustained matrix work depends on the
 * operands' bit patterns (power management).
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* 16-bit elements `src` must hold for `blocks` workgroups (16 per thread,
 * 512 threads per workgroup). */
size_t attn_probe_mfma_src_elems(int blocks);

/*
 * Enqueues `blocks` workgroups of 8 waves (two per SIMD); each wave reads 16
 * bf16 values per lane from `src` once (the A and B operands) and issues
 * 8 * iters v_mfma_f32_32x32x16_bf16 products (32 * 32 * 16 * 2 flops each)
 * round-robin into `chains` (1, 2, 4 or 8) independent accumulators, then
 * writes one float per thread to `dst` (blocks * 512 floats). Flops per
 * call: blocks * 8 * 8 * iters * 32768, whatever `chains`. Device pointers,
 * caller owned, 16-byte aligned src. ATTN_ERR_NULL, ATTN_ERR_SHAPE (blocks
 * not in [1, 2^20], iters not in [1, 2^24], or another chain count) or
 * ATTN_ERR_HIP; asynchronous.
 */
attn_status attn_probe_mfma_rate(const void* src, float* dst, int blocks, int iters, int chains,
                                 hipStream_t stream);

/*
 * The same probe on v_mfma_f32_16x16x32_bf16 (16 * 16 * 32 * 2 flops each):
 * each wave issues 16 * iters products round-robin into `chains` (1, 2, 4 or
 * 8) independent 16x16 accumulators, so the flops per call are those of
 * attn_probe_mfma_rate with the same blocks and iters. Same arguments,
 * ownership and errors.
 */
attn_status attn_probe_mfma16_rate(const void* src, float* dst, int blocks, int iters, int chains,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
