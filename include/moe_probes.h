/*
 * moe_probes.h -- measurement probes of the MI355X MoE library (libmoe.so).
 *
 * Not part of the layer: kernels that measure the part's attainable
 * matrix-core and HBM read rates, so that the layer's kernels can be reported
 * against measured ceilings beside the published peaks.  Same conventions as
 * moe.h (device pointers, asynchronous on `stream`, the caller owns every
 * buffer, arguments checked on the host before any launch).
 */
#ifndef MOE_MI355X_PROBES_H
#define MOE_MI355X_PROBES_H

#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_probe_mfma: `blocks` blocks of 8 waves, each wave issuing `iters`
 *   rounds of 8 independent v_mfma_f32_16x16x32_bf16 on register operands.
 *   out: device fp32, blocks * 512 elements (one word per lane, written so
 *   the work stays live; values meaningless).  MOE_EINVAL if blocks or iters
 *   <= 0 or out is NULL.
 * moe_probe_mfma_flops: the FLOPs one such launch performs (0 for bad sizes).
 * moe_probe_read: `blocks` blocks of 256 threads read `bytes` bytes of the
 *   device buffer `buf` once, in 16-byte non-temporal loads, grid-stride.  out: device
 *   fp32, blocks * 256 elements.  MOE_EINVAL if a pointer is NULL, buf is not
 *   16-byte aligned, bytes <= 0 or not a multiple of 16, or blocks <= 0. */
moe_status moe_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream);
int64_t moe_probe_mfma_flops(int32_t blocks, int32_t iters);
moe_status moe_probe_read(const void* buf, int64_t bytes, int32_t blocks, float* out, void* stream);

/*
 * moe_gemm_plan: host-only (no device call) description of the two grouped
 *   GEMMs a layer call with descriptor `d` runs: the gate_up GEMM (entries
 *   0..5) and the down GEMM (6..11) of the host array `plan` (12 int32, owned
 *   by the caller).  Per GEMM: kernel variant, rows per row tile, output
 *   columns per column tile, column tiles, whether the last partial round of
 *   work items may be split along K (0/1), and the work-list capacity.
 *   Variants: 0 generic 128-row tiles; 1 direct-to-LDS 256-row tiles with
 *   32-row tail strips; 2 direct-to-LDS 128-row tiles; 3 direct-to-LDS 32-row
 *   tiles; 4 generic 64-row tiles; 5 weight-streaming 32-row tiles of 256
 *   weight rows (bf16, contraction length a multiple of 512, output columns a
 *   multiple of 32); 6 the same with 128 weight rows per tile (never split).
 *   The plan depends on the descriptor only (the rows per expert enter through
 *   their mean, T*K/E).  Errors: as moe_workspace_bytes; MOE_EINVAL if plan
 *   is NULL.
 */
moe_status moe_gemm_plan(const moe_desc* d, int32_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_PROBES_H */
