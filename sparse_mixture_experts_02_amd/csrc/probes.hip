// Measurement probes: kernels that measure this part's attainable matrix-core
// rate and HBM read rate under the conditions the layer runs in (clock under
// the power cap, the memory system's real efficiency), so that the layer's
// kernels can be reported against measured ceilings beside the published ones.
// They compute nothing of the layer.
//
//   mfma_probe: waves issue back-to-back v_mfma_f32_16x16x32_bf16 (the
//               instruction of the prefill GEMM tile) on register operands
//               (eight independent accumulators per wave, so that no MFMA
//               waits on the previous one's result); no memory traffic but one
//               word per lane at the end, which keeps the work live.  On
//               MI355X it sustains ~2.4 PFLOP/s where 32x32x16 ones stop at
//               ~1.97.
//   read_probe: a grid-stride read of a buffer in 16-byte loads (consecutive
//               lanes on consecutive addresses), summed per lane; one word per
//               lane written at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probes.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeWaves = 8;   // per block: two per SIMD, as the prefill GEMM tile
constexpr int kProbeChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(kProbeWaves * 64) void mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x4_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][3];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each byte is read once, so the loads carry the non-temporal hint (7.0 TB/s
// on MI355X against 6.4 TB/s without it).
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_probe_kernel(const probe_f32x4* __restrict__ p, int64_t n4, float* out) {
  probe_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) acc += __builtin_nontemporal_load(p + i);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

extern "C" {

int64_t moe_probe_mfma_flops(int32_t blocks, int32_t iters) {
  if (blocks <= 0 || iters <= 0) return 0;
  return (int64_t)blocks * kProbeWaves * iters * kProbeChains * (2LL * 16 * 16 * 32);
}

moe_status moe_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return MOE_EINVAL;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream),
                     iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

moe_status moe_probe_read(const void* buf, int64_t bytes, int32_t blocks, float* out, void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return MOE_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return MOE_EINVAL;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const probe_f32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

}  // extern "C"
