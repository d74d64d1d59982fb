// bf16 grouped expert GEMM for gfx950: the prefill- and decode-sized
// variants of the gate_up and down projections (epilogues in
// gemm_epilogue.h; arithmetic as in grouped_gemm.hip: fp32 accumulation, one
// rounding of h to bf16).
//
// Tile: BM sorted rows x 256 weight rows (SwiGLU: 128 gate + the 128 matching
// up rows, so 128 h columns; otherwise 256 output columns), K step 64.
// 4 waves: 2 x 2 for BM = 256 / 128 (a wave owns BM/2 rows x 128 weight rows),
// 1 x 4 for BM = 32 (32 rows x 64 weight rows).  MFMA v_mfma_f32_16x16x32_bf16
// with the weights as operand 0, so a lane's accumulators are four
// consecutive output columns of one row.
//
// Data path: global_load_lds_dwordx4 writes each 16-byte chunk straight from
// HBM/L2 into LDS (no staging registers), into two LDS stages held in two
// distinct arrays so the compiler sees that the loads in flight into one stage
// do not alias the MFMA fragment reads from the other.  Rows are 128 bytes in
// LDS with the 16-byte chunk index XOR-ed with (row & 7): a wave's fragment
// read of 16 rows at one chunk spreads over all banks.  A lane of a load
// instruction writes LDS byte 16*lane of an 8-row block, so it loads the
// global chunk that the swizzle puts there.  One barrier per K step: waves
// wait for their own loads (vmcnt 0), then the barrier publishes the stage and
// frees the other one for the next loads.
//
// Requires K % 64 == 0, 16-byte aligned operands, and operand regions under
// 4 GiB (32-bit byte offsets); the host routes anything else to the generic
// kernel.
#include "gemm_epilogue.h"
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One 16-byte chunk from global memory straight into LDS: lane l of the wave
// writes LDS bytes [dst + 16*l, dst + 16*l + 16); dst must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm0() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained (gfx9 encoding).
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

template <int EPI, int BM>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs a) {
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, SM = WM / 16;
  constexpr int NBR = 256;                      // weight rows per tile
  constexpr int OUTC = DUAL ? 128 : 256;        // output columns per tile
  constexpr int WN = OUTC / WAVES_N, SN = WN / 16;
  constexpr int NACC = DUAL ? 2 : 1;
  constexpr int AB = BM * 128;                  // A bytes per stage
  constexpr int STAGE = AB + NBR * 128;
  constexpr int AI = BM / 32;                   // A load instructions per wave
  constexpr int BI = NBR / 32;                  // B load instructions per wave

  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

  if ((int)blockIdx.x >= a.num_work[0]) return;
  const int2 wk = a.work[blockIdx.x];
  const int e = wk.x & 0xff;
  const int r0 = wk.y;
  const int rows = min(BM, a.offsets[e + 1] - r0);
  const int64_t n0 = (int64_t)(wk.x >> 8) * OUTC;
  const int64_t N = a.N;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / WAVES_N, wn = w % WAVES_N;

  // Load assignment: instruction i of wave w fills LDS rows 8*(w*XI+i) ..+7;
  // lane l writes physical chunk l%8 of row 8*(..)+l/8, which holds logical
  // chunk (l%8) ^ (l/8).
  const int lr = lane >> 3;
  const uint32_t lcb = (uint32_t)(((lane & 7) ^ lr) * 16);
  uint32_t aoff[AI], boff[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int rA = (w * AI + i) * 8 + lr;
    const int r = r0 + (rA < rows ? rA : 0);
    const int64_t src = a.a_index ? (int64_t)a.a_index[r] : (int64_t)r;
    aoff[i] = (uint32_t)(src * a.lda * 2) + lcb;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int rB = (w * BI + i) * 8 + lr;
    int64_t wr;
    if constexpr (DUAL) {
      const int64_t nn = n0 + (rB & (OUTC - 1));
      wr = (nn < N ? nn : N - 1) + (rB >= OUTC ? a.up_off : 0);
    } else {
      const int64_t nn = n0 + rB;
      wr = nn < N ? nn : N - 1;
    }
    boff[i] = (uint32_t)(wr * a.ldb * 2) + lcb;
  }
  const char* Abase = static_cast<const char*>(a.A);
  const char* Bbase = static_cast<const char*>(a.B) + (int64_t)e * a.b_estride * 2;

  auto issue = [&](int kt, char* dst) {
    const uint32_t kb = (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_dma16(Abase + (aoff[i] + kb), dst + (w * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_dma16(Bbase + (boff[i] + kb), dst + AB + (w * BI + i) * 1024);
  };

  f32x4 acc[NACC][SM][SN];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int mi = 0; mi < SM; ++mi)
#pragma unroll
      for (int ni = 0; ni < SN; ++ni) acc[q][mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, l16 = lane & 15;
  // Fragment addresses (bytes inside a stage): row*128 + swizzled chunk.
  const int arow = wm * WM + l16;
  const int brow = wn * WN + l16;
  int co[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) co[s] = ((s * 4 + g) ^ (l16 & 7)) * 16;

  // One K step from one LDS stage: two sub-steps of 32 k.  A "group" is the
  // NACC*SN MFMAs of one A fragment.  Reads are spread over the groups so that
  // each one is issued a whole group before its use: the A fragments two
  // groups ahead, the second sub-step's B fragments one per group of the first
  // sub-step, and its first two A fragments during the last two groups.  Only
  // the first sub-step's B fragments and first A fragments wait on LDS, once
  // per stage.  Scheduling barriers keep that order.
  constexpr int NB = NACC * SN;
  auto rdA = [&](const char* buf, int s, int mi) {
    return *reinterpret_cast<const bf16x8*>(buf + (arow + mi * 16) * 128 + co[s]);
  };
  auto rdB = [&](const char* buf, int s, int j) {
    return *reinterpret_cast<const bf16x8*>(buf + AB + ((j / SN) * OUTC + brow + (j % SN) * 16) * 128 + co[s]);
  };
  auto compute = [&](const char* buf) {
    bf16x8 fa0[SM], fa1[SM], fb0[NB], fb1[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) fb0[j] = rdB(buf, 0, j);
    fa0[0] = rdA(buf, 0, 0);
    if (SM > 1) fa0[1] = rdA(buf, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < SM; ++mi) {
      if (mi + 2 < SM) fa0[mi + 2] = rdA(buf, 0, mi + 2);
      if (mi + 2 == SM) fa1[0] = rdA(buf, 1, 0);
      if (mi + 1 == SM && SM > 1) fa1[1] = rdA(buf, 1, 1);
#pragma unroll
      for (int j = mi * NB / SM; j < (mi + 1) * NB / SM; ++j) fb1[j] = rdB(buf, 1, j);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j / SN][mi][j % SN] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0[j], fa0[mi], acc[j / SN][mi][j % SN], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mi = 0; mi < SM; ++mi) {
      if (mi + 2 < SM) fa1[mi + 2] = rdA(buf, 1, mi + 2);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j / SN][mi][j % SN] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb1[j], fa1[mi], acc[j / SN][mi][j % SN], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = (int)(a.Kd / 64);
  issue(0, lds);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm0();
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, lds + ((kt + 1) & 1) * STAGE);
    compute(lds + (kt & 1) * STAGE);
  }
  wait_vm0();  // no LDS DMA may outlive the workgroup

  const float* bias = a.bias ? a.bias + (int64_t)e * a.bias_estride : nullptr;
#pragma unroll
  for (int mi = 0; mi < SM; ++mi) {
    const int m = wm * WM + mi * 16 + l16;
    if (m >= rows) continue;
    const RowCtx rc = row_ctx<EPI>(a, r0 + m);
#pragma unroll
    for (int ni = 0; ni < SN; ++ni)
      epilogue4<uint16_t, EPI>(a, rc, n0 + wn * WN + ni * 16 + 4 * g, acc[0][mi][ni], acc[NACC - 1][mi][ni], bias);
  }
}

template <int EPI>
hipError_t launch_rows(int var, const GemmArgs& a, hipStream_t s) {
  switch (var) {
    case VAR_BF16_M256:
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 256>), dim3(a.max_work), dim3(kThreads), 0, s, a);
      break;
    case VAR_BF16_M128:
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 128>), dim3(a.max_work), dim3(kThreads), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 32>), dim3(a.max_work), dim3(kThreads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, int var, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return launch_rows<EPI_SWIGLU>(var, a, s);
    case EPI_RELU: return launch_rows<EPI_RELU>(var, a, s);
    case EPI_DOWN_ATOMIC: return launch_rows<EPI_DOWN_ATOMIC>(var, a, s);
    default: return launch_rows<EPI_DOWN_SLOT>(var, a, s);
  }
}

}  // namespace moe
