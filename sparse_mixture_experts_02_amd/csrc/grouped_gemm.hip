// Grouped expert GEMMs over the expert-sorted rows, with fused epilogues.
//
//   gate_up (SwiGLU): h[r, n] = silu(x_r . Wgu[e][n]) * (x_r . Wgu[e][F + n])
//                     (gate = rows [0,F) of gate_up_proj[e], up = rows [F,2F);
//                     mojolearn "MoEBlock" class description and "Variables")
//   gate_up (ReLU):   h[r, n] = max(0, x_r . W1[e][n] + b1[e][n])
//                     (crackedaicode "Mixture-of-Experts FFN", section
//                     "Compute the experts and router")
//   down:             y[r, n] = h_r . Wd[e][n] (+ b2[e][n]); the routing weight
//                     of row r scales y, which is then added into the token's
//                     output row (the combine of the same exercise, section
//                     "Weight the selected outputs"), either with fp32 atomics
//                     or into the row's own (t,k) slot for an ordered sum.
//
// Rows r are assignments in expert-contiguous order; a work item covers up to
// 128 rows of one expert and 128 output columns (this generic variant).  x
// rows are gathered through the sorted token ids while they are loaded, so no
// permuted copy of x exists.
// Every contraction accumulates in fp32 and the gate_up result is rounded
// once to the compute dtype (Dew "Mixture of experts" page, section "Expert
// computation and placement").
//
// Kernel shape (both dtypes): 256 threads = 2 x 2 waves; tile BM=128 rows x
// BN=128 output columns (SwiGLU: 128 gate + 128 up weight rows); a K step is
// 128 bytes of every row (64 bf16 or 32 fp32).  Operands go HBM -> registers ->
// LDS (16-byte chunks, XOR-swizzled by row so MFMA fragment reads spread over
// the banks); the next K step's global loads are in flight while the MFMAs
// consume the current one.  Weights are MFMA operand 0 and activations operand
// 1, so each lane's four accumulators are four consecutive output columns of
// one row.
#include "gemm_epilogue.h"
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename Tag>
struct Frag;
template <>
struct Frag<BF16> {
  static constexpr int kEPC = 8;  // elements per 16-byte chunk
};
template <>
struct Frag<F32> {
  static constexpr int kEPC = 4;
};

template <typename Tag>
__device__ __forceinline__ uint4 load_chunk(const typename Tag::elem* row, int64_t k, int64_t kd, bool vec) {
  constexpr int EPC = Frag<Tag>::kEPC;
  if (vec && k + EPC <= kd) return *reinterpret_cast<const uint4*>(row + k);
  union {
    typename Tag::elem e[EPC];
    uint4 v;
  } t;
#pragma unroll
  for (int j = 0; j < EPC; ++j) t.e[j] = (k + j < kd) ? row[k + j] : (typename Tag::elem)0;
  return t.v;
}

template <typename Tag, int EPI, int BM, int BN>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs a) {
  using elem = typename Tag::elem;
  constexpr int EPC = Frag<Tag>::kEPC;
  constexpr int BK = 8 * EPC;
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int NB = DUAL ? 2 * BN : BN;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int SM = WTM / 16, SN = WTN / 16;
  constexpr int LA = BM / 32, LB = NB / 32;  // 16-byte loads per thread per K step
  constexpr int NACC = DUAL ? 2 : 1;

  __shared__ uint4 As[BM * 8];
  __shared__ uint4 Bs[NB * 8];

  if ((int)blockIdx.x >= a.num_work[0]) return;
  const int2 wk = a.work[blockIdx.x];
  const int e = item_expert(wk);
  const int r0 = item_first_row(wk);  // the generic lists have neither tails nor splits
  const int rows = item_rows(a.offsets[e + 1] - r0, false, BM, 0);
  const int64_t n0 = (int64_t)item_col_tile(wk) * BN;
  const int64_t N = a.N, Kd = a.Kd;
  const bool vec = a.vec_ok != 0;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int c = tid & 7, rr = tid >> 3;

  const elem* Ab = static_cast<const elem*>(a.A);
  const elem* Bb = static_cast<const elem*>(a.B) + (int64_t)e * a.b_estride;
  const elem* pa[LA];
  const elem* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int lr = rr + 32 * i;
    const int r = r0 + (lr < rows ? lr : 0);
    const int64_t src = a.a_index ? (int64_t)a.a_index[r] : (int64_t)r;
    pa[i] = Ab + src * a.lda;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int lb = rr + 32 * i;
    int64_t wr;
    if (DUAL) {
      const int64_t nn = n0 + (lb % BN);
      wr = (nn < N ? nn : N - 1) + (lb / BN) * a.up_off;
    } else {
      const int64_t nn = n0 + lb;
      wr = nn < N ? nn : N - 1;
    }
    pb[i] = Bb + wr * a.ldb;
  }

  uint4 ra[LA], rb[LB];
  auto gload = [&](int64_t k0) {
    const int64_t k = k0 + c * EPC;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = load_chunk<Tag>(pa[i], k, Kd, vec);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = load_chunk<Tag>(pb[i], k, Kd, vec);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int lr = rr + 32 * i;
      As[lr * 8 + (c ^ (lr & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int lb = rr + 32 * i;
      Bs[lb * 8 + (c ^ (lb & 7))] = rb[i];
    }
  };

  f32x4 acc[NACC][SM][SN];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int mi = 0; mi < SM; ++mi)
#pragma unroll
      for (int ni = 0; ni < SN; ++ni) acc[q][mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, l16 = lane & 15;
  const int nk = (int)((Kd + BK - 1) / BK);
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = s * 4 + g;
      uint4 fa[SM], fb[NACC][SN];
#pragma unroll
      for (int mi = 0; mi < SM; ++mi) {
        const int row = wm * WTM + mi * 16 + l16;
        fa[mi] = As[row * 8 + (cc ^ (row & 7))];
      }
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int ni = 0; ni < SN; ++ni) {
          const int row = q * BN + wn * WTN + ni * 16 + l16;
          fb[q][ni] = Bs[row * 8 + (cc ^ (row & 7))];
        }
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int mi = 0; mi < SM; ++mi)
#pragma unroll
          for (int ni = 0; ni < SN; ++ni) {
            if constexpr (EPC == 8) {
              acc[q][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, fb[q][ni]), __builtin_bit_cast(bf16x8, fa[mi]), acc[q][mi][ni], 0, 0, 0);
            } else {
              const float4 bv = __builtin_bit_cast(float4, fb[q][ni]);
              const float4 av = __builtin_bit_cast(float4, fa[mi]);
              acc[q][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv.x, av.x, acc[q][mi][ni], 0, 0, 0);
              acc[q][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv.y, av.y, acc[q][mi][ni], 0, 0, 0);
              acc[q][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv.z, av.z, acc[q][mi][ni], 0, 0, 0);
              acc[q][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv.w, av.w, acc[q][mi][ni], 0, 0, 0);
            }
          }
    }
    __syncthreads();
    if (kt + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // Epilogue.  Lane holds rows m = wm*WTM + mi*16 + l16 and columns
  // n = n0 + wn*WTN + ni*16 + 4g + i, i = 0..3.
  const float* bias = a.bias ? a.bias + (int64_t)e * a.bias_estride : nullptr;
#pragma unroll
  for (int mi = 0; mi < SM; ++mi) {
    const int m = wm * WTM + mi * 16 + l16;
    if (m >= rows) continue;
    const RowCtx rc = row_ctx<EPI>(a, r0 + m);
#pragma unroll
    for (int ni = 0; ni < SN; ++ni)
      epilogue4<elem, EPI>(a, rc, n0 + wn * WTN + ni * 16 + 4 * g, acc[0][mi][ni], acc[NACC - 1][mi][ni], bias);
  }
}

template <typename Tag, int EPI, int BM>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<Tag, EPI, BM, 128>), dim3(a.max_work), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename Tag, int BM>
hipError_t launch_tag(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return launch_epi<Tag, EPI_SWIGLU, BM>(a, s);
    case EPI_RELU: return launch_epi<Tag, EPI_RELU, BM>(a, s);
    case EPI_DOWN_ATOMIC: return launch_epi<Tag, EPI_DOWN_ATOMIC, BM>(a, s);
    default: return launch_epi<Tag, EPI_DOWN_SLOT, BM>(a, s);
  }
}

// out[t, :] = sum over k ascending of src[t*K + k, :] (K = 1: a copy or
// cast), four columns per thread when the rows are 16-byte aligned.  The
// slot rows are read once, with the non-temporal hint (the 128-expert
// layer's 1.07 GB of slot rows: 0.253 -> 0.208 ms).
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeArgs a) {
  const int64_t D = a.D;
  if ((D & 3) == 0) {
    const int64_t n4 = a.T * D / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
      const int64_t t = (i * 4) / D, d = i * 4 - t * D;
      float4 s = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < a.K; ++k) {
        if (a.slot_expert && a.slot_expert[t * a.K + k] >= a.E) continue;
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.src + (t * a.K + k) * D + d));
        s.x += v[0];
        s.y += v[1];
        s.z += v[2];
        s.w += v[3];
      }
      if (a.out_bf16) {
        uint2 pk;
        pk.x = f32x2_to_bf16x2_bits(s.x, s.y);
        pk.y = f32x2_to_bf16x2_bits(s.z, s.w);
        reinterpret_cast<uint2*>(a.out)[i] = pk;
      } else {
        reinterpret_cast<float4*>(a.out)[i] = s;
      }
    }
    return;
  }
  const int64_t n = a.T * D;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t t = idx / D, d = idx - t * D;
    float s = 0.f;
    for (int k = 0; k < a.K; ++k)
      if (!a.slot_expert || a.slot_expert[t * a.K + k] < a.E) s += __builtin_nontemporal_load(a.src + (t * a.K + k) * D + d);
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[idx] = (uint16_t)f32_to_bf16_bits(s);
    else
      static_cast<float*>(a.out)[idx] = s;
  }
}

}  // namespace

int variant_rows(int var) {
  switch (var) {
    case VAR_BF16_M256: return 256;
    case VAR_BF16_M32:
    case VAR_BF16_S32:
    case VAR_BF16_S32N: return 32;
    case VAR_BF16_S64N: return 64;
    case VAR_GENERIC_M64: return 64;
    default: return 128;
  }
}

int variant_cols(int var, bool dual) {
  if (var == VAR_GENERIC || var == VAR_GENERIC_M64) return 128;
  if (var == VAR_BF16_S32N || var == VAR_BF16_S64N) return dual ? 64 : 128;
  return dual ? 128 : 256;
}

hipError_t launch_grouped_gemm(int dtype, int epi, int var, const GemmArgs& a, hipStream_t s) {
  if (a.max_work <= 0 || a.N <= 0) return hipSuccess;
  if (var == VAR_GENERIC_M64) return dtype == 1 ? launch_tag<BF16, 64>(epi, a, s) : launch_tag<F32, 64>(epi, a, s);
  if (var == VAR_BF16_S32 || var == VAR_BF16_S32N || var == VAR_BF16_S64N)
    return dtype == 1 ? launch_gemm_stream(epi, var == VAR_BF16_S32 ? 8 : 4, var == VAR_BF16_S64N ? 64 : 32, a, s)
                      : hipErrorInvalidValue;
  if (var != VAR_GENERIC) return launch_gemm_bf16(dtype, epi, var, a, s);
  return dtype == 1 ? launch_tag<BF16, 128>(epi, a, s) : launch_tag<F32, 128>(epi, a, s);
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  const int64_t n = a.T * a.D;
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(finalize_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
