// Epilogues of the grouped expert GEMMs, shared by the kernel variants.  A
// lane owns four consecutive output columns nb..nb+3 of one sorted row r.
//
//   SwiGLU:  h = silu(g) * u with g, u the gate and up accumulators (+ bias),
//            rounded once to the compute dtype (mojolearn "MoEBlock": each
//            chosen expert computes down_proj(silu(gate) * up)).
//   ReLU:    h = max(0, acc + b1) (crackedaicode "Mixture-of-Experts FFN":
//            Dense(F) -> ReLU).
//   down:    v = w_r * (acc + b2), then either added into out[token] with fp32
//            atomics, or stored into the (t,k) slot row for an ordered sum
//            (same exercise, "Weight the selected outputs").
#pragma once

#include "moe_common.h"

namespace moe {

template <typename elem>
__device__ __forceinline__ void store4(elem* dst, int64_t nb, int64_t N, bool vec4, const float (&v)[4]) {
  if constexpr (sizeof(elem) == 2) {
    if (vec4 && nb + 4 <= N) {
      uint2 pk;
      pk.x = f32x2_to_bf16x2_bits(v[0], v[1]);
      pk.y = f32x2_to_bf16x2_bits(v[2], v[3]);
      *reinterpret_cast<uint2*>(dst + nb) = pk;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) dst[nb + i] = (uint16_t)f32_to_bf16_bits(v[i]);
    }
  } else {
    if (vec4 && nb + 4 <= N) {
      *reinterpret_cast<float4*>(dst + nb) = float4{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) dst[nb + i] = v[i];
    }
  }
}

// Per-row context of the epilogue.
struct RowCtx {
  int64_t orow;  // output row: sorted row (h), token (atomic combine) or slot
  float wgt;     // routing weight of the row (down projection)
};

template <int EPI>
__device__ __forceinline__ RowCtx row_ctx(const GemmArgs& a, int r) {
  RowCtx c{r, 1.f};
  if constexpr (EPI == EPI_DOWN_ATOMIC) {
    c.orow = a.sorted_tok[r];
    c.wgt = a.sorted_w[r];
  } else if constexpr (EPI == EPI_DOWN_SLOT) {
    c.orow = a.sorted_slot[r];
    c.wgt = a.sorted_w[r];
  }
  return c;
}

// acc0: gate (SwiGLU) or the only accumulator; acc1: up (SwiGLU only).
template <typename elem, int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, const RowCtx& rc, int64_t nb, const f32x4& acc0,
                                          const f32x4& acc1, const float* bias) {
  const int64_t N = a.N;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = nb + i;
    const bool ok = n < N;
    if constexpr (EPI == EPI_SWIGLU) {
      float g = acc0[i], u = acc1[i];
      if (bias && ok) {
        g += bias[n];
        u += bias[a.up_off + n];
      }
      // silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) and the
      // hardware reciprocal (about 1 ulp each, far below the bf16 rounding
      // of h that follows)
      v[i] = g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g)) * u;
    } else if constexpr (EPI == EPI_RELU) {
      float t = acc0[i];
      if (bias && ok) t += bias[n];
      v[i] = fmaxf(t, 0.f);
    } else {
      float t = acc0[i];
      if (bias && ok) t += bias[n];
      v[i] = rc.wgt * t;
    }
  }
  const bool vec4 = (a.ldc & 3) == 0;
  if constexpr (EPI == EPI_DOWN_ATOMIC) {
    float* dst = static_cast<float*>(a.C) + rc.orow * a.ldc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nb + i < N) unsafeAtomicAdd(dst + nb + i, v[i]);
  } else if constexpr (EPI == EPI_DOWN_SLOT) {
    store4<float>(static_cast<float*>(a.C) + rc.orow * a.ldc, nb, N, vec4, v);
  } else {
    store4<elem>(static_cast<elem*>(a.C) + rc.orow * a.ldc, nb, N, vec4, v);
  }
}

// The same epilogue for four columns that all lie inside N, with no bias and
// 16-byte aligned rows (the caller checks both once per tile): no per-column
// checks, one vector store to `dst` (the row's column nb).  SwiGLU, ReLU and
// the slot store only (the atomic combine keeps epilogue4).
template <typename elem, int EPI>
__device__ __forceinline__ void epilogue4_inner(elem* dst, float wgt, const f32x4& acc0, const f32x4& acc1) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (EPI == EPI_SWIGLU) {
      const float g = acc0[i], u = acc1[i];
      v[i] = g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g)) * u;
    } else if constexpr (EPI == EPI_RELU) {
      v[i] = fmaxf(acc0[i], 0.f);
    } else {
      v[i] = wgt * acc0[i];
    }
  }
  if constexpr (sizeof(elem) == 2) {
    uint2 pk;
    pk.x = f32x2_to_bf16x2_bits(v[0], v[1]);
    pk.y = f32x2_to_bf16x2_bits(v[2], v[3]);
    *reinterpret_cast<uint2*>(dst) = pk;
  } else {
    *reinterpret_cast<float4*>(dst) = float4{v[0], v[1], v[2], v[3]};
  }
}

}  // namespace moe
