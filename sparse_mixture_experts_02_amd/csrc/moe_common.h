// Internal declarations of the MI355X MoE forward path: device helpers shared
// by the kernels and the host-side launchers the C ABI sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element tags.  bf16 travels as its 16-bit pattern.
struct F32 {
  typedef float elem;
  static constexpr int kBytes = 4;
};
struct BF16 {
  typedef uint16_t elem;
  static constexpr int kBytes = 2;
};

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_bits_to_f32(v); }

// --------------------------------------------------------- launch limits
constexpr int kMaxExperts = 256;
constexpr int kRouterTokens = 16;     // tokens per router block
constexpr int kDispatchChunk = 1024;  // assignments per count/scatter block
constexpr int kGemmBM = 128;          // rows (tokens) per grouped-GEMM tile

// ------------------------------------------------------------ launchers
struct RouterArgs {
  const void* x;
  const void* router;
  const float* router_bias;
  int64_t T, D;
  int32_t E, K, norm;
  float* logits;      // (T,E) or null
  int64_t* sel64;     // (T,K)
  int32_t* sel32;     // (T,K)
  float* weights;     // (T,K)
  float* zero_rows;   // (T,zero_cols) rows cleared by this kernel, or null
  int64_t zero_cols;
  int32_t vec_ok;     // x and router rows 16-byte aligned: vector loads allowed
};
hipError_t launch_router(int dtype, const RouterArgs& a, hipStream_t s);

struct DispatchArgs {
  const int32_t* sel32;   // (M) expert of assignment i = t*K + k
  const float* weights;   // (M)
  int64_t M;
  int32_t E, K;
  int32_t nchunks;
  int32_t* chunk_counts;  // (nchunks, E)
  int32_t* chunk_base;    // (nchunks, E)
  int32_t* counts;        // (E)
  int32_t* offsets;       // (E+1)
  int32_t* counts_out;    // (E) caller copy or null
  int32_t* offsets_out;   // (E+1) caller copy or null
  int32_t* sorted_tok;    // (M)
  int32_t* sorted_slot;   // (M)
  float* sorted_w;        // (M) or null
  // tile table for the grouped GEMMs: tile j covers rows [tile_r0[j],
  // min(tile_r0[j] + bm, offsets[tile_e[j]+1])) of expert tile_e[j].
  int32_t bm;
  int32_t max_tiles;
  int32_t* tile_e;
  int32_t* tile_r0;
  int32_t* num_tiles;     // (1)
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

enum Epilogue { EPI_SWIGLU = 0, EPI_RELU = 1, EPI_DOWN_ATOMIC = 2, EPI_DOWN_SLOT = 3 };

struct GemmArgs {
  const void* A;            // activation rows
  int64_t lda;
  const int32_t* a_index;   // row of A for sorted row r, or null (row r itself)
  const void* B;            // weights of expert 0: rows of length Kd
  int64_t ldb;
  int64_t b_estride;        // elements between experts
  int64_t up_off;           // rows between gate and up halves (SwiGLU)
  int64_t N;                // output columns
  int64_t Kd;               // contraction length
  const int32_t* tile_e;
  const int32_t* tile_r0;
  const int32_t* num_tiles;
  const int32_t* offsets;
  int32_t max_tiles;
  const float* bias;        // per-expert bias rows or null
  int64_t bias_estride;
  void* C;                  // h (G1) / out accumulation (G2 atomic) / slot rows (G2 slot)
  int64_t ldc;
  const int32_t* sorted_tok;
  const int32_t* sorted_slot;
  const float* sorted_w;
  int32_t vec_ok;           // rows 16-byte aligned: vector loads allowed
};
hipError_t launch_grouped_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s);

struct FinalizeArgs {
  const float* src;   // slot rows (T*K, D) when K > 0 slots, or (T, D) accumulation
  void* out;          // (T, D)
  int64_t T, D;
  int32_t K;          // slots per token to sum (1 = plain copy/cast)
  int32_t out_bf16;
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);

}  // namespace moe
