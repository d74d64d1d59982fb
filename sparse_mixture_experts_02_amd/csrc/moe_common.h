// Internal declarations of the MI355X MoE forward path: device helpers shared
// by the kernels and the host-side launchers the C ABI sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "worklist.h"

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

// float -> bf16 bits, rounded to nearest even by gfx950's conversion
// instruction (v_cvt_pk_bf16_f32; a NaN stays a NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 bits (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_bits_to_f32(v); }

// --------------------------------------------------------- launch limits
constexpr int kMaxExperts = 256;
constexpr int kRouterTokens = 16;     // tokens per router block
constexpr int kDispatchChunk = 1024;  // assignments per count/scatter block

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
  // Routing options (all off when null / 0).
  const int64_t* replay;        // (T,K) recorded experts, or null
  const uint8_t* replay_mask;   // (T) nonzero: the record covers the token; null: all covered
  float threshold;              // dynamic threshold on renormalised weights, 0 = off
  uint8_t* kept;                // (T,K) 1/0 out, or null
  float* stats_part;            // (blocks, 3E) per-block sums of p, gate, [gate > 0], or null
};
hipError_t launch_router(int dtype, const RouterArgs& a, hipStream_t s);
inline int64_t router_blocks(int64_t T) { return (T + kRouterTokens - 1) / kRouterTokens; }

// Balancing statistics from the router's per-block sums: stats (3E + 4) =
// mean p (E), mean gate (E), mean [gate > 0] (E), switch, gshard, master,
// gshard_probs.
struct StatsArgs {
  const float* part;  // (blocks, 3E)
  int64_t blocks, T;
  int32_t E;
  float* stats;       // (3E + 4)
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t s);

// Capacity drops on a stable expert-sorted order: a sorted row whose rank
// among its expert's rows from the same sequence is >= slots is dropped: its
// assignment's expert becomes the sentinel E and its kept flag 0.
struct CapacityArgs {
  const int32_t* offsets;     // (E+1) of the sorted order
  const int32_t* sorted_tok;  // (M)
  const int32_t* sorted_slot; // (M)
  int32_t* sel32;             // (M) by assignment, updated
  uint8_t* kept;              // (M) by assignment, or null
  int64_t M;
  int64_t seq_len;
  int32_t E;
  int32_t slots;
};
hipError_t launch_capacity(const CapacityArgs& a, hipStream_t s);

// A grouped GEMM's work list: item b is one (expert, row tile, column tile).
// Items are ordered so that consecutive items share operands (all row tiles of
// one expert over a group of column tiles) and are laid out so that the items
// one XCD runs (blocks b with b % 8 == xcd) form one contiguous range of that
// order; the GEMM grid is sized by max_work and blocks b >= *num_work exit.
struct WorkSpec {
  int32_t bm;        // rows per tile
  // Tail rows an expert's last tile may add (0 or kTailRows).  The builder
  // uses them when that lowers the estimated number of rounds on `ncu`
  // compute units, and flags such a tile's first row with kTailTile.
  int32_t xr;
  int32_t ncu;
  int32_t ntn;       // column tiles
  int32_t max_work;  // upper bound of the item count (grid size)
  int2* work;        // (max_work) {expert | column_tile << 8, first sorted row}
  int32_t* num_work; // (1)
  // Split of the last partial round along K (0: off).  With `split_ncu`
  // compute units and `tiles` items, the R = tiles % split_ncu items past the
  // last full round are each cut into P = min(kMaxSplitParts, split_ncu / R)
  // K ranges (when P >= 2), so they fill one round of shorter blocks.  Such
  // an item in `work` is {kSplitItem | q, 0} with q = j*P + p: part p of
  // split tile j, whose {expert | column_tile << 8, first row} is
  // split_tiles[j].
  int32_t split_ncu;
  int2* split_tiles;   // (split_ncu)
  int32_t* split_info; // (2): R, P
  // Order in which the XCDs take the items: 1, 32-item windows dealt out in
  // turn (the 256-row tiles, whose rounds then share operands in
  // L2); 0, one contiguous range per XCD (the 32-row decode tile, a weight
  // stream, and the generic kernel).
  int32_t windows;
};

struct DispatchArgs {
  const int32_t* sel32;   // (M) expert of assignment i = t*K + k; E = dropped
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
  int32_t nspec;          // work lists to build (0..2)
  WorkSpec spec[2];
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

enum Epilogue { EPI_SWIGLU = 0, EPI_RELU = 1, EPI_DOWN_ATOMIC = 2, EPI_DOWN_SLOT = 3 };

// Kernel variants of the grouped GEMM.
//   GENERIC: any K / alignment, fp32 or bf16; 128x128 output tiles, operands
//            staged through registers into LDS (GENERIC_M64: 64-row tiles,
//            for GEMMs with too few 128-row items to fill two rounds).
//   BF16_Mxxx: bf16 with K a multiple of 64, or fp32 with K a multiple of 32
//            (whole 128-byte stages), 16-byte aligned rows; LDS stages filled
//            by direct global->LDS loads; xxx rows per tile (256 from 64
//            rows per expert on, 32 for decode-sized segments).  Value 2 is
//            retired (a 128-row tile, slower than the 256-row one).
enum Variant {
  VAR_GENERIC = 0,
  VAR_BF16_M256 = 1,
  VAR_BF16_M32 = 3,
  VAR_GENERIC_M64 = 4,
  VAR_BF16_S32 = 5,   // weight-streaming 32-row tiles of 256 weight rows (gemm_stream.hip)
  VAR_BF16_S32N = 6,  // the same with 128 weight rows per tile, never split along K
  VAR_BF16_S64N = 7,  // the narrow streaming tile over 64 sorted rows (two 32-row halves)
};
int variant_rows(int var);
int variant_cols(int var, bool dual);

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
  const int2* work;
  const int32_t* num_work;
  int32_t max_work;
  const int32_t* offsets;
  const float* bias;        // per-expert bias rows or null
  int64_t bias_estride;
  void* C;                  // h (G1) / out accumulation (G2 atomic) / slot rows (G2 slot)
  int64_t ldc;
  const int32_t* sorted_tok;
  const int32_t* sorted_slot;
  const float* sorted_w;
  int32_t vec_ok;           // rows 16-byte aligned: vector loads allowed
  // K-split items (256- and 32-row bf16 tiles, any epilogue but the atomic
  // combine): the partial sums of part p of split tile j go to partial +
  // (j*P + p) tiles of split_rows x kSplitTileCols fp32, reduced by
  // launch_split_fixup.
  const int2* split_tiles;
  const int32_t* split_info;
  float* partial;
  int32_t split_bm;         // rows per split tile (the kernel variant's tile height)
  int32_t split_rows;       // rows per partial tile in `partial`: split_bm plus the tail rows it may hold
};
hipError_t launch_grouped_gemm(int dtype, int epi, int var, const GemmArgs& a, hipStream_t s);
// Sums the K parts of every split tile in part order and applies the tile's
// epilogue `epi` (SwiGLU, ReLU or the down projection's slot store) to the
// sums.  Sixteen blocks per tile slot, `ncu` slots; blocks past R's exit.
constexpr int kSplitTileCols = 256;  // columns of a partial tile (rows: GemmArgs::split_rows)
hipError_t launch_split_fixup(int dtype, int epi, const GemmArgs& a, int32_t ncu, hipStream_t s);
// The direct-to-LDS variants (VAR_BF16_*) for dtype 1 (bf16) or 0 (fp32).
hipError_t launch_gemm_bf16(int dtype, int epi, int var, const GemmArgs& a, hipStream_t s);
// The weight-streaming variants (bf16 only): `strips` = 8 (VAR_BF16_S32) or
// 4 (VAR_BF16_S32N) strips of 32 weight rows per tile.
constexpr int kStreamChunk = 512;  // K elements per chunk of the weight-streaming kernel
hipError_t launch_gemm_stream(int epi, int strips, int rows, const GemmArgs& a, hipStream_t s);

struct FinalizeArgs {
  const float* src;   // slot rows (T*K, D) when K > 0 slots, or (T, D) accumulation
  void* out;          // (T, D)
  int64_t T, D;
  int32_t K;          // slots per token to sum (1 = plain copy/cast)
  int32_t out_bf16;
  const int32_t* slot_expert;  // (T*K) or null: slots whose entry is >= E were dropped and are skipped
  int32_t E;
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);

}  // namespace moe
