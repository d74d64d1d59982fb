// Weight-streaming grouped GEMM for decode-sized expert segments (bf16, 32
// or 64 rows per expert tile): the gate_up and down projections when each
// expert holds only a few tokens, so the product is bound by reading the
// active experts' weights once from HBM (the Dew "Mixture of experts" page,
// section "Expert computation and placement": the sorted rows of each expert
// run as one grouped product; epilogues as in gemm_epilogue.h).
//
// Tile: up to 32 (or, narrow, 64) sorted rows x 32*NS weight rows, NS = 8 or 4 strips of 32
// (SwiGLU: NS/2 gate strips and the matching up strips -> 16*NS h columns).
// The wide tile (NS = 8) has the shape of gemm_bf16.hip's 32-row tile, with
// its work lists and K split; the narrow one (NS = 4) has twice the column
// tiles and never splits (the host plan picks between them from the
// estimated makespan, so that a GEMM whose narrow items fill whole rounds of
// the CUs needs no fix-up kernel).  What differs from
// gemm_bf16.hip is the order in which the weights are read.  HBM serves a
// weight tile read as 32 rows x 1 KB per step about a fifth faster than as
// 256 rows x 128 bytes per step (a read probe over the Mixtral-shaped gate_up
// weights: 6.27 against 5.25 TB/s): the long runs stay in the DRAM pages they
// open.  So the K range is walked in chunks of 512 (1 KB of every row) and
// each chunk in NS stages of one 32-row weight strip (32 KB, one 1 KB row per
// load instruction).  The four waves split each chunk along K (128 each) and
// hold partial sums for all NS strips; they meet once, in LDS, at the end of
// the tile, summed in wave order (reproducible).  The activation rows go
// straight to registers as MFMA fragments (they are small and every tile of
// an expert reads the same rows, so they come from L2); the weights, read
// once, go around the caches (non-temporal loads, below).
//
// LDS: five weight stages of 32 KB; rows are 1 KB with the 16-byte chunk
// index XOR-ed with the row's low four bits, so the 32 rows of a fragment read
// fall on distinct banks in each 16-lane phase.
//
// Requires bf16, K a multiple of 512, N a multiple of 32 and operands under
// 4 GiB of byte offsets (the host plan selects this kernel only then).
#include <type_traits>

#include "gemm_epilogue.h"
#include "moe_common.h"

namespace moe {
namespace {

// Cache policy of the weight loads: each weight byte is read once per layer
// call, so the loads carry the non-temporal hint (the NT bit of gfx950's
// cache-policy field) and do not displace the activation rows and the rest
// of the caches' contents.  Measured on the 64-token Mixtral-shaped layer:
// gate_up 0.310 -> 0.297 ms, down 0.168 -> 0.146 ms.  (On the prefill GEMM,
// whose operands are re-read from L2 by neighbouring tiles, the same hint
// costs 7-50%.)
constexpr int kWeightCachePolicy = 2;

__device__ __forceinline__ void lds_dma16_stream(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kWeightCachePolicy);
}

// Wait until at most N vector-memory loads of this wave are in flight and
// all of its LDS reads have returned (so no read of a stage can still be
// pending when the barrier that follows frees its buffer for new loads).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kKC = kStreamChunk;  // k per chunk: 1 KB of every bf16 row
constexpr int kRowB = kKC * 2;      // bytes per LDS row
constexpr int kStrip = 32;          // weight rows per stage
constexpr int kStages = 5;          // weight stages in LDS (160 KB), four in flight
constexpr int kStageB = kStrip * kRowB;  // 32 KB
constexpr int kLoads = kStrip / 4;  // load instructions per wave per stage (one row each)

template <int V>
using IC = std::integral_constant<int, V>;

// RH: 32-row halves per tile.  RH = 2 (narrow tiles only) takes 64 sorted
// rows: each weight stage read from HBM feeds the MFMAs of both halves, so
// an expert with 33-64 rows reads its weights once instead of twice.
template <int EPI, int NS, int RH>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a) {
  static_assert(NS == 8 || NS == 4, "strips per tile");
  static_assert(RH == 1 || (RH == 2 && NS == 4), "64-row tiles are narrow");
  using elem = uint16_t;
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int OUTC = DUAL ? 16 * NS : 32 * NS;  // output columns per tile
  constexpr int BM = 32 * RH;
  // LDS: weight stages 0..4; reused at the end for the four waves' partial
  // sums (4 x RH x NS x 4 KB).
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageB];
  char* const bbuf = lds;

  if ((int)blockIdx.x >= a.num_work[0]) return;
  const int nch = (int)(a.Kd / kKC);
  constexpr bool SPLITTABLE = EPI != EPI_DOWN_ATOMIC && NS == 8 && RH == 1;
  int2 wk = a.work[blockIdx.x];
  int c0 = 0, c1 = nch, split_slot = -1;
  if constexpr (SPLITTABLE) {
    if (item_is_split(wk)) {
      // part p of P covers chunks [p*nch/P, (p+1)*nch/P): any partition of
      // the K range is summed by the fix-up
      const int P = a.split_info[1];
      int j, p;
      split_part(wk, P, &j, &p);
      wk = a.split_tiles[j];
      split_k_range(p, P, nch, &c0, &c1);
      split_slot = j * P + p;
    }
  }
  const int e = item_expert(wk);
  const int r0 = item_first_row(wk);
  const int rows = item_rows(a.offsets[e + 1] - r0, false, BM, 0);
  const int64_t n0 = (int64_t)item_col_tile(wk) * OUTC;
  const int64_t N = a.N;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  // Activations go straight to registers as MFMA fragments: lane (l32, h)
  // of wave w holds, for 16-k slice s of the wave's quarter of a chunk, the
  // 8 elements of sorted row 32hh + l32 of half hh at chunk-local 16-byte
  // chunk 16w + 2s + h (rows past the segment repeat its first row).
  const char* arow[RH];
#pragma unroll
  for (int hh = 0; hh < RH; ++hh) {
    const int m = 32 * hh + l32;
    const int r = r0 + (m < rows ? m : 0);
    const int64_t src = a.a_index ? (int64_t)a.a_index[r] : (int64_t)r;
    arow[hh] = static_cast<const char*>(a.A) + src * a.lda * 2 + (16 * w + h) * 16;
  }
  // Chunk i of this item's walk is chunk c0 + (i + rot) mod (c1 - c0): the
  // items of an XCD start their K walks at different chunks, so at any time
  // its CUs read different K offsets of their rows rather than the same one
  // (the decode gate_up stream 3% faster; the sums change order only).
  const int rot = (int)((blockIdx.x >> 3) % (unsigned)(c1 - c0));
  auto chk = [&](int i) {
    const int x = i + rot;
    return c0 + (x >= c1 - c0 ? x - (c1 - c0) : x);
  };
  auto load_a = [&](bf16x8 (&f)[RH][8], int c) {
#pragma unroll
    for (int hh = 0; hh < RH; ++hh) {
      const char* p = arow[hh] + (int64_t)c * kRowB;
#pragma unroll
      for (int s = 0; s < 8; ++s) f[hh][s] = *reinterpret_cast<const bf16x8*>(p + 32 * s);
    }
  };

  // Weights.  Wave w fills rows 8w .. 8w+7 of a 32-row stage, one 1 KB row
  // per instruction; lane l writes LDS bytes [16l, 16l+16) of the row, which
  // hold the row's 16-byte chunk l ^ (row & 15).
  const char* Bbase = static_cast<const char*>(a.B) + (int64_t)e * a.b_estride * 2;
  // First weight row of strip j.  N is a multiple of 32, so a strip lies
  // wholly inside or wholly past the N output rows; one past them re-reads
  // the last strip (its sums are not stored).  SwiGLU: strips [0, NS/2) are
  // gate rows, [NS/2, NS) the matching up rows.
  auto strip_row = [&](int j) -> int64_t {
    if constexpr (DUAL) {
      const int64_t nn = n0 + (j % (NS / 2)) * kStrip;
      return (nn < N ? nn : N - kStrip) + (j >= NS / 2 ? a.up_off : 0);
    } else {
      const int64_t nn = n0 + j * kStrip;
      return nn < N ? nn : N - kStrip;
    }
  };
  // per-lane byte offsets of this wave's rows inside a strip: row 8w + q
  const int64_t ldb_b = a.ldb * 2;
  uint32_t boff[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q)
    boff[q] = (uint32_t)((8 * w + q) * ldb_b) + (uint32_t)((lane ^ ((8 * w + q) & 15)) * 16);
  // stage st (0-based in this item) = strip st % NS of chunk chk(st / NS), in
  // LDS buffer st % kStages
  auto issue_b = [&](int st, int buf) {
    const int j = st % NS;
    const char* src = Bbase + strip_row(j) * ldb_b + (int64_t)chk(st / NS) * kRowB;
    char* dst = bbuf + buf * kStageB;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) lds_dma16_stream(src + boff[q], dst + (8 * w + q) * kRowB);
  };
  // weight fragment of slice s: row l32, logical chunk 16w + 2s + h
  auto frag = [&](const char* buf, int s) {
    const int ch = (16 * w + 2 * s + h) ^ (l32 & 15);
    return *reinterpret_cast<const bf16x8*>(buf + l32 * kRowB + ch * 16);
  };

  f32x16 acc[RH][NS];
#pragma unroll
  for (int hh = 0; hh < RH; ++hh)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[hh][j] = f32x16{};
  bf16x8 af[RH][8], an[RH][8];

  const int nst = (c1 - c0) * NS;  // >= NS
  // Prologue: the first chunk's activations, then weight stages 0..3.
  load_a(af, chk(0));
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) issue_b(t, t);
  int rb = 0;  // LDS buffer of the current stage (st % kStages)

  // Stage st: wait for this wave's loads of stage st, barrier (stage st
  // visible to all waves, all waves done with stage st-1), issue stage st+4
  // into stage st-1's buffer (ISSUE), load the next chunk's activations into
  // registers (NEXTA; used from that chunk's first stage on), read the eight
  // weight fragments, 8 MFMAs.  cur: this chunk's activation fragments, nxt:
  // the next chunk's (two register sets that swap roles chunk by chunk, so no
  // copy ever waits for a load).  WAIT, in stages of kLoads loads: this
  // wave's loads issued after stage st's weights that may stay in flight
  // (the tables at `chunk`).
  auto stage = [&](int st, bf16x8 (&cur)[RH][8], bf16x8 (&nxt)[RH][8], auto J_, auto ISSUE_, auto NEXTA_,
                   auto WAIT_) {
    constexpr int J = decltype(J_)::value, WAIT = decltype(WAIT_)::value;
    constexpr bool ISSUE = decltype(ISSUE_)::value, NEXTA = decltype(NEXTA_)::value;
    wait_vm<WAIT * kLoads>();
    barrier_lds();
    if constexpr (ISSUE) issue_b(st + kStages - 1, rb == 0 ? kStages - 1 : rb - 1);
    if constexpr (NEXTA) load_a(nxt, chk(st / NS + 1));
    // all eight weight fragments first: one LDS round trip per stage
    const char* buf = bbuf + rb * kStageB;
    bf16x8 bf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) bf[s] = frag(buf, s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hh = 0; hh < RH; ++hh)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc[hh][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s], cur[hh][s], acc[hh][J], 0, 0, 0);
    rb = rb == kStages - 1 ? 0 : rb + 1;
  };
  constexpr std::true_type Y{};
  constexpr std::false_type Nn{};
  // Wait counts, in stages: the loads issued after stage st's weights.  Issue
  // order per stage t: the weights of t+4, then (NEXTA) the next chunk's
  // activations (kLoads loads as well).
  // NS = 8, activations at stage 1 of a chunk (after the weights of stage 5):
  //   stage j   0, 1, 6, 7: weights st+1..st+3 (3); 2..5: those and the
  //             activations (4).  At stage 0 this chunk's activations,
  //             issued before the weights of stage 0 itself, have landed.
  //   last chunk (no activations; stages 4..7 issue nothing): 3 for 0..4,
  //             then 2, 1, 0.
  // NS = 4, activations at stage 0 of a chunk (after the weights of stage 4):
  //   stage j   0: weights st+1..st+3 (3; the activations issued after stage
  //             0's weights are this chunk's own, so they have landed too);
  //             1..3: those and the activations (4).
  //   last chunk (its stages issue nothing): 3, 2, 1, 0.
  //   With 64-row tiles the activations are 2 kLoads units (two halves), so
  //   stages 1..3 allow 3 + 2.
  // A chunk that is not the last: every stage issues stage st+4, which exists.
  auto chunk = [&](int st, bf16x8 (&cur)[RH][8], bf16x8 (&nxt)[RH][8]) {
    if constexpr (NS == 8) {
      stage(st + 0, cur, nxt, IC<0>{}, Y, Nn, IC<3>{});
      stage(st + 1, cur, nxt, IC<1>{}, Y, Y, IC<3>{});
      stage(st + 2, cur, nxt, IC<2>{}, Y, Nn, IC<4>{});
      stage(st + 3, cur, nxt, IC<3>{}, Y, Nn, IC<4>{});
      stage(st + 4, cur, nxt, IC<4>{}, Y, Nn, IC<4>{});
      stage(st + 5, cur, nxt, IC<5>{}, Y, Nn, IC<4>{});
      stage(st + 6, cur, nxt, IC<6>{}, Y, Nn, IC<3>{});
      stage(st + 7, cur, nxt, IC<7>{}, Y, Nn, IC<3>{});
    } else {
      stage(st + 0, cur, nxt, IC<0>{}, Y, Y, IC<3>{});
      stage(st + 1, cur, nxt, IC<1>{}, Y, Nn, IC<3 + RH>{});
      stage(st + 2, cur, nxt, IC<2>{}, Y, Nn, IC<3 + RH>{});
      stage(st + 3, cur, nxt, IC<3>{}, Y, Nn, IC<3 + RH>{});
    }
  };
  auto last_chunk = [&](int st, bf16x8 (&cur)[RH][8], bf16x8 (&nxt)[RH][8]) {
    if constexpr (NS == 8) {
      stage(st + 0, cur, nxt, IC<0>{}, Y, Nn, IC<3>{});
      stage(st + 1, cur, nxt, IC<1>{}, Y, Nn, IC<3>{});
      stage(st + 2, cur, nxt, IC<2>{}, Y, Nn, IC<3>{});
      stage(st + 3, cur, nxt, IC<3>{}, Y, Nn, IC<3>{});
      stage(st + 4, cur, nxt, IC<4>{}, Nn, Nn, IC<3>{});
      stage(st + 5, cur, nxt, IC<5>{}, Nn, Nn, IC<2>{});
      stage(st + 6, cur, nxt, IC<6>{}, Nn, Nn, IC<1>{});
      stage(st + 7, cur, nxt, IC<7>{}, Nn, Nn, IC<0>{});
    } else {
      stage(st + 0, cur, nxt, IC<0>{}, Nn, Nn, IC<3>{});
      stage(st + 1, cur, nxt, IC<1>{}, Nn, Nn, IC<2>{});
      stage(st + 2, cur, nxt, IC<2>{}, Nn, Nn, IC<1>{});
      stage(st + 3, cur, nxt, IC<3>{}, Nn, Nn, IC<0>{});
    }
  };
  int st = 0;
  for (; st + 2 * NS < nst; st += 2 * NS) {
    chunk(st, af, an);
    chunk(st + NS, an, af);
  }
  if (st + NS < nst) {
    chunk(st, af, an);
    last_chunk(st + NS, an, af);
  } else {
    last_chunk(st, af, an);
  }

  // The four waves' partial sums meet in LDS (all loads have landed and every
  // wave is past its last fragment read once the barrier is crossed).
  __builtin_amdgcn_s_waitcnt(0xc07f);
  barrier_lds();
  float* part = reinterpret_cast<float*>(lds);  // [wave][half][strip][16][64]
  static_assert(4 * RH * NS * 16 * 64 * 4 <= kStages * kStageB, "wave sums fit the stages");
#pragma unroll
  for (int hh = 0; hh < RH; ++hh)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(((w * RH + hh) * NS + j) * 16 + r) * 64 + lane] = acc[hh][j][r];
  __syncthreads();
  auto sum4 = [&](int hh, int j) {
    f32x16 v = f32x16{};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] += part[(((u * RH + hh) * NS + j) * 16 + r) * 64 + lane];
    return v;
  };
  // Output units (half, strips) each wave finishes.  SwiGLU: the gate and up
  // strips of h columns 32i .. 32i+31 (strips i and i + NS/2); otherwise one
  // strip.  RH = 1: SwiGLU i = w (NS = 4: waves 0 and 1 only), otherwise
  // strips 2w and 2w+1 (NS = 8) or strip w (NS = 4).  RH = 2 (NS = 4):
  // SwiGLU i = w & 1 of half w >> 1; otherwise strip w of both halves.
  constexpr int NPW = DUAL ? 1 : (RH == 2 ? 2 : NS / 4);  // output units per wave
  if (RH == 1 && DUAL && w >= NS / 2) return;
  const float* bias = a.bias ? a.bias + (int64_t)e * a.bias_estride : nullptr;
#pragma unroll
  for (int u = 0; u < NPW; ++u) {
    int hh, ja, jb;
    if constexpr (RH == 2) {
      hh = DUAL ? (w >> 1) : u;
      ja = DUAL ? (w & 1) : w;
      jb = DUAL ? ja + NS / 2 : ja;
    } else {
      hh = 0;
      ja = DUAL ? w : NPW * w + u;
      jb = DUAL ? w + NS / 2 : ja;
    }
    const f32x16 s0 = sum4(hh, ja);
    const f32x16 s1 = DUAL ? sum4(hh, jb) : s0;
    const int m = 32 * hh + l32;
    if (m >= rows) continue;
    if constexpr (SPLITTABLE) {
      if (split_slot >= 0) {
        // raw fp32 partial sums, tile-local rows x 256 columns (SwiGLU: gate
        // sums in [0,128), up sums in [128,256)), as the other tiles store them
        float* dst = a.partial + (int64_t)split_slot * a.split_rows * kSplitTileCols + m * kSplitTileCols;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c = 8 * q4 + 4 * h;
          *reinterpret_cast<float4*>(dst + ja * kStrip + c) =
              float4{s0[4 * q4], s0[4 * q4 + 1], s0[4 * q4 + 2], s0[4 * q4 + 3]};
          if constexpr (DUAL)
            *reinterpret_cast<float4*>(dst + jb * kStrip + c) =
                float4{s1[4 * q4], s1[4 * q4 + 1], s1[4 * q4 + 2], s1[4 * q4 + 3]};
        }
        continue;
      }
    }
    const RowCtx rc = row_ctx<EPI>(a, r0 + m);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v0{s0[4 * q4], s0[4 * q4 + 1], s0[4 * q4 + 2], s0[4 * q4 + 3]};
      const f32x4 v1{s1[4 * q4], s1[4 * q4 + 1], s1[4 * q4 + 2], s1[4 * q4 + 3]};
      epilogue4<elem, EPI>(a, rc, n0 + ja * kStrip + 8 * q4 + 4 * h, v0, DUAL ? v1 : v0, bias);
    }
  }
}

template <int NS, int RH>
hipError_t launch_ns(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_stream_kernel<EPI_SWIGLU, NS, RH>), dim3(a.max_work), dim3(256), 0, s, a);
      break;
    case EPI_RELU:
      hipLaunchKernelGGL((gemm_stream_kernel<EPI_RELU, NS, RH>), dim3(a.max_work), dim3(256), 0, s, a);
      break;
    case EPI_DOWN_ATOMIC:
      hipLaunchKernelGGL((gemm_stream_kernel<EPI_DOWN_ATOMIC, NS, RH>), dim3(a.max_work), dim3(256), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((gemm_stream_kernel<EPI_DOWN_SLOT, NS, RH>), dim3(a.max_work), dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_stream(int epi, int strips, int rows, const GemmArgs& a, hipStream_t s) {
  if (strips == 8 && rows == 32) return launch_ns<8, 1>(epi, a, s);
  if (strips == 4 && rows == 32) return launch_ns<4, 1>(epi, a, s);
  if (strips == 4 && rows == 64) return launch_ns<4, 2>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
