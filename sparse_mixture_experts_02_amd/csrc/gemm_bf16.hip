// Grouped expert GEMM for gfx950 with direct-to-LDS operand loads, bf16 or
// fp32: the prefill- and decode-sized variants of the gate_up and down
// projections (epilogues in gemm_epilogue.h; arithmetic as in
// grouped_gemm.hip: fp32 accumulation, one rounding of h to the compute
// dtype).
//
// Tile: BM sorted rows x 256 weight rows (SwiGLU: 128 gate + the 128 matching
// up rows, so 128 h columns; otherwise 256 output columns).  MFMA
// v_mfma_f32_32x32x16_bf16 (the bf16 256-row tile: v_mfma_f32_16x16x32_bf16;
// fp32: four v_mfma_f32_32x32x2f32 per 16-byte fragment) with the weights as
// operand 0, so a lane's accumulators are groups of four consecutive output
// columns of one row.
// The 256-row tile runs 8 waves (two per SIMD) as a 4 x 2 grid of 64 x 128
// wave tiles and can take an expert's tail of up to kTailRows more rows; the
// decode tile (BM 32) runs 4 waves side by side along the weight rows.  (A
// 4-wave 128-row tile for 64-511 rows per expert measured 17-35% slower than
// the 256-row tile on bf16 layers and up to 3.3x slower on fp32 ones, whose
// partial last round it could not split along K; removed.)
//
// Data path: global_load_lds_dwordx4 writes each 16-byte chunk straight from
// HBM/L2 into LDS (no staging registers).  LDS holds S stages of KB bytes of
// K per row; rows are KB bytes with the 16-byte chunk index XOR-ed with
// bits 1.. of the row index.  gfx950 LDS serves 256 bytes per clock; a
// 32x32 fragment read (32 rows, two chunks) is conflict-free under this
// swizzle, while XOR-ing with the low row bits halves its throughput
// (measured with a probe of the two patterns).  A lane of a load instruction
// writes LDS byte 16*lane of a block of 1024/KB rows, so it loads the global
// chunk the swizzle puts there.
// The 8-wave prefill tile runs a ping-pong schedule (two wave groups take
// turns between matrix-core work and LDS/global traffic, four barriers per
// stage, loads issued a stage ahead); the other shapes issue the loads of a
// stage S-1 steps before it is consumed with one barrier per step, waited on
// only for the loads of the stage being published.
//
// Requires K to fill whole 128-byte stages (K % 64 == 0 for bf16, K % 32 == 0
// for fp32), 16-byte aligned operands, and operand regions under 4 GiB
// (32-bit byte offsets); the host routes anything else to the generic kernel.
#include <type_traits>

#include "gemm_epilogue.h"
#include "moe_common.h"

namespace moe {
namespace {

// One 16-byte chunk from global memory straight into LDS: lane l of the wave
// writes LDS bytes [dst + 16*l, dst + 16*l + 16); dst must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// One pair of 16-byte fragments into a 32x32 fp32 accumulator.  bf16: one
// v_mfma_f32_32x32x16_bf16 (8 k per lane).  fp32: four v_mfma_f32_32x32x2f32
// on the fragments' elements: lanes 0-31 and 32-63 hold 4 consecutive k of
// two chunks, and MFMA i sums element i of both, so every k of the two chunks
// enters once, in the same pairing for both operands.
template <typename T>
__device__ __forceinline__ f32x16 mfma_frag(const bf16x8& b, const bf16x8& a, f32x16 c) {
  if constexpr (T::kBytes == 2) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
  } else {
    const f32x4 bv = __builtin_bit_cast(f32x4, b), av = __builtin_bit_cast(f32x4, a);
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[i], av[i], c, 0, 0, 0);
    return c;
  }
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left unconstrained (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Workgroup barrier for LDS.  The stage data arrives by LDS DMA, whose
// completion each wave has awaited with wait_vm; __syncthreads would also
// drain the loads still in flight for later stages.  The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// Waves per block for a row-tile size.  Prefill tiles run 8 waves (two per
// SIMD): while one wave waits on a barrier, an LDS read or a load issue, the
// other keeps the matrix core busy.  The decode tile runs 4.
// Kernel shape: BM rows per tile, NW waves (M of them along the rows), KB
// bytes of K per LDS stage, S stages.
template <int BM_, int NW_, int M_, int KB_, int S_>
struct Shape {
  static constexpr int BM = BM_, NW = NW_, M = M_, KB = KB_, S = S_;
};
// Chosen by a sweep on the Mixtral-shaped layer (MI355X): for the prefill
// tiles two 64 KB stages with 8 waves beat deeper pipelines of 32 KB stages
// (which need twice the barriers); the decode tile is a weight stream and
// wants more bytes in flight.
using ShapeM256 = Shape<256, 8, 4, 128, 2>;  // 2 x 68 KB of LDS (with the tail rows)
using ShapeM32 = Shape<32, 4, 1, 128, 4>;    // 4 x 36 KB

// SHORT_K: the instance of the bf16 256-row tile for short contractions (at
// most 32 K steps), where a tile's start and end weigh most: the down
// epilogue's row contexts (slot or token, routing weight) are loaded before
// the K loop, and the SwiGLU tile keeps only the stage-end barriers.
template <typename T, int EPI, class SH, bool SHORT_K = false>
__global__ __launch_bounds__(SH::NW * 64) void gemm_bf16_kernel(GemmArgs a) {
  using elem = typename T::elem;
  constexpr int EB = T::kBytes;
  constexpr int BM = SH::BM;
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int NW = SH::NW;
  constexpr int WAVES_M = SH::M;
  constexpr int KB = SH::KB, S = SH::S;
  constexpr int CPR = KB / 16;      // 16-byte chunks per LDS row
  constexpr int RPI = 1024 / KB;    // rows per load instruction
  constexpr int NT = KB / 32;       // 16-k MFMA slices per stage
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int WM = BM / WAVES_M, SM = WM / 32;  // 32-row MFMA tiles per wave
  constexpr int NBR = 256;                      // weight rows per tile
  constexpr int OUTC = DUAL ? 128 : 256;        // output columns per tile
  constexpr int WN = OUTC / WAVES_N, SN = WN / 32;  // 32-column MFMA tiles per wave (per half)
  constexpr int NACC = DUAL ? 2 : 1;
  // The ping-pong tile holds up to XRC rows past BM: an expert's last tile,
  // flagged kTailTile in the work list, takes its tail with it instead of
  // leaving it to a nearly empty tile of its own.  The tail is cut into
  // 32-row strips; strip g is loaded and computed by wave group g (see below).
  constexpr bool PP = S == 2 && NW == 8 && NT == 4 && BM == 256;
  constexpr int XRC = PP ? kTailRows : 0;
  constexpr int AB = (BM + XRC) * KB;           // A bytes per stage
  constexpr int STAGE = AB + NBR * KB;
  constexpr int AI = BM / RPI / NW;             // A load instructions per wave per stage
  constexpr int BI = NBR / RPI / NW;            // B load instructions per wave per stage
  constexpr int NI = AI + BI;
  static_assert(AI >= 1 && BI >= 1 && SM >= 1 && SN >= 1, "tile shape");
  // one or two 32-row strips: wave w loads rows BM + 8w .. (NW * RPI = 64)
  static_assert(XRC == 0 || ((XRC == 32 || XRC == 64) && NW * RPI == 64 && WAVES_M == 4), "tail strips");

  __shared__ __attribute__((aligned(1024))) char lds[S * STAGE];

  if ((int)blockIdx.x >= a.num_work[0]) return;
  // K steps of KB/2 elements; a split item covers steps [kb0, ke0) of its
  // tile and leaves its fp32 partial sums for launch_split_fixup.
  const int nk = (int)(a.Kd / (KB / EB));
  constexpr bool SPLITTABLE = EPI != EPI_DOWN_ATOMIC && (BM == 256 || BM == 32);
  int2 wk = a.work[blockIdx.x];
  int kb0 = 0, ke0 = nk, split_slot = -1;
  if constexpr (SPLITTABLE) {
    if (item_is_split(wk)) {
      const int P = a.split_info[1];
      int j, p;
      split_part(wk, P, &j, &p);
      wk = a.split_tiles[j];
      split_k_range(p, P, nk, &kb0, &ke0);
      split_slot = j * P + p;
    }
  }
  const int e = item_expert(wk);
  const int r0 = item_first_row(wk);
  // A tile flagged kTailTile holds all of its expert's remaining rows (at
  // most BM + XRC by construction of the work lists; clamped all the same).
  const int rows = item_rows(a.offsets[e + 1] - r0, item_is_tail(wk), BM, XRC);
  const int64_t n0 = (int64_t)item_col_tile(wk) * OUTC;
  const int64_t N = a.N;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / WAVES_N, wn = w % WAVES_N;
  const int grp = w >> 2;                          // wave group of the ping-pong tile
  const bool xt = XRC > 0 && rows > BM + 32 * grp;  // this group's tail strip has rows

  // Load assignment: instruction i of wave w fills LDS rows RPI*(w*XI+i) ..;
  // lane l writes physical chunk l%CPR of row r = RPI*(..)+l/CPR, which holds
  // logical chunk (l%CPR) ^ swz(r).
  const int lr = lane / CPR;
  // physical chunk of logical chunk c in row r: c ^ swz(r)
  auto swz = [](int r) { return (r >> 1) & (CPR - 1); };
  uint32_t aoff[AI], boff[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int rA = (w * AI + i) * RPI + lr;
    const int r = r0 + (rA < rows ? rA : 0);
    const int64_t src = a.a_index ? (int64_t)a.a_index[r] : (int64_t)r;
    aoff[i] = (uint32_t)(src * a.lda * EB) + (uint32_t)(((lane % CPR) ^ swz(rA)) * 16);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int rB = (w * BI + i) * RPI + lr;
    int64_t wr;
    if constexpr (DUAL) {
      const int64_t nn = n0 + (rB & (OUTC - 1));
      wr = (nn < N ? nn : N - 1) + (rB >= OUTC ? a.up_off : 0);
    } else {
      const int64_t nn = n0 + rB;
      wr = nn < N ? nn : N - 1;
    }
    boff[i] = (uint32_t)(wr * a.ldb * EB) + (uint32_t)(((lane % CPR) ^ swz(rB)) * 16);
  }
  // Tail rows BM .. BM+XRC-1: wave w loads rows BM + 8w .. BM + 8w + 7, of
  // strip w/4 (a wave whose strip is empty or absent loads nothing).
  uint32_t aoffx = 0;
  if constexpr (XRC > 0) {
    const int rA = BM + w * RPI + lr;
    const int r = r0 + (rA < rows ? rA : 0);
    const int64_t src = a.a_index ? (int64_t)a.a_index[r] : (int64_t)r;
    aoffx = (uint32_t)(src * a.lda * EB) + (uint32_t)(((lane % CPR) ^ swz(rA)) * 16);
  }
  const char* Abase = static_cast<const char*>(a.A);
  const char* Bbase = static_cast<const char*>(a.B) + (int64_t)e * a.b_estride * EB;

  // Loads of stage kt into its buffer.  The stepped schedule of the other
  // shapes issues past the end of the K range: the last stage is then
  // reloaded (into a buffer nobody reads any more), so every step issues the
  // same number of loads and its wait count is one constant.
  // kb0 <= nk - 1 always, so `klast` is a valid step even for an empty range.
  const int klast = ke0 - 1 > kb0 ? ke0 - 1 : kb0;
  // XT_: std::true_type when the tile's tail strips are loaded too (the
  // flag is a compile-time constant so that tiles without tail rows run the
  // plain loop).
  auto issue = [&](int kt, auto XT_) {
    char* dst = lds + (kt % S) * STAGE;
    const uint32_t kb = (uint32_t)min(kt, klast) * (uint32_t)KB;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_dma16(Abase + (aoff[i] + kb), dst + (w * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_dma16(Bbase + (boff[i] + kb), dst + AB + (w * BI + i) * 1024);
    if constexpr (XRC > 0 && decltype(XT_)::value)
      if (xt) lds_dma16(Abase + (aoffx + kb), dst + (BM / RPI + w) * 1024);
  };
  constexpr std::false_type kNoTail{};

  // v_mfma_f32_32x32x16_bf16 with the weights as operand 0: for a 32x32
  // tile, lane l holds output row (token) l%32 and columns 8q + 4(l/32) + r,
  // q, r = 0..3 (accumulator element 4q + r).  Each operand fragment is 16
  // bytes per lane: row l%32, k = 8(l/32)..+8 of a 16-k slice.
  // The bf16 ping-pong tile runs v_mfma_f32_16x16x32_bf16 instead (M16): on
  // this part, with the clock under the power cap, back-to-back 16x16x32
  // MFMAs sustain about a fifth more FLOP/s than 32x32x16 ones (probe: 2.31
  // against 1.90 PFLOP/s at two waves per SIMD), for the same LDS fragment
  // bytes and accumulator registers per wave.  Its 16x16 blocks: lane l
  // holds row l%16 of a block and, as an operand, the 8 k of chunk l/16 of a
  // 32-k half stage; its accumulator holds 4 consecutive output columns
  // 4(l/16).. of row l%16 (the same pairing of k in both operands, and the
  // same fp32 sums as the 32x32 blocks: results are bitwise identical).
  constexpr bool M16 = PP && EB == 2;
  constexpr int FE = M16 ? 16 : 32;            // MFMA block edge
  constexpr int SMb = WM / FE, SNb = WN / FE;  // row blocks per wave, column blocks per half
  using accT = std::conditional_t<M16, f32x4, f32x16>;
  accT acc[NACC][SMb][SNb];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int mi = 0; mi < SMb; ++mi)
#pragma unroll
      for (int ni = 0; ni < SNb; ++ni) acc[q][mi][ni] = accT{};
  // Tail strip g (rows BM + 32g .. +32) of wave group g, with wg = wm - 2g
  // (0 or 1).  32x32 blocks: two per wave, SwiGLU the gate and up blocks of
  // h columns wn*WN + 32*wg ..; otherwise output column blocks 2*wg and
  // 2*wg + 1 of the wave's WN columns.  16x16 blocks: the strip's 16-row
  // block wg times all of the wave's columns.  Both use B fragments the
  // wave already holds.
  constexpr int NX = M16 ? NACC * SNb : 2;
  accT accx[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) accx[i] = accT{};
  const int l16 = lane & 15, h16 = lane >> 4;
  int co16[2];  // 32-k half stage hs is chunks 4hs .. 4hs+3
#pragma unroll
  for (int t = 0; t < 2; ++t) co16[t] = ((4 * t + h16) ^ swz(l16)) * 16;

  const int l32 = lane & 31, h = lane >> 5;
  // Fragment addresses (bytes inside a stage): row*KB + swizzled chunk; the
  // 16-k slice t of the stage is chunk 2t + h.
  const int arow = wm * WM + l32;
  const int brow = wn * WN + l32;
  int co[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) co[t] = ((2 * t + h) ^ swz(l32)) * 16;  // row bases are multiples of 32

  constexpr int NB = NACC * SN;
  auto rdA = [&](const char* buf, int t, int mi) {
    return *reinterpret_cast<const bf16x8*>(buf + (arow + mi * 32) * KB + co[t]);
  };
  auto rdB = [&](const char* buf, int t, int j) {
    return *reinterpret_cast<const bf16x8*>(buf + AB + ((j / SN) * OUTC + brow + (j % SN) * 32) * KB + co[t]);
  };
  // A wave whose rows all lie past the end of the expert's segment (the last
  // row tile of an expert is usually partial) skips its MFMAs and fragment
  // reads; it still loads its share of every stage and meets every barrier.
  const bool busy = wm * WM < rows;
  constexpr bool PFC = SHORT_K && M16 && (EPI == EPI_DOWN_SLOT || EPI == EPI_DOWN_ATOMIC);
  RowCtx pre[PFC ? SMb + 1 : 1];
  if constexpr (PFC) {
#pragma unroll
    for (int mi = 0; mi < SMb; ++mi) pre[mi] = row_ctx<EPI>(a, r0 + min(wm * WM + mi * 16 + l16, rows - 1));
    pre[SMb] = row_ctx<EPI>(a, r0 + min(BM + 32 * grp + 16 * (wm & 1) + l16, rows - 1));
  }
  if constexpr (S == 2 && NW == 8 && NT == 4) {
    // Ping-pong schedule of the 8-wave tile.  Waves 0-3 (group 0) and 4-7
    // (group 1) put one wave of each group on every SIMD.  Time is cut into
    // phases of half a stage (32 k); in every phase one group issues the
    // MFMAs of a half stage (bf16: 32 of 16x16x32) from fragments already in
    // registers while the other group reads the fragments of its next half
    // stage from LDS (and, in its first phase of a stage, issues its loads of
    // the next stage), so the matrix core of a SIMD always has a wave with
    // work and LDS latency is never exposed to it.  Group 1 runs one phase
    // behind group 0.  Every phase ends with a workgroup barrier.
    //   stage k, phase 0: g0 loads k+1, reads half 0  | g1 computes half 1 of k-1
    //            phase 1: g0 computes half 0          | g1 loads k+1, reads half 0
    //            phase 2: g0 reads half 1             | g1 computes half 0
    //            phase 3: g0 computes half 1          | g1 reads half 1; all wait
    //                     for their loads of stage k+1 before the barrier
    // Stage k's buffer is last read in phase 3 of stage k, so the loads of
    // stage k+2 into it (issued in phase 0/1 of stage k+1) follow a barrier.
    bf16x8 fa[2][SM], fb[2][NB];
    constexpr int GB = M16 ? NACC * SNb : 1;  // 16x16: B fragments of a half stage
    bf16x8 ga[M16 ? SMb : 1], gb[GB], gx;
    auto memread = [&](const char* buf, int hs) {
      if (!busy) return;
      if constexpr (M16) {
#pragma unroll
        for (int j = 0; j < GB; ++j)
          gb[j] = *reinterpret_cast<const bf16x8*>(
              buf + AB + ((j / SNb) * OUTC + wn * WN + (j % SNb) * 16 + l16) * KB + co16[hs]);
#pragma unroll
        for (int mi = 0; mi < SMb; ++mi)
          ga[mi] = *reinterpret_cast<const bf16x8*>(buf + (wm * WM + mi * 16 + l16) * KB + co16[hs]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int j = 0; j < NB; ++j) fb[u][j] = rdB(buf, 2 * hs + u, j);
#pragma unroll
          for (int mi = 0; mi < SM; ++mi) fa[u][mi] = rdA(buf, 2 * hs + u, mi);
        }
      }
    };
    bf16x8 fx[2];
    // The MFMAs of a half stage.  With the tail strip (XT), its two blocks
    // follow the first and the last row strip of each slice, so that the
    // dependent MFMAs on one tail accumulator are several MFMAs apart.
    auto mma = [&](auto XT_) {
      if (!busy) return;
      constexpr bool XT = XRC > 0 && decltype(XT_)::value;
      if constexpr (M16) {
        // the tail blocks follow the row blocks, GB / SMb after each
#pragma unroll
        for (int mi = 0; mi < SMb; ++mi) {
#pragma unroll
          for (int j = 0; j < GB; ++j)
            acc[j / SNb][mi][j % SNb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(gb[j], ga[mi], acc[j / SNb][mi][j % SNb], 0, 0, 0);
          if constexpr (XT) {
#pragma unroll
            for (int u = 0; u < GB / SMb; ++u) {
              const int j = mi * (GB / SMb) + u;
              accx[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gb[j], gx, accx[j], 0, 0, 0);
            }
          }
        }
      } else {
        // B fragment indices of the two tail blocks for wg = 0; wg = 1 adds DJ
        constexpr int J0 = 0, J1 = DUAL ? SN : 1, DJ = DUAL ? 1 : 2;
        const bool wg = wm & 1;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mi = 0; mi < SM; ++mi) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[j / SN][mi][j % SN] = mfma_frag<T>(fb[u][j], fa[u][mi], acc[j / SN][mi][j % SN]);
            if constexpr (XT) {
              if (mi == 0) {
                const bf16x8 b0 = wg ? fb[u][J0 + DJ] : fb[u][J0];
                accx[0] = mfma_frag<T>(b0, fx[u], accx[0]);
              }
              if (mi == SM - 1) {
                const bf16x8 b1 = wg ? fb[u][J1 + DJ] : fb[u][J1];
                accx[1] = mfma_frag<T>(b1, fx[u], accx[1]);
              }
            }
          }
      }
    };
    auto memread_x = [&](const char* buf, int hs, auto XT_) {
      if constexpr (XRC > 0 && decltype(XT_)::value) {
        if (!xt) return;
        if constexpr (M16) {
          gx = *reinterpret_cast<const bf16x8*>(buf + (BM + 32 * grp + 16 * (wm & 1) + l16) * KB + co16[hs]);
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            fx[u] = *reinterpret_cast<const bf16x8*>(buf + (BM + 32 * grp + l32) * KB + co[2 * hs + u]);
        }
      }
    };
    // A wave's fragment reads need to have landed before the barrier only at
    // the end of a stage (loads into the buffer they read may follow it);
    // elsewhere the first MFMA that uses them waits, so a reading wave does
    // not hold up the barrier with its LDS latency (prefill gate_up -1%).
    // Only the stage-end barrier orders memory; the three inside a stage
    // keep the groups in step.  The SwiGLU tile keeps them (without them its
    // prefill GEMM is 1% slower, its 32-step 128-expert GEMM 1% faster: the
    // short-contraction instance drops them); the other epilogues drop them
    // (prefill down GEMM -2.5%, the two groups then fall into step by
    // themselves).
    auto phase_end = [&](bool stage_end) {
      if (stage_end) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's fragment reads have landed
        wait_vm<0>();                        // and its loads of the next stage
      }
      if ((DUAL && !SHORT_K) || stage_end) barrier_lds();
    };
    // The two groups run separate straight-line loops (a branch-free body
    // keeps the fragments in registers); both meet the same barriers.  Each
    // loop exists twice: with the tail strips (XT) and without.
    auto run = [&](auto XT) {
      issue(kb0, XT);
      wait_vm<0>();
      barrier_lds();
      if (grp == 0) {
        for (int k = kb0; k < ke0; ++k) {
          const char* buf = lds + (k & 1) * STAGE;
          if (k + 1 < ke0) issue(k + 1, XT);
          memread(buf, 0);
          memread_x(buf, 0, XT);
          phase_end(false);
          mma(XT);
          phase_end(false);
          memread(buf, 1);
          memread_x(buf, 1, XT);
          phase_end(false);
          mma(XT);
          phase_end(true);
        }
      } else {
        for (int k = kb0; k < ke0; ++k) {
          const char* buf = lds + (k & 1) * STAGE;
          if (k > kb0) {
            mma(XT);
          }
          phase_end(false);
          if (k + 1 < ke0) issue(k + 1, XT);
          memread(buf, 0);
          memread_x(buf, 0, XT);
          phase_end(false);
          mma(XT);
          phase_end(false);
          memread(buf, 1);
          memread_x(buf, 1, XT);
          phase_end(true);
        }
        if (ke0 > kb0) {
          mma(XT);
        }
      }
    };
    // xt differs between the wave groups (a group whose strip is empty runs
    // the plain loop); both loops meet the same barriers.
    if (xt)
      run(std::true_type{});
    else
      run(kNoTail);
    wait_vm<0>();  // no LDS DMA may outlive the workgroup
  } else {
    // Other shapes: every wave loads, waits and computes each stage in step.
    // One K step from one LDS stage = NT 16-k slices.  A "group" is the NB
    // MFMAs of one A fragment (NB*32 cycles of matrix core work).  Every LDS
    // read is issued at least one group before its use: the next A fragment
    // one group ahead, the next slice's B fragments spread over the current
    // slice's groups.  Only the first slice's first reads wait on LDS, once
    // per stage.  Scheduling barriers keep this order.
    // Step kt: wait for this wave's loads of stage kt (the S-2 later stages
    // stay in flight), barrier (stage kt visible to all waves; all waves done
    // with stage kt-1), issue stage kt+S-1 into the buffer of stage kt-1,
    // then the MFMAs of stage kt.
    auto compute = [&](const char* buf) {
      bf16x8 fb[2][NB], fa[2];
#pragma unroll
      for (int j = 0; j < NB; ++j) fb[0][j] = rdB(buf, 0, j);
      fa[0] = rdA(buf, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int mi = 0; mi < SM; ++mi) {
          const int g = t * SM + mi;  // group index in the stage
          if (mi + 1 < SM)
            fa[(g + 1) & 1] = rdA(buf, t, mi + 1);
          else if (t + 1 < NT)
            fa[(g + 1) & 1] = rdA(buf, t + 1, 0);
          if (t + 1 < NT) {
#pragma unroll
            for (int j = mi * NB / SM; j < (mi + 1) * NB / SM; ++j) fb[(t + 1) & 1][j] = rdB(buf, t + 1, j);
          }
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[j / SN][mi][j % SN] = mfma_frag<T>(fb[t & 1][j], fa[g & 1], acc[j / SN][mi][j % SN]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(kb0 + p, kNoTail);
    for (int kt = kb0; kt < ke0; ++kt) {
      wait_vm<(S - 2) * NI>();
      barrier_lds();
      issue(kt + S - 1, kNoTail);
      if (busy) compute(lds + (kt % S) * STAGE);
    }
    wait_vm<0>();  // no LDS DMA may outlive the workgroup
  }

  // Output column (tile-local) of tail block i of this wave; SwiGLU's two
  // blocks are the gate and up sums of the same h columns.
  auto xcol = [&](int i) { return wn * WN + 32 * (DUAL ? (wm & 1) : 2 * (wm & 1) + i); };
  const bool xw = xt;  // this wave holds tail-row sums (strip grp)
  if constexpr (SPLITTABLE) {
    if (split_slot >= 0) {
      // raw fp32 partial sums of this K range, tile-local rows x 256 columns
      // (SwiGLU: the gate sums in columns [0,128), the up sums in [128,256))
      float* dst = a.partial + (int64_t)split_slot * a.split_rows * kSplitTileCols;
      if constexpr (M16) {
#pragma unroll
        for (int mi = 0; mi < SMb; ++mi) {
          const int m = wm * WM + mi * 16 + l16;
          if (m >= rows) continue;
#pragma unroll
          for (int j = 0; j < NACC * SNb; ++j) {
            const accT& c0 = acc[j / SNb][mi][j % SNb];
            const int c = (j / SNb) * OUTC + wn * WN + (j % SNb) * 16 + 4 * h16;
            *reinterpret_cast<float4*>(dst + m * kSplitTileCols + c) = float4{c0[0], c0[1], c0[2], c0[3]};
          }
        }
        const int m = BM + 32 * grp + 16 * (wm & 1) + l16;
        if (xw && m < rows) {
#pragma unroll
          for (int j = 0; j < NX; ++j) {
            const accT& c0 = accx[j];
            const int c = (j / SNb) * OUTC + wn * WN + (j % SNb) * 16 + 4 * h16;
            *reinterpret_cast<float4*>(dst + m * kSplitTileCols + c) = float4{c0[0], c0[1], c0[2], c0[3]};
          }
        }
        return;
      } else {
#pragma unroll
        for (int mi = 0; mi < SM; ++mi) {
          const int m = wm * WM + mi * 32 + l32;
          if (m >= rows) continue;
#pragma unroll
          for (int q = 0; q < NACC; ++q)
#pragma unroll
            for (int ni = 0; ni < SN; ++ni)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16& c0 = acc[q][mi][ni];
                const int c = q * OUTC + wn * WN + ni * 32 + 8 * q4 + 4 * h;
                *reinterpret_cast<float4*>(dst + m * kSplitTileCols + c) =
                    float4{c0[4 * q4], c0[4 * q4 + 1], c0[4 * q4 + 2], c0[4 * q4 + 3]};
              }
        }
        if constexpr (XRC > 0) {
          const int m = BM + 32 * grp + l32;
          if (xw && m < rows) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16& c0 = accx[i];
                const int c = (DUAL ? i * OUTC : 0) + xcol(i) + 8 * q4 + 4 * h;
                *reinterpret_cast<float4*>(dst + m * kSplitTileCols + c) =
                    float4{c0[4 * q4], c0[4 * q4 + 1], c0[4 * q4 + 2], c0[4 * q4 + 3]};
              }
          }
        }
        return;
      }
    }
  }

  const float* bias = a.bias ? a.bias + (int64_t)e * a.bias_estride : nullptr;
  if constexpr (M16) {
    // Tiles whose columns all lie inside N, without a bias, over 16-byte
    // aligned rows (the common case) store through one row pointer per row
    // with no per-column checks (the SwiGLU epilogue's bookkeeping otherwise
    // costs more than its transcendentals).
    if constexpr (EPI != EPI_DOWN_ATOMIC) {
      using OT = std::conditional_t<EPI == EPI_DOWN_SLOT, float, elem>;
      if (!bias && n0 + OUTC <= N && (a.ldc & 3) == 0) {
        OT* const C = static_cast<OT*>(a.C) + n0 + wn * WN + 4 * h16;
#pragma unroll
        for (int mi = 0; mi < SMb; ++mi) {
          const int m = wm * WM + mi * 16 + l16;
          if (m >= rows) continue;
          const RowCtx rc = PFC ? pre[mi] : row_ctx<EPI>(a, r0 + m);
          OT* const dst = C + rc.orow * a.ldc;
#pragma unroll
          for (int ni = 0; ni < SNb; ++ni)
            epilogue4_inner<OT, EPI>(dst + ni * 16, rc.wgt, acc[0][mi][ni], acc[NACC - 1][mi][ni]);
        }
        const int m = BM + 32 * grp + 16 * (wm & 1) + l16;
        if (xw && m < rows) {
          const RowCtx rc = PFC ? pre[SMb] : row_ctx<EPI>(a, r0 + m);
          OT* const dst = C + rc.orow * a.ldc;
#pragma unroll
          for (int ni = 0; ni < SNb; ++ni)
            epilogue4_inner<OT, EPI>(dst + ni * 16, rc.wgt, accx[ni], accx[(NACC - 1) * SNb + ni]);
        }
        return;
      }
    }
#pragma unroll
    for (int mi = 0; mi < SMb; ++mi) {
      const int m = wm * WM + mi * 16 + l16;
      if (m >= rows) continue;
      const RowCtx rc = PFC ? pre[mi] : row_ctx<EPI>(a, r0 + m);
#pragma unroll
      for (int ni = 0; ni < SNb; ++ni)
        epilogue4<elem, EPI>(a, rc, n0 + wn * WN + ni * 16 + 4 * h16, acc[0][mi][ni], acc[NACC - 1][mi][ni], bias);
    }
    const int m = BM + 32 * grp + 16 * (wm & 1) + l16;
    if (xw && m < rows) {
      const RowCtx rc = PFC ? pre[SMb] : row_ctx<EPI>(a, r0 + m);
#pragma unroll
      for (int ni = 0; ni < SNb; ++ni)
        epilogue4<elem, EPI>(a, rc, n0 + wn * WN + ni * 16 + 4 * h16, accx[ni], accx[(NACC - 1) * SNb + ni], bias);
    }
    return;
  } else {
#pragma unroll
    for (int mi = 0; mi < SM; ++mi) {
      const int m = wm * WM + mi * 32 + l32;
      if (m >= rows) continue;
      const RowCtx rc = row_ctx<EPI>(a, r0 + m);
#pragma unroll
      for (int ni = 0; ni < SN; ++ni)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& c0 = acc[0][mi][ni];
          const f32x16& c1 = acc[NACC - 1][mi][ni];
          const f32x4 v0{c0[4 * q4], c0[4 * q4 + 1], c0[4 * q4 + 2], c0[4 * q4 + 3]};
          const f32x4 v1{c1[4 * q4], c1[4 * q4 + 1], c1[4 * q4 + 2], c1[4 * q4 + 3]};
          epilogue4<elem, EPI>(a, rc, n0 + wn * WN + ni * 32 + 8 * q4 + 4 * h, v0, v1, bias);
        }
    }
    if constexpr (XRC > 0) {
      const int m = BM + 32 * grp + l32;
      if (xw && m < rows) {
        const RowCtx rc = row_ctx<EPI>(a, r0 + m);
#pragma unroll
        for (int i = 0; i < (DUAL ? 1 : 2); ++i)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x16& c0 = accx[i];
            const f32x16& c1 = accx[DUAL ? 1 : i];
            const f32x4 v0{c0[4 * q4], c0[4 * q4 + 1], c0[4 * q4 + 2], c0[4 * q4 + 3]};
            const f32x4 v1{c1[4 * q4], c1[4 * q4 + 1], c1[4 * q4 + 2], c1[4 * q4 + 3]};
            epilogue4<elem, EPI>(a, rc, n0 + xcol(i) + 8 * q4 + 4 * h, v0, v1, bias);
          }
      }
    }
  }
}

// Reduction of the split tiles: kFixupBlocksPerTile blocks share the rows of
// split tile j; each sums the P partial tiles in part order (reproducible)
// and applies the tile's epilogue to the
// sums, exactly as an unsplit tile applies it to its accumulators (SwiGLU:
// gate and up sums; ReLU; the down projection's weighted slot store).
// 16 blocks of ~18 rows: each thread's chain of dependent loads stays short
// (4 blocks per tile measured 7% slower on the fp32 ReLU layer).
constexpr int kFixupBlocksPerTile = 16;

template <typename T, int EPI>
__global__ __launch_bounds__(256) void split_fixup_kernel(GemmArgs a) {
  const int R = a.split_info[0], P = a.split_info[1];
  const int j = blockIdx.x / kFixupBlocksPerTile;
  const int sub = blockIdx.x - j * kFixupBlocksPerTile;
  if (j >= R) return;
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int OUTC = DUAL ? kSplitTileCols / 2 : kSplitTileCols;
  const int2 wk = a.split_tiles[j];
  const int e = item_expert(wk);
  const int r0 = item_first_row(wk);
  // as the GEMM's tiles
  const int rows = item_rows(a.offsets[e + 1] - r0, item_is_tail(wk), a.split_bm, kTailRows);
  // this block's share of the tile's rows
  const int rs = (rows + kFixupBlocksPerTile - 1) / kFixupBlocksPerTile;
  const int m0 = sub * rs, m1 = min(rows, m0 + rs);
  const int64_t n0 = (int64_t)item_col_tile(wk) * OUTC;
  const float* bias = a.bias ? a.bias + (int64_t)e * a.bias_estride : nullptr;
  constexpr int C4 = OUTC / 4;
  for (int idx = m0 * C4 + (int)threadIdx.x; idx < m1 * C4; idx += 256) {
    const int m = idx / C4, c = (idx - m * C4) * 4;
    // all parts' loads first (one memory round trip, not P); parts past P
    // re-read the last one and are not added
    f32x4 v[kMaxSplitParts], u[kMaxSplitParts];
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
      const int pp = p < P ? p : P - 1;
      const float* src = a.partial + ((int64_t)(j * P + pp) * a.split_rows + m) * kSplitTileCols + c;
      v[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
      if constexpr (DUAL) u[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + OUTC));
    }
    f32x4 s0{0.f, 0.f, 0.f, 0.f}, s1{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
      if (p < P) {
        s0 += v[p];
        if constexpr (DUAL) s1 += u[p];
      }
    }
    const RowCtx rc = row_ctx<EPI>(a, r0 + m);
    epilogue4<typename T::elem, EPI>(a, rc, n0 + c, s0, s1, bias);
  }
}

template <typename T, int EPI>
hipError_t launch_rows(int var, const GemmArgs& a, hipStream_t s) {
  switch (var) {
    case VAR_BF16_M256:
      // short contractions (at most 32 K steps of 64): the down tile loads
      // its epilogue's row contexts up front (128-expert down GEMM, 12 steps:
      // -3.2%; over 224 steps the 14 more registers cost 1.3%), the SwiGLU
      // tile drops its phase barriers
      if constexpr (T::kBytes == 2 && EPI != EPI_RELU) {
        if (a.Kd <= 32 * 64) {
          hipLaunchKernelGGL((gemm_bf16_kernel<T, EPI, ShapeM256, true>), dim3(a.max_work), dim3(ShapeM256::NW * 64), 0, s,
                             a);
          break;
        }
      }
      hipLaunchKernelGGL((gemm_bf16_kernel<T, EPI, ShapeM256>), dim3(a.max_work), dim3(ShapeM256::NW * 64), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_kernel<T, EPI, ShapeM32>), dim3(a.max_work), dim3(ShapeM32::NW * 64), 0, s, a);
      break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fixup_tag(int epi, const GemmArgs& a, int32_t ncu, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((split_fixup_kernel<T, EPI_SWIGLU>), dim3(ncu * kFixupBlocksPerTile), dim3(256), 0, s, a);
      break;
    case EPI_RELU:
      hipLaunchKernelGGL((split_fixup_kernel<T, EPI_RELU>), dim3(ncu * kFixupBlocksPerTile), dim3(256), 0, s, a);
      break;
    case EPI_DOWN_SLOT:
      hipLaunchKernelGGL((split_fixup_kernel<T, EPI_DOWN_SLOT>), dim3(ncu * kFixupBlocksPerTile), dim3(256), 0, s,
                         a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm_tag(int epi, int var, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_SWIGLU: return launch_rows<T, EPI_SWIGLU>(var, a, s);
    case EPI_RELU: return launch_rows<T, EPI_RELU>(var, a, s);
    case EPI_DOWN_ATOMIC: return launch_rows<T, EPI_DOWN_ATOMIC>(var, a, s);
    default: return launch_rows<T, EPI_DOWN_SLOT>(var, a, s);
  }
}

}  // namespace

hipError_t launch_split_fixup(int dtype, int epi, const GemmArgs& a, int32_t ncu, hipStream_t s) {
  if (ncu <= 0) return hipSuccess;
  return dtype == 1 ? launch_fixup_tag<BF16>(epi, a, ncu, s) : launch_fixup_tag<F32>(epi, a, ncu, s);
}

hipError_t launch_gemm_bf16(int dtype, int epi, int var, const GemmArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_gemm_tag<BF16>(epi, var, a, s) : launch_gemm_tag<F32>(epi, var, a, s);
}

}  // namespace moe
