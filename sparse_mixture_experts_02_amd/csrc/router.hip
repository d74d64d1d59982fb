// Router kernel: logits = x . router^T (+ bias), softmax over the experts,
// top-k in descending order with ties to the lower expert index, and the
// routing weights p_sel / (sum p_sel + 1e-9) when renormalising (mojolearn
// "MoEBlock" class description; crackedaicode "Mixture-of-Experts FFN",
// sections "Compute the experts and router" and "Weight the selected
// outputs").
//
// One block of 256 threads (4 waves) owns 16 tokens.
//  * Logits: an MFMA product with the experts as the 16-wide MFMA rows and the
//    16 tokens as its columns.  The four waves split the model width D into
//    four ranges (split-K) and their partial sums meet in LDS, so one block
//    reads its 16 token rows exactly once straight from HBM into registers.
//    bf16 routers over more than 64 experts take their logits instead from
//    router_logits_kernel (64 tokens per block, router rows staged in LDS),
//    launched just before, and this kernel reads them back.
//  * Selection: L lanes per token, each lane holding up to PL experts: up to 64
//    experts, L = E rounded up to a power of two and PL = 1..4 (L <= 64);
//    more than 64 experts, PL = 8 and L = 16 (E <= 128) or 32 (E <= 256), so
//    that one wave pass covers several tokens and each reduction has fewer
//    exchange steps.  Maximum, sum and the K top-k rounds are reductions
//    inside the L-lane group: DPP register moves within 16 lanes, ds_bpermute
//    beyond (see group_reduce).  The
//    top-k key packs (probability bits << 32) | (0xffffffff - expert): since
//    probabilities are >= 0 their bit patterns order like the values, and the
//    larger key on equal probabilities is the lower expert index.
//  * The same block clears the rows of the fp32 combine buffer for its tokens
//    (the down projection adds into them with atomics).
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* row, int64_t k, int64_t n, bool vec) {
  if (vec && k + 8 <= n) {
    uint4 v = *reinterpret_cast<const uint4*>(row + k);
    return __builtin_bit_cast(bf16x8, v);
  }
  union {
    uint16_t h[8];
    uint4 v;
  } t;
#pragma unroll
  for (int j = 0; j < 8; ++j) t.h[j] = (k + j < n) ? row[k + j] : (uint16_t)0;
  return __builtin_bit_cast(bf16x8, t.v);
}

__device__ __forceinline__ float4 load_f32x4(const float* row, int64_t k, int64_t n, bool vec) {
  if (vec && k + 4 <= n) return *reinterpret_cast<const float4*>(row + k);
  float4 v;
  v.x = (k + 0 < n) ? row[k + 0] : 0.f;
  v.y = (k + 1 < n) ? row[k + 1] : 0.f;
  v.z = (k + 2 < n) ? row[k + 2] : 0.f;
  v.w = (k + 3 < n) ? row[k + 3] : 0.f;
  return v;
}

// Reductions over aligned groups of 2^lg lanes, every lane receiving the
// result.  Step i pairs each lane with one of the other half of its 2^(i+1)
// group: xor 1 and xor 2 (DPP quad permutations), the mirror inside 8 lanes
// and the mirror inside 16 lanes (DPP row_half_mirror and row_mirror: lane i
// with 7 - i and 15 - i), then xor 16 and xor 32 through ds_bpermute.  The
// first four are register moves, not LDS round trips.  Both lanes of a pair
// combine the same two values, so with a commutative op every lane of the
// group ends with the same bits.
template <int STEP>
__device__ __forceinline__ int xchg(int v) {
  if constexpr (STEP == 0) return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  else if constexpr (STEP == 1) return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (STEP == 2) return __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false); // row_half_mirror
  else if constexpr (STEP == 3) return __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false); // row_mirror
  else return __shfl_xor(v, 1 << STEP);
}
template <int STEP>
__device__ __forceinline__ float xchg(float v) { return __int_as_float(xchg<STEP>(__float_as_int(v))); }
template <int STEP>
__device__ __forceinline__ uint64_t xchg(uint64_t v) {
  const uint32_t lo = (uint32_t)xchg<STEP>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)xchg<STEP>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, int lg, Op op) {
  if (lg > 0) v = op(v, xchg<0>(v));
  if (lg > 1) v = op(v, xchg<1>(v));
  if (lg > 2) v = op(v, xchg<2>(v));
  if (lg > 3) v = op(v, xchg<3>(v));
  if (lg > 4) v = op(v, xchg<4>(v));
  if (lg > 5) v = op(v, xchg<5>(v));
  return v;
}

// Partial logits of this wave's D range: acc[nt][i] = sum over the range of
// x[t0 + lane%16] . router[nt*16 + 4*(lane/16) + i].
template <typename Tag, int NT>
__device__ __forceinline__ void logits_partial(const RouterArgs& a, int64_t t0, int w, int lane, f32x4 (&acc)[NT]) {
  const int64_t D = a.D;
  const int64_t tok = min(t0 + (lane & 15), a.T - 1);
  const int g = lane >> 4;
  const bool vec = a.vec_ok != 0;
  int64_t erow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) erow[nt] = min(nt * 16 + (lane & 15), a.E - 1);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // U k-steps per iteration: all their loads are issued before the MFMAs so
  // several HBM round trips overlap (16 for one expert tile: the 64-token
  // decode router -2 us against 8).  Elements at or past ke read as zero.
  constexpr int U = NT <= 1 ? 16 : NT <= 2 ? 8 : (NT <= 4 ? 4 : (NT <= 8 ? 2 : 1));
  if constexpr (sizeof(typename Tag::elem) == 2) {
    constexpr int KS = 32;
    const int64_t steps = (D + KS - 1) / KS;
    const int64_t per = (steps + 3) / 4;
    const int64_t kb = w * per * KS, ke = min(D, (w + 1) * per * KS);
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + tok * D;
    const uint16_t* R = static_cast<const uint16_t*>(a.router);
    for (int64_t k = kb; k < ke; k += U * KS) {
      bf16x8 xa[U], rb[U][NT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t kk = k + u * KS + 8 * g;
        xa[u] = load_bf16x8(xr, kk, ke, vec);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) rb[u][nt] = load_bf16x8(R + erow[nt] * D, kk, ke, vec);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[u][nt], xa[u], acc[nt], 0, 0, 0);
    }
  } else {
    constexpr int KS = 16;
    const int64_t steps = (D + KS - 1) / KS;
    const int64_t per = (steps + 3) / 4;
    const int64_t kb = w * per * KS, ke = min(D, (w + 1) * per * KS);
    const float* xr = static_cast<const float*>(a.x) + tok * D;
    const float* R = static_cast<const float*>(a.router);
    for (int64_t k = kb; k < ke; k += U * KS) {
      float4 xa[U], rv[U][NT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t kk = k + u * KS + 4 * g;
        xa[u] = load_f32x4(xr, kk, ke, vec);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) rv[u][nt] = load_f32x4(R + erow[nt] * D, kk, ke, vec);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(rv[u][nt].x, xa[u].x, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(rv[u][nt].y, xa[u].y, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(rv[u][nt].z, xa[u].z, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(rv[u][nt].w, xa[u].w, acc[nt], 0, 0, 0);
        }
    }
  }
}

// Logits of the layers with more than 64 experts (bf16, D a multiple of 256,
// 16-byte aligned rows): logits[t,e] = x[t] . router[e] (+ bias[e]) for 64
// tokens per block, so that the router weights (E x D, 0.5 MB at E = 128,
// D = 2048) are read once per 64 tokens instead of once per 16.  With NW
// waves, wave w owns tokens 16 (w % 4) .. +16 of the block and the experts
// of part w / 4 of the NW / 4 equal parts: MFMA 16x16x32 with the experts as
// rows and the tokens as columns, as in logits_partial.  The router rows go
// HBM/L2 -> LDS by direct loads in chunks of 64 elements (128-byte rows,
// 16-byte chunk index XOR-ed with bits 1..3 of the row), kLogitStages chunks
// in flight; the token rows go straight into registers.  The sum over D runs
// in one order per (t, e), so the result does not depend on the grid.
constexpr int kLogitTokens = 64;
constexpr int kLogitStages = 4;
constexpr int kLogitWaves = 8;  // two waves per SIMD (four waves, or eight chunks in flight, measured the same)

// One 16-byte chunk from global memory straight into LDS: lane l writes LDS
// bytes [dst + 16 l, dst + 16 l + 16); dst must be wave-uniform.  (Kept out
// of the kernel template: the host pass does not accept the builtin there.)
__device__ __forceinline__ void lds_dma16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

template <int NT, int NW>
__global__ __launch_bounds__(NW * 64) void router_logits_kernel(RouterArgs a) {
  constexpr int EP = NT * 16;
  constexpr int CHUNK = EP * 128;          // bytes of one chunk (EP rows x 64 elements)
  constexpr int NI = EP / 8 / NW;          // 1 KB load instructions per wave per chunk
  constexpr int NTW = NT / (NW / 4);       // 16-expert tiles per wave
  constexpr int S = kLogitStages;
  static_assert(NW == 4 || NW == 8, "4 token groups of 16, 1 or 2 expert parts");
  static_assert(NI >= 1 && NI * NW * 8 == EP, "whole 8-row load instructions per wave");
  __shared__ __attribute__((aligned(1024))) char lds[S * CHUNK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t D = a.D;
  const int E = a.E;
  const int ebase = (w / 4) * NTW * 16;    // this wave's first expert row
  const int64_t tbase = (int64_t)blockIdx.x * kLogitTokens + (w % 4) * 16;
  const int64_t tok = min(tbase + (lane & 15), a.T - 1);
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + tok * D;
  const char* R = static_cast<const char*>(a.router);
  const int g = lane >> 4;
  auto swz = [](int r) { return (r >> 1) & 7; };

  // Loads of chunk c (elements 64c ..): instruction i of wave w fills LDS
  // rows 8(w + NW i) .. +8; lane l writes physical 16-byte chunk l%8 of row
  // 8(w + NW i) + l/8, which holds logical chunk (l%8) ^ swz(row).  Rows past
  // E repeat row E - 1; their logits are not written.
  uint32_t roff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (w + NW * i) * 8 + (lane >> 3);
    const int er = r < E ? r : E - 1;
    roff[i] = (uint32_t)((int64_t)er * D * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
  const int nch = (int)(D / 64);
  bf16x8 xa[S][2];
  // chunk c into stage b = c % S (b passed as a constant)
  auto issue = [&](int c, int b) {
    char* dst = lds + b * CHUNK;
    const uint32_t kb = (uint32_t)c * 128u;
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_dma16(R + (roff[i] + kb), dst + (w + NW * i) * 1024);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      xa[b][s] = *reinterpret_cast<const bf16x8*>(xr + (int64_t)c * 64 + s * 32 + 8 * g);
  };
  f32x4 acc[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Every step issues one chunk (past the end: the last one again, into a
  // stage nobody reads), so that S - 2 chunks are always in flight behind
  // the one awaited and the wait count is a constant.
  constexpr int LATER = (S - 2) * (NI + 2);  // loads per chunk: NI + 2
  static_assert(S >= 3 && LATER < 64, "vmcnt is 6 bits");
#pragma unroll
  for (int p = 0; p < S - 1; ++p) issue(min(p, nch - 1), p);
  // Unrolled by S (nch is a multiple of S) so that every register-buffer
  // index is a constant and the loop body has no exit.
  for (int c0 = 0; c0 < nch; c0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int c = c0 + j;
      __builtin_amdgcn_s_waitcnt((LATER & 15) | ((LATER >> 4) << 14) | 0x0f70);
      // Chunk c visible; every wave is done with chunk c - 1.  A plain
      // s_barrier: __syncthreads would also drain the later chunks' loads.
      // The memory clobber keeps LDS accesses on their side of it.
      asm volatile("s_barrier" ::: "memory");
      issue(min(c + S - 1, nch - 1), (j + S - 1) % S);
      const char* buf = lds + j * CHUNK;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int row = ebase + nt * 16 + (lane & 15);
          const bf16x8 rb = *reinterpret_cast<const bf16x8*>(buf + row * 128 + (((s * 4 + g) ^ swz(row)) * 16));
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb, xa[j][s], acc[nt], 0, 0, 0);
        }
    }
  }
  // No LDS write may land after the block ends.
  __builtin_amdgcn_s_waitcnt(0x0f70);
  // lane: token tbase + lane%16, experts ebase + nt*16 + 4*(lane/16) + i
  const int64_t t = tbase + (lane & 15);
  if (t < a.T) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = ebase + nt * 16 + 4 * g + i;
        if (e < E) a.logits[t * E + e] = acc[nt][i] + (a.router_bias ? a.router_bias[e] : 0.f);
      }
  }
}

template <typename Tag, int NT>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a, int pre) {
  constexpr int EP = NT * 16;
  extern __shared__ float part[];  // [4 waves][16 tokens][EP]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTokens;
  const int E = a.E, K = a.K;

  // Clear this block's rows of the combine buffer.
  if (a.zero_rows) {
    const int64_t cols = a.zero_cols;
    const int64_t rows = min((int64_t)kRouterTokens, a.T - t0);
    float* z = a.zero_rows + t0 * cols;
    const int64_t n = rows * cols;
    if ((cols & 3) == 0) {
      for (int64_t i = (int64_t)tid * 4; i < n; i += kThreads * 4)
        *reinterpret_cast<float4*>(z + i) = float4{0.f, 0.f, 0.f, 0.f};
    } else {
      for (int64_t i = tid; i < n; i += kThreads) z[i] = 0.f;
    }
  }

  if (pre) {
    // Logits (with the bias) written by router_logits_kernel: all of a
    // thread's loads issued before the first is awaited.
    constexpr int PER = 16 * EP / kThreads;
    float v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      // in-bounds address for every lane (no branch around the load)
      const int idx = tid + q * kThreads, tk = idx / EP, e = idx % EP;
      const bool ok = e < E && t0 + tk < a.T;
      const float lv = a.logits[min(t0 + tk, a.T - 1) * E + min(e, E - 1)];
      v[q] = ok ? lv : 0.f;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) part[tid + q * kThreads] = v[q];
    __syncthreads();
  } else {
    f32x4 acc[NT];
    logits_partial<Tag, NT>(a, t0, w, lane, acc);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[(w * 16 + (lane & 15)) * EP + nt * 16 + 4 * (lane >> 4) + i] = acc[nt][i];
    __syncthreads();

    // Sum the four partials; add the bias; publish the logits.
    for (int idx = tid; idx < 16 * EP; idx += kThreads) {
      const int tk = idx / EP, e = idx % EP;
      float v = part[idx] + part[16 * EP + idx] + part[32 * EP + idx] + part[48 * EP + idx];
      if (e < E && a.router_bias) v += a.router_bias[e];
      part[idx] = v;
      if (a.logits && e < E && t0 + tk < a.T) a.logits[(t0 + tk) * E + e] = v;
    }
    __syncthreads();
  }

  // Regions of `part` free after the sum above: p (16 x EP), and the
  // weights and experts of the 16 tokens' K slots (16 x K, K <= EP), read
  // by the per-block statistics.
  float* pbuf = part + 16 * EP;
  float* wbuf = part + 32 * EP;
  int* sbuf = reinterpret_cast<int*>(part + 48 * EP);

  // Softmax and top-k with L lanes per token, PL experts per lane.
  constexpr int PL = NT > 4 ? 8 : 4;
  // L is a power of two: divisions by it are shifts by lgL.
  int L = 1;
  if constexpr (PL == 4) {
    while (L < E && L < 64) L <<= 1;
  } else {
    while (L * PL < E) L <<= 1;
  }
  const int lgL = __builtin_ctz(L);
  const int per_wave = 64 >> lgL;   // tokens one wave pass covers
  const int j = lane & (L - 1);     // lane inside the token's group
  for (int base = 0; base < 4; base += per_wave) {
    const int slot = base + (lane >> lgL);     // 0..3 inside this wave's four tokens
    const int tk = w * 4 + slot;
    const bool active = (slot < 4) && (t0 + tk < a.T);
    const float* lg = part + (active ? tk : w * 4) * EP;

    float lv[PL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = j + i * L;
      lv[i] = (e < E) ? lg[e] : -INFINITY;
      m = fmaxf(m, lv[i]);
    }
    m = group_reduce(m, lgL, [](float u, float v) { return fmaxf(u, v); });
    float ev[PL], s = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = j + i * L;
      ev[i] = (e < E) ? expf(lv[i] - m) : 0.f;
      s += ev[i];
    }
    s = group_reduce(s, lgL, [](float u, float v) { return u + v; });

    float pr[PL];
    uint64_t key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = j + i * L;
      pr[i] = ev[i] / s;
      key[i] = (e < E) ? (((uint64_t)__float_as_uint(pr[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e)) : 0ull;
    }
    const int64_t t = t0 + tk;

    // Routing replay (the Dew "Mixture of experts" page, section "Router
    // behavior"): a token the record covers takes the recorded experts, with
    // this forward's probabilities.  A record holding an index outside
    // [0, E) does not cover its token.  `covered` is uniform in the group.
    bool covered = false;
    if (a.replay) {
      int bad = 0;
      if (active) {
        for (int k = j; k < K; k += L) {
          const int64_t e = a.replay[t * K + k];
          bad |= (e < 0 || e >= E) ? 1 : 0;
        }
      }
      bad = group_reduce(bad, lgL, [](int u, int v) { return u | v; });
      covered = active && !bad && (!a.replay_mask || a.replay_mask[t] != 0);
    }

    float psum = 0.f;
    int mysel[PL];
    float myp[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      mysel[i] = 0;
      myp[i] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < PL; ++i) best = key[i] > best ? key[i] : best;
      best = group_reduce(best, lgL, [](uint64_t u, uint64_t v) { return u > v ? u : v; });
      int e = (int)(0xffffffffu - (uint32_t)best);
      float p = __uint_as_float((uint32_t)(best >> 32));
      if ((e & (L - 1)) == j) {
#pragma unroll
        for (int i = 0; i < PL; ++i)
          if ((e >> lgL) == i) key[i] = 0ull;
      }
      if (a.replay) {
        // p of the recorded expert: lane (e % L) of the group holds it as pr[e / L]
        const int er = covered ? (int)a.replay[t * K + k] : 0;
        const int q = er >> lgL;
        float mine = pr[0];
#pragma unroll
        for (int i = 1; i < PL; ++i) mine = q == i ? pr[i] : mine;
        const float pe = __shfl(mine, (lane & ~(L - 1)) | (er & (L - 1)));
        if (covered) {
          e = er;
          p = pe;
        }
      }
      psum += p;
      const int kq = k >> lgL, kr = k & (L - 1);
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (kq == i && kr == j) {
          mysel[i] = e;
          myp[i] = p;
        }
    }

    // Weights; the dynamic threshold (the ES-MoE "API" page, settings table
    // of "ESMoE"): a non-leading slot whose renormalised weight is below the
    // threshold is dropped and the kept weights are renormalised.
    const float denom = psum + 1e-9f;
    float wk[PL];
    bool keep[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int k = j + i * L;
      wk[i] = a.norm ? myp[i] / denom : myp[i];
      keep[i] = k < K;
    }
    if (a.threshold > 0.f) {
      float ks = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int k = j + i * L;
        if (k > 0 && wk[i] < a.threshold) keep[i] = false;
        if (keep[i]) ks += wk[i];
      }
      ks = group_reduce(ks, lgL, [](float u, float v) { return u + v; });
#pragma unroll
      for (int i = 0; i < PL; ++i) wk[i] = keep[i] ? wk[i] / ks : 0.f;
    }

    if (active) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int k = j + i * L;
        if (k < K) {
          a.sel64[t * K + k] = mysel[i];
          a.sel32[t * K + k] = keep[i] ? mysel[i] : E;  // E: dropped, takes no row
          a.weights[t * K + k] = wk[i];
          if (a.kept) a.kept[t * K + k] = keep[i] ? 1 : 0;
          if (a.stats_part) {
            wbuf[tk * EP + k] = wk[i];
            sbuf[tk * EP + k] = mysel[i];
          }
        }
      }
      if (a.stats_part) {
#pragma unroll
        for (int i = 0; i < PL; ++i) {
          const int e = j + i * L;
          if (e < E) pbuf[tk * EP + e] = pr[i];
        }
      }
    }
  }

  // Per-block sums for the balancing statistics, in a fixed order: for each
  // expert, the sum over this block's tokens of p, of the gate (the token's
  // weights at that expert) and of [gate > 0].
  if (a.stats_part) {
    __syncthreads();
    const int nt = (int)min((int64_t)kRouterTokens, a.T - t0);
    float* dst = a.stats_part + (int64_t)blockIdx.x * 3 * E;
    for (int e = tid; e < E; e += kThreads) {
      float sp = 0.f, sg = 0.f, sc = 0.f;
      for (int tk = 0; tk < nt; ++tk) {
        sp += pbuf[tk * EP + e];
        float g = 0.f;
        for (int k = 0; k < K; ++k) g += sbuf[tk * EP + k] == e ? wbuf[tk * EP + k] : 0.f;
        sg += g;
        sc += g > 0.f ? 1.f : 0.f;
      }
      dst[e] = sp;
      dst[E + e] = sg;
      dst[2 * E + e] = sc;
    }
  }
}

// Balancing objectives (the ES-MoE "API" page, section "Balancing
// objectives") from the router's per-block sums.  One block: wave w sums the
// columns c = w, w+4, ... over the blocks with a fixed lane split and a fixed
// shuffle tree (reproducible), then one thread forms the four objectives in
// double precision from the E means.
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  __shared__ float mean[3 * kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = a.E, C = 3 * E;
  for (int c = w; c < C; c += kThreads / 64) {
    float v = 0.f;
    for (int64_t b = lane; b < a.blocks; b += 64) v += a.part[b * C + c];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) {
      mean[c] = v / (float)a.T;
      a.stats[c] = mean[c];
    }
  }
  __syncthreads();
  if (tid == 0) {
    double sp = 0.0, sg = 0.0, sw = 0.0;
    for (int e = 0; e < E; ++e) {
      sp += mean[e];
      sg += mean[E + e];
      sw += (double)mean[e] * mean[2 * E + e];
    }
    double gs = 0.0, ms = 0.0, ps = 0.0;
    for (int e = 0; e < E; ++e) {
      const double ug = sg > 0.0 ? mean[E + e] / sg : 0.0;
      const double up = sp > 0.0 ? mean[e] / sp : 0.0;
      gs += ug * ug;
      ms += (ug - 1.0 / E) * (ug - 1.0 / E);
      ps += up * up;
    }
    a.stats[C + 0] = (float)(E * sw);   // switch
    a.stats[C + 1] = (float)(E * gs);   // gshard
    a.stats[C + 2] = (float)(ms / E);   // master
    a.stats[C + 3] = (float)(E * ps);   // gshard_probs
  }
}

// Launches router_logits_kernel when it applies; returns whether it did.
template <int NT>
int launch_logits(const RouterArgs& a, hipStream_t s) {
  // (router offsets are 32-bit byte offsets)
  if (!(a.vec_ok && a.D % (64 * kLogitStages) == 0 && a.logits && (int64_t)a.E * a.D * 2 < (int64_t)UINT32_MAX))
    return 0;
  const unsigned grid = (unsigned)((a.T + kLogitTokens - 1) / kLogitTokens);
  hipLaunchKernelGGL((router_logits_kernel<NT, kLogitWaves>), dim3(grid), dim3(kLogitWaves * 64), 0, s, a);
  return 1;
}

template <typename Tag, int NT>
hipError_t launch_nt(const RouterArgs& a, hipStream_t s) {
  int pre = 0;
  if constexpr (NT >= 8 && Tag::kBytes == 2) pre = launch_logits<NT>(a, s);
  const unsigned grid = (unsigned)((a.T + kRouterTokens - 1) / kRouterTokens);
  const size_t lds = (size_t)4 * 16 * NT * 16 * sizeof(float);
  hipLaunchKernelGGL((router_kernel<Tag, NT>), dim3(grid), dim3(kThreads), lds, s, a, pre);
  return hipGetLastError();
}

template <typename Tag>
hipError_t launch_tag(const RouterArgs& a, hipStream_t s) {
  const int nt = (a.E + 15) / 16;
  if (nt <= 1) return launch_nt<Tag, 1>(a, s);
  if (nt <= 2) return launch_nt<Tag, 2>(a, s);
  if (nt <= 4) return launch_nt<Tag, 4>(a, s);
  if (nt <= 8) return launch_nt<Tag, 8>(a, s);
  return launch_nt<Tag, 16>(a, s);
}

}  // namespace

hipError_t launch_router(int dtype, const RouterArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return dtype == 1 ? launch_tag<BF16>(a, s) : launch_tag<F32>(a, s);
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
