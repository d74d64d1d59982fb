// C ABI of the MI355X MoE layer forward (declared in include/moe.h):
// host-side validation, the workspace layout and the launch sequence
//   router -> count/scan/scatter -> gate_up GEMM -> down GEMM (+ finalize).
// Everything is enqueued on the caller's stream; nothing here waits on the
// device or reads device memory, and nothing is allocated.
#include "moe.h"

#include <limits.h>
#include <math.h>

#include <mutex>

#include "moe_common.h"
#include "moe_probes.h"

// Workspace of moe_forward_noalloc: one copy per device, held from the first
// call on that device until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_MAX_BYTES];

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// One grouped GEMM's plan: kernel variant and work-list geometry.
struct GemmPlan {
  int var = VAR_GENERIC;
  int32_t bm = 128, cols = 128, ntn = 0, max_work = 0;
  int32_t xr = 0;  // tail rows an expert's last tile may add (256-row bf16 tile only)
};

// Compute units the K-split of a GEMM's last round is planned for (the split
// buffers are sized for this many; a part with more CUs plans for this many).
constexpr int32_t kSplitMaxCU = 256;

struct Layout {
  int64_t M = 0;
  int32_t nchunks = 0;
  GemmPlan g1, g2;
  bool split1 = false, split2 = false;  // gate_up / down may cut their last round along K
  size_t split_tiles1 = 0, split_info1 = 0, split_tiles2 = 0, split_info2 = 0, partial = 0;
  size_t sel32 = 0, chunk_counts = 0, chunk_base = 0, counts = 0, offsets = 0, work1 = 0, work2 = 0,
         num_work = 0, sorted_tok = 0, sorted_slot = 0, sorted_w = 0, logits = 0, stats_part = 0, h = 0, slots = 0,
         acc = 0, total = 0;
};

int elem_bytes(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_EINVAL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ETYPE;
  if (d->out_dtype != MOE_F32 && d->out_dtype != MOE_BF16) return MOE_ETYPE;
  if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_RELU) return MOE_ENOTSUP;
  if (d->T < 0 || d->D <= 0 || d->F <= 0) return MOE_EINVAL;
  if (d->E < 1 || d->E > MOE_MAX_EXPERTS || d->K < 1 || d->K > d->E) return MOE_EINVAL;
  if (d->D > INT_MAX || d->F > INT_MAX) return MOE_EINVAL;
  if (d->T > (int64_t)INT_MAX / d->K) return MOE_EINVAL;  // row ids are int32
  // work-list sizes stay within int32 (checked at the smallest tile shape)
  const int64_t M = d->T * d->K;
  const int64_t tiles = M / 32 + d->E + 1;
  const int64_t cols = d->F / 128 + d->D / 128 + 2;
  if (tiles * cols > (int64_t)INT_MAX) return MOE_EINVAL;
  return MOE_OK;
}

// Variant for one GEMM: the direct-to-LDS kernel (bf16 or fp32) when K fills
// whole 128-byte stages and byte offsets fit in 32 bits; its row tile follows
// the mean number of rows per expert (decode-sized segments get 32-row tiles).
// `may_split`: the GEMM's last partial round may be cut along K.
GemmPlan plan_gemm(const moe_desc* d, int64_t M, int64_t N, int64_t Kd, int64_t a_rows, int64_t b_expert_elems,
                   bool dual, bool may_split) {
  GemmPlan p;
  // whole 128-byte K stages and 32-bit byte offsets
  const int eb = elem_bytes(d->dtype);
  const bool direct_ok = Kd % (128 / eb) == 0 && a_rows * Kd * eb < (int64_t)UINT32_MAX &&
                         b_expert_elems * eb < (int64_t)UINT32_MAX;
  if (direct_ok) {
    const int64_t mean = M / d->E;
    // The 8-wave ping-pong 256-row tile from 58 rows per expert on, even
    // where most of its rows are empty (the idle waves skip their MFMAs): on
    // the Mixtral-shaped layer at 256-1536 tokens (64-384 rows per expert) it
    // runs the layer 17-35% faster than the 4-wave 128-row tile it replaced,
    // on fp32 ReLU layers with 32-256 rows per expert 1.8-3.3x faster (that
    // tile could not split its partial last round along K).  Below it, the
    // 64-row streaming tile (bf16) wins up to about 55 rows per expert (180-
    // 220 tokens: 0.50-0.52 against 0.65 ms) and loses from about 60 (240
    // tokens: 0.728 against 0.656 ms, once experts pass 64 rows).
    p.var = mean >= 58 ? VAR_BF16_M256 : VAR_BF16_M32;
    // Decode-sized bf16 segments: the weight-streaming kernel, which reads
    // every weight row in 1 KB runs.  Its wide tiles (256 weight rows) have
    // their last partial round split along K, which costs a fix-up launch;
    // its narrow tiles (128 weight rows) never split.  The narrow ones are
    // taken when their estimated makespan, in wide-tile times over rounds of
    // kSplitMaxCU blocks, is no longer (min(E, M) experts with rows, each with
    // ceil(mean / 32) row tiles, at least one, times the column tiles).  On
    // the 64-token Mixtral-shaped layer: gate_up 1792 narrow tiles in 7
    // rounds (5 us faster than split wide tiles); down 256 narrow tiles in
    // one round, 8 us faster than 128 wide ones in two K parts and the
    // fix-up (15 us slower before the items' K walks were rotated).
    if (p.var == VAR_BF16_M32 && d->dtype == MOE_BF16 && Kd % kStreamChunk == 0 && N % 32 == 0) {
      const int64_t act = M < d->E ? M : d->E;
      const int64_t rt = mean > 32 ? (mean + 31) / 32 : 1;
      const int64_t c8 = dual ? 128 : 256;
      const int64_t n8 = act * rt * ((N + c8 - 1) / c8), n4 = act * rt * ((N + c8 / 2 - 1) / (c8 / 2));
      const bool split8 = may_split && Kd / kStreamChunk >= kMaxSplitParts;
      const auto clamp = [](int64_t v) { return (int)(v < INT_MAX / 2 ? v : INT_MAX / 2); };
      const float e8 = est_rounds(clamp(n8), kSplitMaxCU, split8 ? kSplitMaxCU : 0);
      const float e4 = est_rounds(clamp(n4), kSplitMaxCU, 0) / 2;
      p.var = e4 <= e8 ? VAR_BF16_S32N : VAR_BF16_S32;
      // From 28 rows per expert on average, many experts exceed a 32-row
      // tile and would read their weights twice; the 64-row narrow tile
      // reads them once for up to 64 rows (its second half's MFMAs ride on
      // the same weight stages: the product stays a weight stream).  On the
      // Mixtral-shaped layer: 128 tokens 0.731 -> 0.477 ms, 200 tokens
      // 0.896 -> 0.509 ms; at 100 tokens (25 rows per expert, few past 32)
      // the 32-row tile is 2% faster, hence the threshold.
      if (mean >= 28) p.var = VAR_BF16_S64N;
    }
  } else {
    // Generic kernel: 64-row tiles when 128-row ones would not fill two
    // rounds of a 256-CU part (a fixed count, so the workspace size does not
    // depend on the device).
    const int64_t bound128 = ((M + 127) / 128 + d->E) * ((N + 127) / 128);
    if (bound128 < 2 * kSplitMaxCU) p.var = VAR_GENERIC_M64;
  }
  p.bm = variant_rows(p.var);
  p.xr = p.var == VAR_BF16_M256 ? kTailRows : 0;
  p.cols = variant_cols(p.var, dual);
  p.ntn = (int32_t)((N + p.cols - 1) / p.cols);
  const int64_t bound = (M + p.bm - 1) / p.bm + d->E;
  const int64_t tiles = M < bound ? M : bound;
  p.max_work = (int32_t)(tiles * p.ntn);
  return p;
}

Layout layout_of(const moe_desc* d) {
  Layout L;
  const int64_t T = d->T, D = d->D, F = d->F, E = d->E, K = d->K;
  const int64_t M = T * K;
  const bool swiglu = d->act == MOE_ACT_SWIGLU;
  const int64_t G = swiglu ? 2 : 1;
  L.M = M;
  L.nchunks = (int32_t)((M + kDispatchChunk - 1) / kDispatchChunk);
  L.g1 = plan_gemm(d, M, F, D, T, G * F * D, swiglu, true);
  L.g2 = plan_gemm(d, M, D, F, M, D * F, false, d->deterministic != 0);
  // With 256- or 32-row tiles, a GEMM's items past its last full round of CUs
  // are cut along K (fp32 partial tiles, reduced in part order by a fix-up
  // kernel that then applies the epilogue) so they fill one round of shorter
  // blocks (decode: 8 experts x 16 down column tiles is half a round).  The
  // down projection splits only in deterministic mode (the atomic combine
  // would add more than two terms per output).
  // A split needs enough K steps to give every part some (8 parts at most):
  // with fewer, the fix-up launch costs more than the shorter round saves
  // (the tiny fp32 block has 2 K steps per GEMM).
  const int eb = elem_bytes(d->dtype);
  auto splits = [&](int var, int64_t Kd) {
    if (var == VAR_BF16_S32N || var == VAR_BF16_S64N) return false;
    if (var == VAR_BF16_S32) return Kd / kStreamChunk >= kMaxSplitParts;  // K steps of 512
    return (var == VAR_BF16_M256 || var == VAR_BF16_M32) && Kd * eb / 128 >= kMaxSplitParts;
  };
  L.split1 = splits(L.g1.var, D);
  L.split2 = d->deterministic && splits(L.g2.var, F);
  if (L.split1) L.g1.max_work += kSplitMaxCU;
  if (L.split2) L.g2.max_work += kSplitMaxCU;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.sel32 = take(sizeof(int32_t) * M);
  L.chunk_counts = take(sizeof(int32_t) * (size_t)L.nchunks * E);
  L.chunk_base = take(sizeof(int32_t) * (size_t)L.nchunks * E);
  L.counts = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 1));
  L.work1 = take(sizeof(int2) * (size_t)L.g1.max_work);
  L.work2 = take(sizeof(int2) * (size_t)L.g2.max_work);
  L.num_work = take(sizeof(int32_t) * 2);
  L.sorted_tok = take(sizeof(int32_t) * M);
  L.sorted_slot = take(sizeof(int32_t) * M);
  L.sorted_w = take(sizeof(float) * M);
  L.logits = take(sizeof(float) * T * E);
  L.stats_part = take(sizeof(float) * (size_t)router_blocks(T) * 3 * E);
  L.h = take((size_t)elem_bytes(d->dtype) * M * F);
  if (d->deterministic) L.slots = take(sizeof(float) * M * D);
  if (L.split1) {
    L.split_tiles1 = take(sizeof(int2) * kSplitMaxCU);
    L.split_info1 = take(sizeof(int32_t) * 2);
  }
  if (L.split2) {
    L.split_tiles2 = take(sizeof(int2) * kSplitMaxCU);
    L.split_info2 = take(sizeof(int32_t) * 2);
  }
  if (L.split1 || L.split2) {  // shared: the two GEMMs and their fix-ups run in order
    const int32_t rows1 = L.split1 ? L.g1.bm + L.g1.xr : 0, rows2 = L.split2 ? L.g2.bm + L.g2.xr : 0;
    L.partial = take(sizeof(float) * (size_t)kSplitMaxCU * (rows1 > rows2 ? rows1 : rows2) * kSplitTileCols);
  }
  if (!d->deterministic && d->out_dtype == MOE_BF16) L.acc = take(sizeof(float) * T * D);
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (0 if it cannot be read: no K-split).
int32_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n < kSplitMaxCU ? n : kSplitMaxCU;
}

// Routing options resolved on the host.
struct RoutePlan {
  const int64_t* replay = nullptr;
  const uint8_t* replay_mask = nullptr;
  float threshold = 0.f;
  bool capacity = false;  // drops for capacity are possible
  int64_t seq_len = 0;
  int32_t slots = 0;
  uint8_t* kept = nullptr;
  float* stats = nullptr;
  bool drops() const { return threshold > 0.f || capacity; }
};

moe_status plan_routing(const moe_desc* d, const moe_routing* r, RoutePlan* out) {
  RoutePlan p;
  if (r) {
    if (!(r->dynamic_threshold >= 0.f) || !(r->capacity_factor >= 0.0) || r->seq_len < 0) return MOE_EINVAL;
    if (r->dynamic_threshold > 0.f && !d->norm_topk) return MOE_EINVAL;
    p.replay = r->replay_experts;
    p.replay_mask = r->replay_experts ? r->replay_mask : nullptr;
    p.threshold = r->dynamic_threshold;
    p.kept = r->kept;
    p.stats = r->stats;
    if (r->capacity_factor > 0.0) {
      const int64_t L = r->seq_len ? r->seq_len : d->T;
      if (L > 0 && d->T % L != 0) return MOE_EINVAL;
      if (L > 0) {
        // the Dew page, section "Expert computation and placement":
        // max(ceil(L*K/E) * cf, cf) slots, rounded down to whole slots
        const double base = (double)((L * d->K + d->E - 1) / d->E);
        double c = base * r->capacity_factor;
        if (c < r->capacity_factor) c = r->capacity_factor;
        c = floor(c);
        // a sequence holds L*K assignments: more slots than that drop nothing
        if (c < (double)(L * d->K)) {
          p.capacity = true;
          p.seq_len = L;
          p.slots = (int32_t)c;
        }
      }
    }
  }
  *out = p;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Records events[i] on s when the caller asked for it.
struct Marks {
  void* const* ev;
  int32_t n;
  hipStream_t s;
  bool mark(int i) const {
    if (!ev || i >= n || !ev[i]) return true;
    return hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) == hipSuccess;
  }
};

moe_status route_and_sort(const moe_desc* d, const RoutePlan& rp, const Layout& L, const void* x, const void* router,
                          const float* router_bias, int64_t* sel, float* weights, float* logits,
                          int32_t* counts_out, int32_t* offsets_out, int32_t* sorted_tok, int32_t* sorted_slot,
                          float* zero_rows, void* ws, hipStream_t s, const Marks& mk, bool build_work) {
  const int eb = elem_bytes(d->dtype);
  RouterArgs ra{};
  ra.x = x;
  ra.router = router;
  ra.router_bias = router_bias;
  ra.T = d->T;
  ra.D = d->D;
  ra.E = d->E;
  ra.K = d->K;
  ra.norm = d->norm_topk ? 1 : 0;
  ra.logits = logits ? logits : at<float>(ws, L.logits);
  ra.sel64 = sel;
  ra.sel32 = at<int32_t>(ws, L.sel32);
  ra.weights = weights;
  ra.zero_rows = zero_rows;
  ra.zero_cols = d->D;
  ra.vec_ok = aligned16(x) && aligned16(router) && ((d->D * eb) % 16 == 0);
  ra.replay = rp.replay;
  ra.replay_mask = rp.replay_mask;
  ra.threshold = rp.threshold;
  ra.kept = rp.kept;
  ra.stats_part = rp.stats ? at<float>(ws, L.stats_part) : nullptr;
  if (launch_router(d->dtype, ra, s) != hipSuccess) return MOE_EDEVICE;
  if (rp.stats) {
    StatsArgs sa{};
    sa.part = ra.stats_part;
    sa.blocks = router_blocks(d->T);
    sa.T = d->T;
    sa.E = d->E;
    sa.stats = rp.stats;
    if (launch_stats(sa, s) != hipSuccess) return MOE_EDEVICE;
  }
  if (!mk.mark(1)) return MOE_EDEVICE;

  DispatchArgs da{};
  da.sel32 = ra.sel32;
  da.weights = weights;
  da.M = L.M;
  da.E = d->E;
  da.K = d->K;
  da.nchunks = L.nchunks;
  da.chunk_counts = at<int32_t>(ws, L.chunk_counts);
  da.chunk_base = at<int32_t>(ws, L.chunk_base);
  da.counts = at<int32_t>(ws, L.counts);
  da.offsets = at<int32_t>(ws, L.offsets);
  da.counts_out = counts_out;
  da.offsets_out = offsets_out;
  da.sorted_tok = sorted_tok ? sorted_tok : at<int32_t>(ws, L.sorted_tok);
  da.sorted_slot = sorted_slot ? sorted_slot : at<int32_t>(ws, L.sorted_slot);
  da.sorted_w = at<float>(ws, L.sorted_w);
  da.nspec = build_work ? 2 : 0;
  const GemmPlan* plans[2] = {&L.g1, &L.g2};
  const size_t works[2] = {L.work1, L.work2};
  for (int i = 0; i < 2; ++i) {
    da.spec[i].bm = plans[i]->bm;
    da.spec[i].xr = plans[i]->xr;
    da.spec[i].windows = plans[i]->var == VAR_BF16_M256;
    da.spec[i].ncu = plans[i]->xr > 0 ? device_cus() : 0;
    da.spec[i].ntn = plans[i]->ntn;
    da.spec[i].max_work = plans[i]->max_work;
    da.spec[i].work = at<int2>(ws, works[i]);
    da.spec[i].num_work = at<int32_t>(ws, L.num_work) + i;
  }
  if (build_work && (L.split1 || L.split2)) {
    const int32_t ncu = device_cus();
    if (L.split1) {
      da.spec[0].split_ncu = ncu;
      da.spec[0].split_tiles = at<int2>(ws, L.split_tiles1);
      da.spec[0].split_info = at<int32_t>(ws, L.split_info1);
    }
    if (L.split2) {
      da.spec[1].split_ncu = ncu;
      da.spec[1].split_tiles = at<int2>(ws, L.split_tiles2);
      da.spec[1].split_info = at<int32_t>(ws, L.split_info2);
    }
  }
  if (rp.capacity) {
    // Sort the (threshold-kept) assignments once, drop the slots past each
    // sequence's capacity, then sort the survivors for the GEMMs.
    DispatchArgs first = da;
    first.counts_out = nullptr;
    first.offsets_out = nullptr;
    first.nspec = 0;
    if (launch_dispatch(first, s) != hipSuccess) return MOE_EDEVICE;
    CapacityArgs ca{};
    ca.offsets = da.offsets;
    ca.sorted_tok = da.sorted_tok;
    ca.sorted_slot = da.sorted_slot;
    ca.sel32 = ra.sel32;
    ca.kept = rp.kept;
    ca.M = L.M;
    ca.seq_len = rp.seq_len;
    ca.E = d->E;
    ca.slots = rp.slots;
    if (launch_capacity(ca, s) != hipSuccess) return MOE_EDEVICE;
  }
  if (launch_dispatch(da, s) != hipSuccess || !mk.mark(2)) return MOE_EDEVICE;
  return MOE_OK;
}

moe_status forward_impl(const moe_desc* d, const moe_routing* r, const void* x, const void* router, const void* gate_up_proj,
                        const void* down_proj, const float* router_bias, const float* up_bias,
                        const float* down_bias, void* out, int64_t* selected_experts, float* routing_weights,
                        float* router_logits, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events, int32_t n_events) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !router || !gate_up_proj || !down_proj || !out || !selected_experts || !routing_weights || !workspace)
    return MOE_EINVAL;
  // the GEMMs' direct-to-LDS loads move 16-byte chunks
  if (!aligned16(x) || !aligned16(gate_up_proj) || !aligned16(down_proj) || !aligned16(workspace)) return MOE_EINVAL;
  RoutePlan rp;
  st = plan_routing(d, r, &rp);
  if (st != MOE_OK) return st;
  const Layout L = layout_of(d);
  if (workspace_bytes < L.total) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks mk{events, n_events, s};
  const int eb = elem_bytes(d->dtype);
  const bool swiglu = d->act == MOE_ACT_SWIGLU;
  const int64_t G = swiglu ? 2 : 1;

  // The fp32 buffer the down projection adds into (atomic mode).
  float* acc = nullptr;
  if (!d->deterministic) acc = d->out_dtype == MOE_F32 ? static_cast<float*>(out) : at<float>(workspace, L.acc);

  if (!mk.mark(0)) return MOE_EDEVICE;
  st = route_and_sort(d, rp, L, x, router, router_bias, selected_experts, routing_weights, router_logits,
                      expert_counts, nullptr, nullptr, nullptr, acc, workspace, s, mk, true);
  if (st != MOE_OK) return st;

  GemmArgs g{};
  g.A = x;
  g.lda = d->D;
  g.a_index = at<int32_t>(workspace, L.sorted_tok);
  g.B = gate_up_proj;
  g.ldb = d->D;
  g.b_estride = G * d->F * d->D;
  g.up_off = d->F;
  g.N = d->F;
  g.Kd = d->D;
  g.work = at<int2>(workspace, L.work1);
  g.num_work = at<int32_t>(workspace, L.num_work);
  g.max_work = L.g1.max_work;
  g.offsets = at<int32_t>(workspace, L.offsets);
  g.bias = up_bias;
  g.bias_estride = G * d->F;
  g.C = at<void>(workspace, L.h);
  g.ldc = d->F;
  g.sorted_tok = at<int32_t>(workspace, L.sorted_tok);
  g.sorted_slot = at<int32_t>(workspace, L.sorted_slot);
  g.sorted_w = at<float>(workspace, L.sorted_w);
  g.vec_ok = aligned16(x) && aligned16(gate_up_proj) && ((d->D * eb) % 16 == 0);
  const int32_t ncu = (L.split1 || L.split2) ? device_cus() : 0;
  if (L.split1) {
    g.split_tiles = at<int2>(workspace, L.split_tiles1);
    g.split_info = at<int32_t>(workspace, L.split_info1);
    g.partial = at<float>(workspace, L.partial);
    g.split_bm = L.g1.bm;
    g.split_rows = L.g1.bm + L.g1.xr;
  }
  const int epi1 = swiglu ? EPI_SWIGLU : EPI_RELU;
  if (launch_grouped_gemm(d->dtype, epi1, L.g1.var, g, s) != hipSuccess) return MOE_EDEVICE;
  if (L.split1 && ncu > 0 && launch_split_fixup(d->dtype, epi1, g, ncu, s) != hipSuccess) return MOE_EDEVICE;
  if (!mk.mark(3)) return MOE_EDEVICE;

  GemmArgs h = g;
  h.A = at<void>(workspace, L.h);
  h.lda = d->F;
  h.a_index = nullptr;
  h.B = down_proj;
  h.ldb = d->F;
  h.b_estride = d->D * d->F;
  h.up_off = 0;
  h.N = d->D;
  h.Kd = d->F;
  h.bias = down_bias;
  h.bias_estride = d->D;
  h.C = d->deterministic ? at<void>(workspace, L.slots) : static_cast<void*>(acc);
  h.ldc = d->D;
  h.work = at<int2>(workspace, L.work2);
  h.num_work = at<int32_t>(workspace, L.num_work) + 1;
  h.max_work = L.g2.max_work;
  h.vec_ok = aligned16(down_proj) && ((d->F * eb) % 16 == 0);
  h.split_tiles = nullptr;
  h.split_info = nullptr;
  h.partial = nullptr;
  if (L.split2) {
    h.split_tiles = at<int2>(workspace, L.split_tiles2);
    h.split_info = at<int32_t>(workspace, L.split_info2);
    h.partial = at<float>(workspace, L.partial);
    h.split_bm = L.g2.bm;
    h.split_rows = L.g2.bm + L.g2.xr;
  }
  if (launch_grouped_gemm(d->dtype, d->deterministic ? EPI_DOWN_SLOT : EPI_DOWN_ATOMIC, L.g2.var, h, s) !=
      hipSuccess)
    return MOE_EDEVICE;
  if (L.split2 && ncu > 0 && launch_split_fixup(d->dtype, EPI_DOWN_SLOT, h, ncu, s) != hipSuccess) return MOE_EDEVICE;
  if (!mk.mark(4)) return MOE_EDEVICE;

  if (d->deterministic || d->out_dtype == MOE_BF16) {
    FinalizeArgs f{};
    f.src = d->deterministic ? at<float>(workspace, L.slots) : acc;
    f.out = out;
    f.T = d->T;
    f.D = d->D;
    f.K = d->deterministic ? d->K : 1;
    f.out_bf16 = d->out_dtype == MOE_BF16;
    if (d->deterministic && rp.drops()) {  // dropped slots have no row: skip them
      f.slot_expert = at<int32_t>(workspace, L.sel32);
      f.E = d->E;
    }
    if (launch_finalize(f, s) != hipSuccess) return MOE_EDEVICE;
  }
  if (!mk.mark(5)) return MOE_EDEVICE;
  return MOE_OK;
}

moe_status dispatch_impl(const moe_desc* d, const moe_routing* r, const void* x, const void* router,
                         const float* router_bias, int64_t* selected_experts, float* routing_weights,
                         float* router_logits, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* sorted_token, int32_t* sorted_slot, void* workspace, size_t workspace_bytes,
                         void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !router || !selected_experts || !routing_weights || !expert_counts || !expert_offsets ||
      !sorted_token || !sorted_slot || !workspace)
    return MOE_EINVAL;
  RoutePlan rp;
  st = plan_routing(d, r, &rp);
  if (st != MOE_OK) return st;
  const Layout L = layout_of(d);
  if (workspace_bytes < L.total) return MOE_EWORKSPACE;
  const Marks none{nullptr, 0, nullptr};
  return route_and_sort(d, rp, L, x, router, router_bias, selected_experts, routing_weights, router_logits,
                        expert_counts, expert_offsets, sorted_token, sorted_slot, nullptr, workspace,
                        static_cast<hipStream_t>(stream), none, false);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
constexpr int kMaxDevices = 64;
void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (size out of range or NULL required pointer)";
    case MOE_ENOTSUP: return "unsupported activation (SwiGLU and ReLU only)";
    case MOE_ETYPE: return "unsupported dtype (fp32 and bf16 only)";
    case MOE_EWORKSPACE: return "workspace smaller than moe_workspace_bytes";
    case MOE_EDEVICE: return "HIP launch or runtime failure";
  }
  return "unknown status";
}

moe_status moe_workspace_bytes(const moe_desc* d, size_t* bytes) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_EINVAL;
  *bytes = d->T == 0 ? 0 : layout_of(d).total;
  return MOE_OK;
}

moe_status moe_forward(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                       const void* down_proj, const float* router_bias, const float* up_bias,
                       const float* down_bias, void* out, int64_t* selected_experts, float* routing_weights,
                       float* router_logits, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return forward_impl(d, nullptr, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                      selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                      stream, nullptr, 0);
}

moe_status moe_forward_routed(const moe_desc* d, const moe_routing* r, const void* x, const void* router,
                              const void* gate_up_proj, const void* down_proj, const float* router_bias,
                              const float* up_bias, const float* down_bias, void* out, int64_t* selected_experts,
                              float* routing_weights, float* router_logits, int32_t* expert_counts,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(d, r, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                      selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                      stream, nullptr, 0);
}

moe_status moe_forward_noalloc(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                               const void* down_proj, const float* router_bias, const float* up_bias,
                               const float* down_bias, void* out, int64_t* selected_experts,
                               float* routing_weights, float* router_logits, int32_t* expert_counts, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (layout_of(d).total > (size_t)MOE_NOALLOC_MAX_BYTES) return MOE_EWORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MOE_EDEVICE;
  // Every workspace section the layer reads is written earlier in the same
  // call (nothing has to start at zero), so the previous call's contents do
  // no harm.
  return forward_impl(d, nullptr, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                      selected_experts, routing_weights, router_logits, expert_counts, ws,
                      (size_t)MOE_NOALLOC_MAX_BYTES, stream, nullptr, 0);
}

moe_status moe_forward_timed(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                             const void* down_proj, const float* router_bias, const float* up_bias,
                             const float* down_bias, void* out, int64_t* selected_experts,
                             float* routing_weights, float* router_logits, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                             int32_t n_events) {
  return forward_impl(d, nullptr, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out,
                      selected_experts, routing_weights, router_logits, expert_counts, workspace, workspace_bytes,
                      stream, events, n_events);
}

moe_status moe_dispatch(const moe_desc* d, const void* x, const void* router, const float* router_bias,
                        int64_t* selected_experts, float* routing_weights, float* router_logits,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token,
                        int32_t* sorted_slot, void* workspace, size_t workspace_bytes, void* stream) {
  return dispatch_impl(d, nullptr, x, router, router_bias, selected_experts, routing_weights, router_logits,
                       expert_counts, expert_offsets, sorted_token, sorted_slot, workspace, workspace_bytes, stream);
}

moe_status moe_dispatch_routed(const moe_desc* d, const moe_routing* r, const void* x, const void* router,
                               const float* router_bias, int64_t* selected_experts, float* routing_weights,
                               float* router_logits, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* sorted_token, int32_t* sorted_slot, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return dispatch_impl(d, r, x, router, router_bias, selected_experts, routing_weights, router_logits,
                       expert_counts, expert_offsets, sorted_token, sorted_slot, workspace, workspace_bytes, stream);
}

moe_status moe_gemm_plan(const moe_desc* d, int32_t* plan) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!plan) return MOE_EINVAL;
  const Layout L = layout_of(d);
  const GemmPlan* g[2] = {&L.g1, &L.g2};
  const bool split[2] = {L.split1, L.split2};
  for (int i = 0; i < 2; ++i) {
    int32_t* o = plan + 6 * i;
    o[0] = g[i]->var;
    o[1] = g[i]->bm;
    o[2] = g[i]->cols;
    o[3] = g[i]->ntn;
    o[4] = split[i] ? 1 : 0;
    o[5] = g[i]->max_work;
  }
  return MOE_OK;
}

}  // extern "C"
