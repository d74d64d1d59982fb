// C ABI of the MI355X MoE layer forward (declared in include/moe.h):
// host-side validation, the workspace layout and the launch sequence
//   router -> count/scan/scatter -> gate_up GEMM -> down GEMM (+ finalize).
// Everything is enqueued on the caller's stream; nothing here waits on the
// device or reads device memory, and nothing is allocated.
#include "moe.h"

#include <limits.h>

#include "moe_common.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t M = 0;
  int32_t nchunks = 0, max_tiles = 0;
  size_t sel32 = 0, chunk_counts = 0, chunk_base = 0, counts = 0, offsets = 0, tile_e = 0, tile_r0 = 0,
         num_tiles = 0, sorted_tok = 0, sorted_slot = 0, sorted_w = 0, logits = 0, h = 0, slots = 0, acc = 0,
         total = 0;
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
  return MOE_OK;
}

Layout layout_of(const moe_desc* d) {
  Layout L;
  const int64_t T = d->T, D = d->D, F = d->F, E = d->E, K = d->K;
  const int64_t M = T * K;
  const int64_t G = d->act == MOE_ACT_SWIGLU ? 2 : 1;
  (void)G;
  L.M = M;
  L.nchunks = (int32_t)((M + kDispatchChunk - 1) / kDispatchChunk);
  const int64_t bound = (M + kGemmBM - 1) / kGemmBM + E;
  L.max_tiles = (int32_t)(M < bound ? M : bound);
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
  L.tile_e = take(sizeof(int32_t) * (size_t)L.max_tiles);
  L.tile_r0 = take(sizeof(int32_t) * (size_t)L.max_tiles);
  L.num_tiles = take(sizeof(int32_t));
  L.sorted_tok = take(sizeof(int32_t) * M);
  L.sorted_slot = take(sizeof(int32_t) * M);
  L.sorted_w = take(sizeof(float) * M);
  L.logits = take(sizeof(float) * T * E);
  L.h = take((size_t)elem_bytes(d->dtype) * M * F);
  if (d->deterministic) L.slots = take(sizeof(float) * M * D);
  if (!d->deterministic && d->out_dtype == MOE_BF16) L.acc = take(sizeof(float) * T * D);
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

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

moe_status route_and_sort(const moe_desc* d, const Layout& L, const void* x, const void* router,
                          const float* router_bias, int64_t* sel, float* weights, float* logits,
                          int32_t* counts_out, int32_t* offsets_out, int32_t* sorted_tok, int32_t* sorted_slot,
                          float* zero_rows, void* ws, hipStream_t s, const Marks& mk) {
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
  if (launch_router(d->dtype, ra, s) != hipSuccess || !mk.mark(1)) return MOE_EDEVICE;

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
  da.bm = kGemmBM;
  da.max_tiles = L.max_tiles;
  da.tile_e = at<int32_t>(ws, L.tile_e);
  da.tile_r0 = at<int32_t>(ws, L.tile_r0);
  da.num_tiles = at<int32_t>(ws, L.num_tiles);
  if (launch_dispatch(da, s) != hipSuccess || !mk.mark(2)) return MOE_EDEVICE;
  return MOE_OK;
}

moe_status forward_impl(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                        const void* down_proj, const float* router_bias, const float* up_bias,
                        const float* down_bias, void* out, int64_t* selected_experts, float* routing_weights,
                        float* router_logits, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events, int32_t n_events) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !router || !gate_up_proj || !down_proj || !out || !selected_experts || !routing_weights || !workspace)
    return MOE_EINVAL;
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
  st = route_and_sort(d, L, x, router, router_bias, selected_experts, routing_weights, router_logits, expert_counts,
                      nullptr, nullptr, nullptr, acc, workspace, s, mk);
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
  g.tile_e = at<int32_t>(workspace, L.tile_e);
  g.tile_r0 = at<int32_t>(workspace, L.tile_r0);
  g.num_tiles = at<int32_t>(workspace, L.num_tiles);
  g.offsets = at<int32_t>(workspace, L.offsets);
  g.max_tiles = L.max_tiles;
  g.bias = up_bias;
  g.bias_estride = G * d->F;
  g.C = at<void>(workspace, L.h);
  g.ldc = d->F;
  g.sorted_tok = at<int32_t>(workspace, L.sorted_tok);
  g.sorted_slot = at<int32_t>(workspace, L.sorted_slot);
  g.sorted_w = at<float>(workspace, L.sorted_w);
  g.vec_ok = aligned16(x) && aligned16(gate_up_proj) && ((d->D * eb) % 16 == 0);
  if (launch_grouped_gemm(d->dtype, swiglu ? EPI_SWIGLU : EPI_RELU, g, s) != hipSuccess || !mk.mark(3))
    return MOE_EDEVICE;

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
  h.vec_ok = aligned16(down_proj) && ((d->F * eb) % 16 == 0);
  if (launch_grouped_gemm(d->dtype, d->deterministic ? EPI_DOWN_SLOT : EPI_DOWN_ATOMIC, h, s) != hipSuccess ||
      !mk.mark(4))
    return MOE_EDEVICE;

  if (d->deterministic || d->out_dtype == MOE_BF16) {
    FinalizeArgs f{};
    f.src = d->deterministic ? at<float>(workspace, L.slots) : acc;
    f.out = out;
    f.T = d->T;
    f.D = d->D;
    f.K = d->deterministic ? d->K : 1;
    f.out_bf16 = d->out_dtype == MOE_BF16;
    if (launch_finalize(f, s) != hipSuccess) return MOE_EDEVICE;
  }
  if (!mk.mark(5)) return MOE_EDEVICE;
  return MOE_OK;
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
  return forward_impl(d, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out, selected_experts,
                      routing_weights, router_logits, expert_counts, workspace, workspace_bytes, stream, nullptr, 0);
}

moe_status moe_forward_timed(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                             const void* down_proj, const float* router_bias, const float* up_bias,
                             const float* down_bias, void* out, int64_t* selected_experts,
                             float* routing_weights, float* router_logits, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                             int32_t n_events) {
  return forward_impl(d, x, router, gate_up_proj, down_proj, router_bias, up_bias, down_bias, out, selected_experts,
                      routing_weights, router_logits, expert_counts, workspace, workspace_bytes, stream, events,
                      n_events);
}

moe_status moe_dispatch(const moe_desc* d, const void* x, const void* router, const float* router_bias,
                        int64_t* selected_experts, float* routing_weights, float* router_logits,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token,
                        int32_t* sorted_slot, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !router || !selected_experts || !routing_weights || !expert_counts || !expert_offsets ||
      !sorted_token || !sorted_slot || !workspace)
    return MOE_EINVAL;
  const Layout L = layout_of(d);
  if (workspace_bytes < L.total) return MOE_EWORKSPACE;
  const Marks none{nullptr, 0, nullptr};
  return route_and_sort(d, L, x, router, router_bias, selected_experts, routing_weights, router_logits,
                        expert_counts, expert_offsets, sorted_token, sorted_slot, nullptr, workspace,
                        static_cast<hipStream_t>(stream), none);
}

}  // extern "C"
