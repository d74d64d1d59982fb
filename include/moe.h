/*
 * moe.h -- C ABI of the MI355X (gfx950) token-choice top-k mixture-of-experts
 * feed-forward layer, forward pass.
 *
 * What the layer computes (per token t of x, D features):
 *   logits[t,e] = x[t] . router[e] (+ router_bias[e])            e < E
 *   p[t]        = softmax over the E logits
 *   sel[t,0..K) = the K largest p[t,e] in descending order, equal values to
 *                 the lower expert index
 *   w[t,k]      = p[t,sel] / (sum_k p[t,sel] + 1e-9) if norm_topk, else p[t,sel]
 *   y_e(x)      = SwiGLU: down_proj[e] (silu(gate) * up), gate = rows [0,F) of
 *                 gate_up_proj[e] times x, up = rows [F,2F);
 *                 ReLU:   W2[e] relu(W1[e] x + b1[e]) + b2[e]
 *   out[t]      = sum_k w[t,k] * y_{sel[t,k]}(x[t])
 * Sources: the mojolearn "MoEBlock" API page (class description, "Variables",
 * "Parameters"), the crackedaicode "Mixture-of-Experts FFN" exercise (sections
 * "Compute the experts and router" and "Weight the selected outputs"), and the
 * Dew "Mixture of experts" page, section "Expert computation and placement"
 * (tokens are sorted into expert order and the experts run as one grouped
 * matrix product; a product's running sums are kept in fp32 or wider and its
 * result is rounded to the working precision a single time).
 *
 * Conventions for every entry point
 *   - Tensors are contiguous, row-major DEVICE pointers unless stated.  Weights
 *     use the Hugging Face layouts: router (E,D), gate_up_proj (E,G*F,D) with
 *     G=2 for SwiGLU (W1 (E,F,D) with G=1 for ReLU), down_proj (E,D,F).
 *   - The layer entry points (moe_forward*) read x, gate_up_proj and down_proj
 *     and use the workspace in 16-byte units: those four pointers must be
 *     16-byte aligned (MOE_EINVAL otherwise; fresh device allocations are).
 *   - The caller owns every buffer.  The library never writes its inputs,
 *     allocates no device memory and keeps no state; scratch memory is the
 *     caller's workspace, sized by moe_workspace_bytes.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  No entry point synchronises with the host.
 *   - Arguments are validated on the host before anything is enqueued.  On an
 *     error nothing is written and nothing is launched.  MOE_EDEVICE means a
 *     launch failed; outputs are then undefined.
 *   - T = 0 is valid: MOE_OK and no work.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,     /* a size out of range (K not in [1,E], D/F/E <= 0, T < 0,
                         sizes over the library limits) or a NULL required pointer */
  MOE_ENOTSUP = 2,    /* activation other than SwiGLU / ReLU */
  MOE_ETYPE = 3,      /* dtype other than fp32 / bf16 */
  MOE_EWORKSPACE = 4, /* workspace smaller than moe_workspace_bytes */
  MOE_EDEVICE = 5     /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU = 1 } moe_act;

/* Shape and mode of one layer call. */
typedef struct {
  int64_t T;             /* tokens (rows of x), >= 0                        */
  int64_t D;             /* model width, >= 1                               */
  int64_t F;             /* expert hidden width, >= 1                       */
  int32_t E;             /* experts, 1..MOE_MAX_EXPERTS                     */
  int32_t K;             /* experts per token, 1..E                         */
  int32_t norm_topk;     /* 1: renormalise the kept probabilities           */
  int32_t act;           /* moe_act                                         */
  int32_t dtype;         /* moe_dtype of x, router, gate_up_proj, down_proj */
  int32_t out_dtype;     /* moe_dtype of out                                */
  int32_t deterministic; /* 1: out[t] sums its K expert outputs in k order,
                            bitwise reproducible for any K; 0: the down
                            projection adds into out with fp32 atomics
                            (reproducible for K <= 2 only)                 */
} moe_desc;

#define MOE_MAX_EXPERTS 256

/*
 * moe_workspace_bytes -- device scratch needed by moe_forward / moe_dispatch
 * for *d.  Writes the size to *bytes.  MOE_EINVAL / MOE_ETYPE / MOE_ENOTSUP as
 * for moe_forward.  Host-only; touches no device.
 */
moe_status moe_workspace_bytes(const moe_desc* d, size_t* bytes);

/*
 * moe_forward -- the whole layer forward.
 *   x            (T,D)       dtype
 *   router       (E,D)       dtype
 *   gate_up_proj (E,G*F,D)   dtype  (SwiGLU: gate rows [0,F), up rows [F,2F))
 *   down_proj    (E,D,F)     dtype
 *   router_bias  (E)         fp32 or NULL
 *   up_bias      (E,G*F)     fp32 or NULL  (added before the activation)
 *   down_bias    (E,D)       fp32 or NULL  (added to the expert output before
 *                                            it is weighted)
 * Outputs:
 *   out              (T,D)   out_dtype (fp32 recommended for bf16 inputs)
 *   selected_experts (T,K)   int64, descending probability
 *   routing_weights  (T,K)   fp32
 *   router_logits    (T,E)   fp32, or NULL
 *   expert_counts    (E)     int32 tokens routed to each expert, or NULL
 * Precision: router logits and softmax in fp32; expert contractions with
 * fp32 accumulation; for bf16 the gate/up accumulators stay fp32 and the
 * activation output is rounded once to bf16 before the down projection.
 */
moe_status moe_forward(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                       const void* down_proj, const float* router_bias, const float* up_bias,
                       const float* down_bias, void* out, int64_t* selected_experts, float* routing_weights,
                       float* router_logits, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results without the workspace.
 * The scratch memory is a fixed array of MOE_NOALLOC_MAX_BYTES in the
 * library's device code, one per device, held from the first call on a
 * device until the process ends; nothing is allocated per call.  A call whose
 * moe_workspace_bytes exceeds MOE_NOALLOC_MAX_BYTES returns MOE_EWORKSPACE
 * before any launch.  All calls on one device share that device's array:
 * calls that may overlap on one device (other streams, other host threads)
 * race and must be ordered by the caller.  Runs the kernels of moe_forward,
 * so its outputs are bitwise those of moe_forward with deterministic = 1
 * (and of the same atomic adds with 0).  MOE_EDEVICE if the array's device
 * address cannot be obtained.
 */
#define MOE_NOALLOC_MAX_BYTES (128u << 20)
moe_status moe_forward_noalloc(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                               const void* down_proj, const float* router_bias, const float* up_bias,
                               const float* down_bias, void* out, int64_t* selected_experts,
                               float* routing_weights, float* router_logits, int32_t* expert_counts, void* stream);

/*
 * moe_forward_timed -- moe_forward that also records caller-created HIP events
 * (hipEvent_t handles passed as void*) on `stream` at its stage boundaries, so
 * a caller can time each stage with hipEventElapsedTime.  events[0] is
 * recorded before the router, [1] after the router, [2] after the sort into
 * expert order, [3] after the gate_up GEMM, [4] after the down GEMM and [5]
 * after the finalize step (recorded right after [4] when there is none).
 * Only the first min(n_events, MOE_STAGE_EVENTS) are recorded; events may be
 * NULL.  Everything else is exactly moe_forward.
 */
#define MOE_STAGE_EVENTS 6
moe_status moe_forward_timed(const moe_desc* d, const void* x, const void* router, const void* gate_up_proj,
                             const void* down_proj, const float* router_bias, const float* up_bias,
                             const float* down_bias, void* out, int64_t* selected_experts,
                             float* routing_weights, float* router_logits, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                             int32_t n_events);

/*
 * moe_dispatch -- the router and the sort into expert order alone (the
 * "global" dispatch of the Dew page: tokens sorted into expert order so each
 * expert's rows are contiguous).  The order is stable: inside an expert's
 * segment, assignments appear in increasing (t, k).
 *   selected_experts (T,K) int64, routing_weights (T,K) fp32,
 *   router_logits (T,E) fp32 or NULL,
 *   expert_counts (E) int32, expert_offsets (E+1) int32 (exclusive scan of
 *   the counts, expert_offsets[E] = T*K),
 *   sorted_token (T*K) int32: token of the r-th row of the sorted order,
 *   sorted_slot  (T*K) int32: t*K + k of that row.
 * Uses the same workspace as moe_forward (moe_workspace_bytes of d).
 */
moe_status moe_dispatch(const moe_desc* d, const void* x, const void* router, const float* router_bias,
                        int64_t* selected_experts, float* routing_weights, float* router_logits,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token,
                        int32_t* sorted_slot, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routing options (all off when the pointer to this struct is NULL, or when
 * every field is 0 / NULL).
 *
 *   replay_experts   (T,K) int64 device, or NULL.  Routing replay (the Dew
 *                    "Mixture of experts" concepts page, section "Router
 *                    behavior"): a covered token uses the recorded experts in
 *                    place of its own top-k, in the recorded order, and its
 *                    weights still come from this forward's probabilities
 *                    (p_rec / (sum p_rec + 1e-9) when norm_topk).  A token
 *                    whose record holds an index outside [0,E) is not
 *                    covered.  A record may name one expert twice.
 *   replay_mask      (T) uint8 device, or NULL: nonzero where the record covers
 *                    the token (NULL: it covers every token).  An uncovered
 *                    token keeps the router's own top-k.
 *   dynamic_threshold >= 0; 0 is off.  The ES-MoE "API" page, settings table
 *                    of "ESMoE": a slot k >= 1 whose renormalised weight is
 *                    below the threshold is dropped (compared in fp32), the
 *                    leader (k = 0) is always kept, and the kept weights are
 *                    renormalised to sum to one.  Needs norm_topk = 1.  A
 *                    dropped slot keeps its expert in selected_experts, gets
 *                    weight 0 and adds nothing.
 *   capacity_factor  >= 0; 0 is off (every slot kept).  The Dew page, section
 *                    "Expert computation and placement": each sequence of
 *                    seq_len tokens keeps floor(max(ceil(seq_len*K/E) * cf,
 *                    cf)) slots per expert, the first in token order (t, then
 *                    k); a slot dropped by the threshold takes none.  A slot
 *                    dropped for capacity keeps its weight in routing_weights
 *                    but adds nothing to out.
 *   seq_len          tokens per sequence for the capacity; 0 means T.  T must
 *                    be a multiple of it.
 *   kept             (T,K) uint8 device out, or NULL: 1 where the slot
 *                    contributes to out, 0 where the threshold or the
 *                    capacity dropped it.
 *   stats            (MOE_STATS_LEN(E)) fp32 device out, or NULL.  Router
 *                    statistics and the balancing objectives of the ES-MoE
 *                    "API" page, section "Balancing objectives", over the T
 *                    tokens of the call.  With gate (T,E) = each token's
 *                    routing weights at its selected experts (after the
 *                    threshold, before the capacity) and u = the per-expert
 *                    mean normalised to sum to one:
 *                      [0,E)    mean over tokens of p
 *                      [E,2E)   mean over tokens of the gate
 *                      [2E,3E)  mean over tokens of [gate > 0]
 *                      [3E]     switch       = E * sum_i mean(p)_i * mean(gate>0)_i
 *                      [3E+1]   gshard       = E * sum_i u_i^2 (u of the gate)
 *                      [3E+2]   master       = (1/E) * sum_i (u_i - 1/E)^2
 *                      [3E+3]   gshard_probs = E * sum_i u_i^2 (u of p)
 *                    Summed in a fixed order: bitwise reproducible.
 * expert_counts then counts the slots each expert computes (after drops).
 * Invalid values (negative or NaN threshold / factor, a threshold without
 * norm_topk, seq_len < 0 or not dividing T) return MOE_EINVAL.
 */
typedef struct {
  const int64_t* replay_experts;
  const uint8_t* replay_mask;
  float dynamic_threshold;
  double capacity_factor;
  int64_t seq_len;
  uint8_t* kept;
  float* stats;
} moe_routing;
#define MOE_STATS_LEN(E) (3 * (E) + 4)
/* moe_forward with routing options r (NULL: exactly moe_forward). */
moe_status moe_forward_routed(const moe_desc* d, const moe_routing* r, const void* x, const void* router,
                              const void* gate_up_proj, const void* down_proj, const float* router_bias,
                              const float* up_bias, const float* down_bias, void* out, int64_t* selected_experts,
                              float* routing_weights, float* router_logits, int32_t* expert_counts,
                              void* workspace, size_t workspace_bytes, void* stream);
/* moe_dispatch with routing options r (NULL: exactly moe_dispatch).  The
 * sorted order then holds only the kept slots; expert_offsets[E] is their
 * number. */
moe_status moe_dispatch_routed(const moe_desc* d, const moe_routing* r, const void* x, const void* router,
                               const float* router_bias, int64_t* selected_experts, float* routing_weights,
                               float* router_logits, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* sorted_token, int32_t* sorted_slot, void* workspace, size_t workspace_bytes,
                               void* stream);
/* Human-readable text of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* ABI version of this header (bumped on any signature change). */
int32_t moe_abi_version(void);
#define MOE_ABI_VERSION 2

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
