/*
 * moe_oracle.c -- CPU fp64 oracle of the token-choice top-k MoE feed-forward
 * layer forward pass.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * code, header, table or helper with the HIP path.
 *
 * It is written to be checked by eye against the pages it follows:
 *   [MB]  mojolearn "MoEBlock" API page: the block computes router logits,
 *         a softmax over the experts, keeps the top_k probabilities
 *         (renormalised when norm_topk_prob), each chosen expert computes
 *         down_proj(silu(gate) * up), the output is the weighted sum; ties go
 *         to the lower expert index; weights in the Hugging Face layouts
 *         router (E,D), gate_up_proj (E,2F,D), down_proj (E,D,F) (class
 *         description and "Variables").
 *   [FX]  crackedaicode "Mixture-of-Experts FFN" exercise: ReLU experts
 *         Dense(F)->ReLU->Dense(D) with biases, a Dense(E) router with bias,
 *         softmax, top_k in descending order with equal scores favouring the
 *         lower index, weights = p_sel / (sum p_sel + 1e-9), out[t] =
 *         sum_k w[t,k] * y_{sel[t,k]}[t] (sections "Compute the experts and
 *         router" and "Weight the selected outputs").
 *   [DW]  Dew "Mixture of experts" concepts page, section "Router behavior":
 *         routing replay uses recorded experts in place of the router's own
 *         top-k while the weights still come from this forward's scores; a
 *         token the record does not cover keeps the router's own choice.
 *   [DC]  the same page, section "Expert computation and placement",
 *         capacity_factor: each sequence keeps max(ceil(length * top_k /
 *         experts) * capacity_factor, capacity_factor) slots per expert, taken
 *         in token order; a dropped slot adds nothing to its token's output.
 *   [ES]  ES-MoE "API" page, the settings table of "ESMoE": outside training
 *         dynamic_threshold drops a routed expert whose weight after the top-k
 *         renormalisation is below the threshold, keeps the leader and
 *         renormalises.  (The balancing objectives of its "Balancing
 *         objectives" section are computed in oracle/__init__.py.)
 *
 * Everything is evaluated in double precision from the already-rounded inputs
 * (fp32 values, or bf16 bit patterns widened exactly), with no intermediate
 * rounding, except one step: the top-k *decision* is taken on the
 * probabilities rounded to float32.  Both pages describe the block on float32
 * arrays, so fp32 is the precision in which the pages rank the experts; the
 * weights themselves use the unrounded fp64 probabilities.
 *
 * Parity pins (tests/test_oracle_pins.py): the exercise's two-token worked
 * example, the closed-form parameter count, independent runs of the installed
 * transformers Mixtral and Qwen3-MoE blocks in float64, the E=1/K=1 reduction
 * to plain matrix products, a dense evaluate-every-expert brute force, and
 * the routing invariants.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_SWIGLU = 0, OR_RELU = 1 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENOMEM = 2 };

/* One element of a tensor, widened to double.  bf16 is the top half of a
 * float32, so the widening is exact. */
static double elem(const void *base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float *)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* sum_j row[off + j] * v[j], j = 0..n-1, in order. */
static double dot(const void *w, int dtype, int64_t off, const double *v, int64_t n) {
  double s = 0.0;
  if (dtype == OR_F32) {
    const float *p = (const float *)w + off;
    for (int64_t j = 0; j < n; ++j) s += (double)p[j] * v[j];
  } else {
    for (int64_t j = 0; j < n; ++j) s += elem(w, dtype, off + j) * v[j];
  }
  return s;
}

/* [MB]/[FX]: softmax over the E router logits. */
static void softmax(const double *l, int32_t E, double *p) {
  double m = l[0];
  for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
  double s = 0.0;
  for (int32_t e = 0; e < E; ++e) s += exp(l[e] - m);
  for (int32_t e = 0; e < E; ++e) p[e] = exp(l[e] - m) / s;
}

/* [FX]/[MB]: the K largest probabilities in descending order, equal scores to
 * the lower expert index.  Ranked on float32-rounded probabilities.  Each
 * round scans the experts in ascending order and only a strictly greater
 * value replaces the current best, so a tie keeps the lower index. */
static void select_top_k(const double *p, int32_t E, int32_t K, int64_t *sel, unsigned char *taken) {
  memset(taken, 0, (size_t)E);
  for (int32_t k = 0; k < K; ++k) {
    int32_t best = -1;
    float bv = 0.0f;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      float v = (float)p[e];
      if (best < 0 || v > bv) { best = e; bv = v; }
    }
    taken[best] = 1;
    sel[k] = best;
  }
}

/* [FX] "Weight the selected outputs": w = p_sel / (sum_k p_sel + 1e-9) when
 * renormalising ([MB] norm_topk_prob), the raw p_sel otherwise. */
static void routing_weights(const double *p, const int64_t *sel, int32_t K, int32_t norm, double *w) {
  double denom = 0.0;
  for (int32_t k = 0; k < K; ++k) denom += p[sel[k]];
  denom += 1e-9;
  for (int32_t k = 0; k < K; ++k) w[k] = norm ? p[sel[k]] / denom : p[sel[k]];
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
  int64_t T, D, F;
  int32_t E, K, norm, act, dtype;
  const void *x, *router, *gate_up, *down;
  const float *router_bias, *up_bias, *down_bias;
  const int64_t *tokens; /* which tokens to evaluate; NULL = 0..n-1 */
  int64_t n;
  const int64_t *forced_sel; /* (n,K) replayed selection or NULL */
  const unsigned char *replay_mask; /* (n) tokens the record covers, or NULL: all */
  int32_t replay_lenient;    /* 1: a record with an index outside [0,E) is not used */
  double threshold;          /* [ES] dynamic threshold, 0 = off */
  int32_t mode;              /* which parts one_token runs */
  double *out, *weights, *logits, *probs;
  int64_t *sel;
  unsigned char *kept;       /* (n,K) slot kept, or NULL */
  int64_t begin, end; /* this worker's share of 0..n-1 */
  int status;
} job_t;

enum { RUN_ALL = 0, RUN_ROUTE = 1, RUN_EXPERTS = 2 };

/* Router, softmax, selection and weights of one token (x row already in xr). */
static int route_token(const job_t *J, int64_t i, const double *xr, unsigned char *taken) {
  const int64_t D = J->D;
  const int32_t E = J->E, K = J->K;
  double *l = J->logits + i * E, *p = J->probs + i * E, *w = J->weights + i * K;
  int64_t *sel = J->sel + i * K;

  /* router logits l_e = x . router[e] (+ router bias) */
  for (int32_t e = 0; e < E; ++e)
    l[e] = dot(J->router, J->dtype, (int64_t)e * D, xr, D) + (J->router_bias ? (double)J->router_bias[e] : 0.0);
  softmax(l, E, p);

  int replayed = 0;
  if (J->forced_sel && (!J->replay_mask || J->replay_mask[i])) {
    /* [DW] routing replay: recorded experts, this forward's probabilities. */
    int valid = 1;
    for (int32_t k = 0; k < K; ++k) {
      const int64_t e = J->forced_sel[i * K + k];
      if (e < 0 || e >= E) valid = 0;
    }
    if (!valid && !J->replay_lenient) return OR_EINVAL;
    if (valid) {
      for (int32_t k = 0; k < K; ++k) sel[k] = J->forced_sel[i * K + k];
      replayed = 1;
    }
  }
  if (!replayed) select_top_k(p, E, K, sel, taken);
  routing_weights(p, sel, K, J->norm, w);

  unsigned char keep[K > 0 ? K : 1];
  for (int32_t k = 0; k < K; ++k) keep[k] = 1;
  if (J->threshold > 0.0) {
    /* [ES] dynamic threshold: a non-leading slot whose renormalised weight is
     * below the threshold is dropped (decided in float32, the precision the
     * pages' arrays are in); the kept weights are renormalised to sum to one. */
    double kept_sum = 0.0;
    for (int32_t k = 0; k < K; ++k) {
      if (k > 0 && (float)w[k] < (float)J->threshold) keep[k] = 0;
      if (keep[k]) kept_sum += w[k];
    }
    for (int32_t k = 0; k < K; ++k) w[k] = keep[k] ? w[k] / kept_sum : 0.0;
  }
  if (J->kept)
    for (int32_t k = 0; k < K; ++k) J->kept[i * K + k] = keep[k];
  return OR_OK;
}

/* The selected experts of one token and the weighted sum in ascending k.
 * A slot whose kept flag is 0 adds nothing ([DC]). */
static void experts_token(const job_t *J, int64_t i, const double *xr, double *h, double *y) {
  const int64_t D = J->D, F = J->F;
  const int32_t K = J->K;
  const double *w = J->weights + i * K;
  const int64_t *sel = J->sel + i * K;
  double *o = J->out + i * D;

  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  for (int32_t k = 0; k < K; ++k) {
    if (J->kept && !J->kept[i * K + k]) continue;
    const int64_t e = sel[k];
    if (J->act == OR_SWIGLU) {
      /* gate = rows [0,F) of gate_up_proj[e], up = rows [F,2F) */
      const int64_t base = e * 2 * F * D;
      for (int64_t f = 0; f < F; ++f) {
        double g = dot(J->gate_up, J->dtype, base + f * D, xr, D);
        double u = dot(J->gate_up, J->dtype, base + (F + f) * D, xr, D);
        if (J->up_bias) {
          g += (double)J->up_bias[e * 2 * F + f];
          u += (double)J->up_bias[e * 2 * F + F + f];
        }
        h[f] = silu(g) * u;
      }
    } else {
      /* ReLU expert: h = max(0, W1[e] x + b1[e]) */
      const int64_t base = e * F * D;
      for (int64_t f = 0; f < F; ++f) {
        double a = dot(J->gate_up, J->dtype, base + f * D, xr, D);
        if (J->up_bias) a += (double)J->up_bias[e * F + f];
        h[f] = a > 0.0 ? a : 0.0;
      }
    }
    /* y = down[e] h (+ b2[e]); out += w_k * y */
    for (int64_t d = 0; d < D; ++d) {
      y[d] = dot(J->down, J->dtype, (e * D + d) * F, h, F);
      if (J->down_bias) y[d] += (double)J->down_bias[e * D + d];
      o[d] += w[k] * y[d];
    }
  }
}

/* One token: load its x row, then the parts this job runs. */
static int one_token(const job_t *J, int64_t i, double *xr, double *h, double *y, unsigned char *taken) {
  const int64_t D = J->D;
  const int64_t t = J->tokens ? J->tokens[i] : i;
  for (int64_t d = 0; d < D; ++d) xr[d] = elem(J->x, J->dtype, t * D + d);
  if (J->mode != RUN_EXPERTS) {
    int rc = route_token(J, i, xr, taken);
    if (rc != OR_OK) return rc;
  }
  if (J->mode != RUN_ROUTE) experts_token(J, i, xr, h, y);
  return OR_OK;
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  double *xr = malloc(sizeof(double) * (size_t)J->D);
  double *h = malloc(sizeof(double) * (size_t)J->F);
  double *y = malloc(sizeof(double) * (size_t)J->D);
  unsigned char *taken = malloc((size_t)J->E);
  if (!xr || !h || !y || !taken) {
    J->status = OR_ENOMEM;
  } else {
    for (int64_t i = J->begin; i < J->end && J->status == OR_OK; ++i) J->status = one_token(J, i, xr, h, y, taken);
  }
  free(xr);
  free(h);
  free(y);
  free(taken);
  return NULL;
}

/* Runs `proto` over tokens 0..n-1 split across nthreads workers. */
static int run_jobs(const job_t *proto, int64_t n, int32_t nthreads) {
  if (n == 0) return OR_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int32_t)n;
  job_t *jobs = calloc((size_t)nthreads, sizeof(job_t));
  pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return OR_ENOMEM;
  }
  for (int32_t j = 0; j < nthreads; ++j) {
    jobs[j] = *proto;
    jobs[j].n = n;
    jobs[j].begin = n * j / nthreads;
    jobs[j].end = n * (j + 1) / nthreads;
    jobs[j].status = OR_OK;
  }
  int rc = OR_OK;
  int32_t started = 0;
  for (; started < nthreads; ++started)
    if (pthread_create(&th[started], NULL, worker, &jobs[started]) != 0) break;
  for (int32_t j = started; j < nthreads; ++j) worker(&jobs[j]); /* could not start: run inline */
  for (int32_t j = 0; j < started; ++j) pthread_join(th[j], NULL);
  for (int32_t j = 0; j < nthreads; ++j)
    if (jobs[j].status != OR_OK) rc = jobs[j].status;
  free(jobs);
  free(th);
  return rc;
}

static int check_common(int64_t T, int64_t D, int32_t E, int32_t K, int32_t dtype, const int64_t *tokens,
                        int64_t n) {
  if (T < 0 || D <= 0 || E <= 0 || K < 1 || K > E || n < 0) return OR_EINVAL;
  if (dtype != OR_F32 && dtype != OR_BF16) return OR_EINVAL;
  if (!tokens && n > T) return OR_EINVAL;
  if (tokens)
    for (int64_t i = 0; i < n; ++i)
      if (tokens[i] < 0 || tokens[i] >= T) return OR_EINVAL;
  return OR_OK;
}

/*
 * oracle_forward: evaluate the layer for n tokens.
 *   x (T,D), router (E,D), gate_up (E,G*F,D) with G=2 for SwiGLU and 1 for
 *   ReLU, down (E,D,F): dtype OR_F32 (float) or OR_BF16 (uint16 bit patterns).
 *   router_bias (E), up_bias (E,G*F), down_bias (E,D): float32 or NULL.
 *   tokens (n) selects token rows of x (NULL: tokens 0..n-1, n <= T).
 *   forced_sel (n,K) replays a selection (every index must lie in [0,E)), or
 *   NULL.
 *   Outputs, all row i for the i-th evaluated token: out (n,D), sel (n,K),
 *   weights (n,K), logits (n,E), probs (n,E).
 */
int oracle_forward(int64_t T, int64_t D, int64_t F, int32_t E, int32_t K, int32_t norm, int32_t act,
                   int32_t dtype, const void *x, const void *router, const void *gate_up, const void *down,
                   const float *router_bias, const float *up_bias, const float *down_bias, const int64_t *tokens,
                   int64_t n, const int64_t *forced_sel, double *out, int64_t *sel, double *weights,
                   double *logits, double *probs, int32_t nthreads) {
  if (check_common(T, D, E, K, dtype, tokens, n) != OR_OK || F <= 0) return OR_EINVAL;
  if (act != OR_SWIGLU && act != OR_RELU) return OR_EINVAL;
  if (!x || !router || !gate_up || !down || !out || !sel || !weights || !logits || !probs) return OR_EINVAL;
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.D = D; J.F = F; J.E = E; J.K = K; J.norm = norm; J.act = act; J.dtype = dtype;
  J.x = x; J.router = router; J.gate_up = gate_up; J.down = down;
  J.router_bias = router_bias; J.up_bias = up_bias; J.down_bias = down_bias;
  J.tokens = tokens; J.forced_sel = forced_sel;
  J.out = out; J.weights = weights; J.logits = logits; J.probs = probs; J.sel = sel;
  J.mode = RUN_ALL;
  return run_jobs(&J, n, nthreads);
}

/*
 * oracle_route: the router part alone for n tokens -- logits, softmax,
 * selection, weights -- with the routing options:
 *   replay (n,K) or NULL: [DW] recorded experts.  replay_mask (n) or NULL
 *     (NULL: the record covers every token); a token the record does not
 *     cover, or whose record holds an index outside [0,E), keeps the router's
 *     own top-k.
 *   threshold: [ES] dynamic threshold (0 = off; needs norm).
 * Outputs sel (n,K), weights (n,K) (0 for a dropped slot), logits (n,E),
 * probs (n,E), kept (n,K) 1/0.
 */
int oracle_route(int64_t T, int64_t D, int32_t E, int32_t K, int32_t norm, int32_t dtype, const void *x,
                 const void *router, const float *router_bias, const int64_t *tokens, int64_t n,
                 const int64_t *replay, const unsigned char *replay_mask, double threshold, int64_t *sel,
                 double *weights, double *logits, double *probs, unsigned char *kept, int32_t nthreads) {
  if (check_common(T, D, E, K, dtype, tokens, n) != OR_OK) return OR_EINVAL;
  if (!x || !router || !sel || !weights || !logits || !probs || !kept) return OR_EINVAL;
  if (threshold < 0.0 || (threshold > 0.0 && !norm)) return OR_EINVAL;
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.D = D; J.F = 1; J.E = E; J.K = K; J.norm = norm; J.dtype = dtype;
  J.x = x; J.router = router; J.router_bias = router_bias;
  J.tokens = tokens; J.forced_sel = replay; J.replay_mask = replay_mask; J.replay_lenient = 1;
  J.threshold = threshold;
  J.weights = weights; J.logits = logits; J.probs = probs; J.sel = sel; J.kept = kept;
  J.mode = RUN_ROUTE;
  return run_jobs(&J, n, nthreads);
}

/*
 * oracle_capacity_slots: [DC] slots per expert per sequence,
 * max(ceil(seq_len * K / E) * cf, cf), rounded down to a whole slot count
 * (the page leaves the rounding of a fractional product open).
 */
int64_t oracle_capacity_slots(int64_t seq_len, int32_t K, int32_t E, double cf) {
  const double base = (double)((seq_len * K + E - 1) / E);
  double c = base * cf;
  if (c < cf) c = cf;
  return (int64_t)floor(c);
}

/*
 * oracle_capacity: [DC] capacity drops over sequences of seq_len tokens
 * (T a multiple of seq_len).  Inside each sequence, each expert takes at most
 * `slots` assignments, the first ones in token order (t ascending, then k);
 * an assignment already dropped (kept = 0 on entry, e.g. by the dynamic
 * threshold) takes no slot.  kept (T,K) is updated in place.
 */
int oracle_capacity(int64_t T, int32_t K, int32_t E, int64_t seq_len, int64_t slots, const int64_t *sel,
                    unsigned char *kept) {
  if (T < 0 || K < 1 || E < 1 || seq_len < 1 || T % seq_len != 0 || slots < 0 || !sel || !kept) return OR_EINVAL;
  int64_t *used = malloc(sizeof(int64_t) * (size_t)E);
  if (!used) return OR_ENOMEM;
  for (int64_t s0 = 0; s0 < T; s0 += seq_len) {
    for (int32_t e = 0; e < E; ++e) used[e] = 0;
    for (int64_t t = s0; t < s0 + seq_len; ++t)
      for (int32_t k = 0; k < K; ++k) {
        if (!kept[t * K + k]) continue;
        const int64_t e = sel[t * K + k];
        if (e < 0 || e >= E) {
          free(used);
          return OR_EINVAL;
        }
        if (used[e] < slots)
          used[e] += 1;
        else
          kept[t * K + k] = 0;
      }
  }
  free(used);
  return OR_OK;
}

/*
 * oracle_experts: the expert part alone for n tokens, given each token's
 * selection sel (n,K), weights (n,K) and kept flags (n,K) or NULL (all kept):
 * out[i] = sum over kept k, ascending, of w[i,k] * y_{sel[i,k]}(x[tokens[i]]).
 */
int oracle_experts(int64_t T, int64_t D, int64_t F, int32_t E, int32_t K, int32_t act, int32_t dtype,
                   const void *x, const void *gate_up, const void *down, const float *up_bias,
                   const float *down_bias, const int64_t *tokens, int64_t n, const int64_t *sel,
                   const double *weights, const unsigned char *kept, double *out, int32_t nthreads) {
  if (check_common(T, D, E, K, dtype, tokens, n) != OR_OK || F <= 0) return OR_EINVAL;
  if (act != OR_SWIGLU && act != OR_RELU) return OR_EINVAL;
  if (!x || !gate_up || !down || !sel || !weights || !out) return OR_EINVAL;
  for (int64_t i = 0; i < n * K; ++i)
    if (sel[i] < 0 || sel[i] >= E) return OR_EINVAL;
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.D = D; J.F = F; J.E = E; J.K = K; J.act = act; J.dtype = dtype;
  J.x = x; J.gate_up = gate_up; J.down = down; J.up_bias = up_bias; J.down_bias = down_bias;
  J.tokens = tokens;
  J.out = out;
  J.weights = (double *)weights;  /* read only in this mode */
  J.sel = (int64_t *)sel;         /* read only in this mode */
  J.kept = (unsigned char *)kept; /* read only in this mode */
  J.mode = RUN_EXPERTS;
  return run_jobs(&J, n, nthreads);
}

/*
 * oracle_combine: the selection, weighting and weighted sum alone ([FX]
 * "Weight the selected outputs", the stage its two-token example checks),
 * from given probabilities probs (T,E) and expert outputs expert_outs (T,E,D).
 * Outputs sel (T,K), weights (T,K), out (T,D).
 */
int oracle_combine(int64_t T, int32_t E, int64_t D, int32_t K, int32_t norm, const double *probs,
                   const double *expert_outs, int64_t *sel, double *weights, double *out) {
  if (T < 0 || E <= 0 || D <= 0 || K < 1 || K > E) return OR_EINVAL;
  unsigned char *taken = malloc((size_t)E);
  if (!taken) return OR_ENOMEM;
  for (int64_t t = 0; t < T; ++t) {
    const double *p = probs + t * E;
    int64_t *s = sel + t * K;
    double *w = weights + t * K, *o = out + t * D;
    select_top_k(p, E, K, s, taken);
    routing_weights(p, s, K, norm, w);
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int32_t k = 0; k < K; ++k)
      for (int64_t d = 0; d < D; ++d) o[d] += w[k] * expert_outs[(t * E + s[k]) * D + d];
  }
  free(taken);
  return OR_OK;
}

/* Number of parameters of the layer: per expert G*F*D + D*F weights (+ G*F +
 * D biases), router E*D (+ E bias).  For the exercise's ReLU layer with all
 * biases this is E*(2*D*F + F + D) + D*E + E. */
int64_t oracle_param_count(int64_t D, int64_t F, int32_t E, int32_t act, int32_t expert_biases,
                           int32_t router_bias) {
  const int64_t G = act == OR_SWIGLU ? 2 : 1;
  int64_t per_expert = G * F * D + D * F + (expert_biases ? G * F + D : 0);
  return (int64_t)E * per_expert + (int64_t)E * D + (router_bias ? E : 0);
}
