/*
 * moe_oracle.c -- plain CPU reference of the sparse-MoE FFN layer forward
 * pass.  TEST INFRASTRUCTURE ONLY (see moe_oracle.h): used by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product.
 *
 * Sources (web pages on sparse Mixture-of-Experts):
 *  [MoE-notes]  "Mixture-of-Experts (MoE)", ML notes quoting DeepSeekMoE:
 *               the MoE-layer equation h_t = sum_i g_{i,t} FFN_i(u_t) + u_t,
 *               g = s if s is among the Top-K affinities else 0,
 *               s = Softmax_i(u_t^T e_i).
 *  [LLM-sys]    "MoE: Choosing Which MLPs to Use for Each Token":
 *               Figure 1 (gated-MLP experts with Gate, Up, Down weights),
 *               Figure 2 (Router: top-2 then softmax over the two scores),
 *               Figure 3 (Router -> Dispatch -> Expert -> Combine),
 *               Figure 4 (shared expert: y = S(x) + R(x)).
 *  [Noisy-topk] "Noise Top-k Gating": Gaussian noise scaled by W_noise is
 *               added to the logits before the top-k selection.
 *  [Glossary]   "Mixture of Experts (MoE)" glossary: expert capacity =
 *               (tokens per batch / experts) * capacity factor; overflow is
 *               dropped and takes the residual bypass.
 *  [Switch]     "Switch Transformers ... explained", "Making it work":
 *               overflow tokens skip the layer; higher router precision.
 *
 * Build: plain C11, -O2 -ffp-contract=off, no fast-math (oracle/build.py).
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* element access                                                      */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper half of an IEEE binary32 pattern. */
static double bf16_to_double(uint16_t h) {
  uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int dtype, size_t i) {
  if (dtype == OR_BF16) return bf16_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* dot(a[0..n), b[0..n)) in double, summed left to right */
static double dot_elems(const void* a, size_t a_off, const void* b,
                        size_t b_off, int dtype, int n) {
  double acc = 0.0;
  if (dtype == OR_BF16) {
    const uint16_t* pa = (const uint16_t*)a + a_off;
    const uint16_t* pb = (const uint16_t*)b + b_off;
    for (int j = 0; j < n; ++j) acc += bf16_to_double(pa[j]) * bf16_to_double(pb[j]);
  } else {
    const float* pa = (const float*)a + a_off;
    const float* pb = (const float*)b + b_off;
    for (int j = 0; j < n; ++j) acc += (double)pa[j] * (double)pb[j];
  }
  return acc;
}

/* dot of a double vector with stored elements */
static double dot_dbl_elems(const double* a, const void* b, size_t b_off,
                            int dtype, int n) {
  double acc = 0.0;
  if (dtype == OR_BF16) {
    const uint16_t* pb = (const uint16_t*)b + b_off;
    for (int j = 0; j < n; ++j) acc += a[j] * bf16_to_double(pb[j]);
  } else {
    const float* pb = (const float*)b + b_off;
    for (int j = 0; j < n; ++j) acc += a[j] * (double)pb[j];
  }
  return acc;
}

double oracle_round_bf16(double v) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int e;
  (void)frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
  int q = e - 8;                     /* weight of the 8th significant bit */
  if (q < -133) q = -133;            /* below 2^-126: subnormal step 2^-133 */
  double r = nearbyint(ldexp(fabs(v), -q));  /* default mode: ties to even */
  double out = ldexp(r, q);
  if (out >= ldexp(1.0, 128)) out = INFINITY;
  return copysign(out, v);
}

/* round a value to the storage type of the expert path */
static double round_storage(double v, int dtype) {
  if (dtype == OR_BF16) return oracle_round_bf16(v);
  return (double)(float)v;
}

/* ------------------------------------------------------------------ */
/* threads: contiguous static partition of [0, n)                       */
/* ------------------------------------------------------------------ */

typedef void (*range_fn)(void* ctx, int begin, int end);
typedef struct { range_fn fn; void* ctx; int begin, end; } range_job;

static void* range_entry(void* arg) {
  range_job* j = (range_job*)arg;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

static void parallel_for(int n, int nthreads, range_fn fn, void* ctx) {
  if (n <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = n;
  if (nthreads == 1) { fn(ctx, 0, n); return; }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].begin = (int)((long long)n * i / nthreads);
    jobs[i].end = (int)((long long)n * (i + 1) / nthreads);
    if (pthread_create(&th[i], NULL, range_entry, &jobs[i]) == 0) {
      ++started;
    } else {                         /* no thread: do the range here */
      fn(ctx, jobs[i].begin, jobs[i].end);
      th[i] = (pthread_t)0;
      jobs[i].fn = NULL;
    }
  }
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].fn) pthread_join(th[i], NULL);
  (void)started;
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------ */
/* router logits  [MoE-notes] affinity u_t^T e_i; [Noisy-topk] noise    */
/* ------------------------------------------------------------------ */

typedef struct { const oracle_problem* p; const oracle_inputs* in; float* H; } logits_ctx;

static void logits_range(void* vctx, int t0, int t1) {
  logits_ctx* c = (logits_ctx*)vctx;
  const oracle_problem* p = c->p;
  const oracle_inputs* in = c->in;
  for (int t = t0; t < t1; ++t) {
    for (int i = 0; i < p->N; ++i) {
      double acc = 0.0;
      for (int j = 0; j < p->d; ++j)
        acc += load_elem(in->u, p->dtype, (size_t)t * p->d + j) *
               (double)in->w_router[(size_t)i * p->d + j];
      if (in->b_router) acc += (double)in->b_router[i];
      if (in->noise)
        acc += (double)p->noise_weight * (double)in->noise[(size_t)t * p->N + i];
      c->H[(size_t)t * p->N + i] = (float)acc;   /* the router's fp32 output */
    }
  }
}

void oracle_router_logits(const oracle_problem* p, const oracle_inputs* in,
                          float* H, int nthreads) {
  logits_ctx c = {p, in, H};
  parallel_for(p->T, nthreads, logits_range, &c);
}

/* ------------------------------------------------------------------ */
/* routing  [MoE-notes] softmax, Top-K, gates; [LLM-sys] Figure 2       */
/* ------------------------------------------------------------------ */

void oracle_route(const oracle_problem* p, const float* H, int32_t* topk_idx,
                  double* topk_gate, double* lse_sq, double* mean_prob,
                  double* probs) {
  const int N = p->N, K = p->K;
  double* s = (double*)malloc(sizeof(double) * (size_t)N);
  unsigned char* taken = (unsigned char*)malloc((size_t)N);
  double* psum = (double*)calloc((size_t)N, sizeof(double));
  for (int t = 0; t < p->T; ++t) {
    const float* h = H + (size_t)t * N;
    /* affinity s_i = softmax over all N experts */
    double m = (double)h[0];
    for (int i = 1; i < N; ++i)
      if ((double)h[i] > m) m = (double)h[i];
    double Z = 0.0;
    for (int i = 0; i < N; ++i) Z += exp((double)h[i] - m);
    for (int i = 0; i < N; ++i) {
      s[i] = exp((double)h[i] - m) / Z;
      psum[i] += s[i];
      if (probs) probs[(size_t)t * N + i] = s[i];
    }
    if (lse_sq) {
      double lse = m + log(Z);
      lse_sq[t] = lse * lse;
    }
    /* the K highest scores: K rounds of "largest remaining, lowest index
     * on ties" (a strict > while scanning upwards keeps the lower index) */
    memset(taken, 0, (size_t)N);
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int i = 0; i < N; ++i) {
        if (taken[i]) continue;
        if (best < 0 || h[i] > h[best]) best = i;
      }
      taken[best] = 1;
      topk_idx[(size_t)t * K + k] = best;
    }
    /* gates */
    if (p->gating == OR_GATE_SOFTMAX_TOPK) {
      for (int k = 0; k < K; ++k)
        topk_gate[(size_t)t * K + k] = s[topk_idx[(size_t)t * K + k]];
    } else {
      const double h0 = (double)h[topk_idx[(size_t)t * K]];  /* the largest */
      double zk = 0.0;
      for (int k = 0; k < K; ++k) zk += exp((double)h[topk_idx[(size_t)t * K + k]] - h0);
      for (int k = 0; k < K; ++k)
        topk_gate[(size_t)t * K + k] = exp((double)h[topk_idx[(size_t)t * K + k]] - h0) / zk;
    }
  }
  if (mean_prob)
    for (int i = 0; i < N; ++i) mean_prob[i] = p->T > 0 ? psum[i] / (double)p->T : 0.0;
  free(s);
  free(taken);
  free(psum);
}

/* ------------------------------------------------------------------ */
/* capacity and dispatch  [Glossary] capacity; [LLM-sys] Figure 3       */
/* ------------------------------------------------------------------ */

int32_t oracle_capacity(int32_t T, int32_t K, int32_t N, float cf) {
  if (!(cf > 0.0f)) return -1;
  double c = ceil((double)cf * (double)((int64_t)T * K) / (double)N);
  if (c > (double)T) c = (double)T;
  return (int32_t)c;
}

void oracle_dispatch(const oracle_problem* p, const int32_t* topk_idx,
                     int32_t capacity, int32_t* expert_counts,
                     int32_t* kept_counts, int32_t* offsets, int32_t* row_of,
                     int32_t* token_of_row) {
  const int N = p->N, K = p->K, T = p->T;
  const size_t TK = (size_t)T * K;
  int32_t* prio = (int32_t*)malloc(sizeof(int32_t) * (TK + 1));
  int32_t* fill = (int32_t*)calloc((size_t)N, sizeof(int32_t));
  for (int e = 0; e < N; ++e) expert_counts[e] = 0;
  /* priority rank of each assignment within its expert: first come, first
   * served in ascending token order, or by (choice rank, token) */
  if (p->drop_order == OR_DROP_CHOICE_RANK) {
    for (int k = 0; k < K; ++k)
      for (int t = 0; t < T; ++t) {
        int e = topk_idx[(size_t)t * K + k];
        prio[(size_t)t * K + k] = expert_counts[e]++;
      }
  } else {
    for (int t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k) {
        int e = topk_idx[(size_t)t * K + k];
        prio[(size_t)t * K + k] = expert_counts[e]++;
      }
  }
  for (int e = 0; e < N; ++e)
    kept_counts[e] = (capacity >= 0 && expert_counts[e] > capacity) ? capacity : expert_counts[e];
  offsets[0] = 0;
  for (int e = 0; e < N; ++e) offsets[e + 1] = offsets[e] + kept_counts[e];
  for (size_t r = 0; r < TK; ++r) token_of_row[r] = -1;
  /* the kept assignments take the expert's rows in ascending token order */
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      int e = topk_idx[(size_t)t * K + k];
      if (capacity >= 0 && prio[(size_t)t * K + k] >= capacity) {
        row_of[(size_t)t * K + k] = -1;          /* overflow: dropped */
      } else {
        int32_t row = offsets[e] + fill[e]++;
        row_of[(size_t)t * K + k] = row;
        token_of_row[row] = t;
      }
    }
  free(prio);
  free(fill);
}

/* ------------------------------------------------------------------ */
/* expert FFN  [LLM-sys] Figure 1 gated MLP; [MoE-notes] FFN_i          */
/* ------------------------------------------------------------------ */

/* Unrounded output of one FFN of width dff on vector x (stored at x_off
 * elements into x): act rounded to storage, y in double. */
static void ffn_one(int d, int dff, int act_kind, int dtype, const void* x,
                    size_t x_off, const void* wg, const void* wu,
                    const void* wd, size_t wg_off, size_t wd_off, double* act,
                    double* y) {
  for (int f = 0; f < dff; ++f) {
    double a;
    double g = dot_elems(x, x_off, wg, wg_off + (size_t)f * d, dtype, d);
    if (act_kind == OR_ACT_SWIGLU) {
      double up = dot_elems(x, x_off, wu, wg_off + (size_t)f * d, dtype, d);
      double silu = g / (1.0 + exp(-g));
      a = silu * up;
    } else {
      a = g > 0.0 ? g : 0.0;
    }
    act[f] = round_storage(a, dtype);
  }
  for (int j = 0; j < d; ++j)
    y[j] = dot_dbl_elems(act, wd, wd_off + (size_t)j * dff, dtype, dff);
}

/* routed expert e (e >= 0) or the sum of all shared experts (e == -1),
 * rounded once to storage */
static void expert_output(const oracle_problem* p, const oracle_inputs* in,
                          int e, const void* x, size_t x_off, double* act,
                          double* ytmp, double* y) {
  const int d = p->d;
  if (e >= 0) {
    ffn_one(d, p->d_ff, p->act, p->dtype, x, x_off, in->w_gate, in->w_up,
            in->w_down, (size_t)e * p->d_ff * d, (size_t)e * d * p->d_ff, act, y);
  } else {
    for (int j = 0; j < d; ++j) y[j] = 0.0;
    for (int s = 0; s < p->n_shared; ++s) {
      ffn_one(d, p->d_ff_shared, p->act, p->dtype, x, x_off, in->ws_gate,
              in->ws_up, in->ws_down, (size_t)s * p->d_ff_shared * d,
              (size_t)s * d * p->d_ff_shared, act, ytmp);
      for (int j = 0; j < d; ++j) y[j] += ytmp[j];
    }
  }
  for (int j = 0; j < d; ++j) y[j] = round_storage(y[j], p->dtype);
}

static int max_width(const oracle_problem* p) {
  int w = p->d_ff;
  if (p->n_shared > 0 && p->d_ff_shared > w) w = p->d_ff_shared;
  return w;
}

typedef struct {
  const oracle_problem* p; const oracle_inputs* in;
  const void* x; const int32_t* expert_of_row; double* y;
} ffn_rows_ctx;

static void ffn_rows_range(void* vctx, int r0, int r1) {
  ffn_rows_ctx* c = (ffn_rows_ctx*)vctx;
  const oracle_problem* p = c->p;
  double* act = (double*)malloc(sizeof(double) * (size_t)max_width(p));
  double* ytmp = (double*)malloc(sizeof(double) * (size_t)p->d);
  for (int r = r0; r < r1; ++r)
    expert_output(p, c->in, c->expert_of_row[r], c->x, (size_t)r * p->d, act,
                  ytmp, c->y + (size_t)r * p->d);
  free(act);
  free(ytmp);
}

void oracle_ffn_rows(const oracle_problem* p, const oracle_inputs* in,
                     int32_t n_rows, const void* x, const int32_t* expert_of_row,
                     double* y, int nthreads) {
  ffn_rows_ctx c = {p, in, x, expert_of_row, y};
  parallel_for(n_rows, nthreads, ffn_rows_range, &c);
}

/* ------------------------------------------------------------------ */
/* combine  [MoE-notes] layer equation; [LLM-sys] Figures 3 and 4;     */
/* [Glossary]/[Switch] dropped assignments contribute nothing           */
/* ------------------------------------------------------------------ */

typedef struct {
  const oracle_problem* p; const oracle_inputs* in;
  const int32_t* topk_idx; const double* topk_gate; const int32_t* row_of;
  const int32_t* tokens; double* out;
} layer_ctx;

static void layer_range(void* vctx, int r0, int r1) {
  layer_ctx* c = (layer_ctx*)vctx;
  const oracle_problem* p = c->p;
  const int d = p->d, K = p->K;
  double* act = (double*)malloc(sizeof(double) * (size_t)max_width(p));
  double* ytmp = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  for (int r = r0; r < r1; ++r) {
    int t = c->tokens ? c->tokens[r] : r;
    double* o = c->out + (size_t)r * d;
    size_t u_off = (size_t)t * d;
    for (int j = 0; j < d; ++j) o[j] = load_elem(c->in->u, p->dtype, u_off + j);
    for (int k = 0; k < K; ++k) {
      if (c->row_of[(size_t)t * K + k] < 0) continue;   /* dropped */
      int e = c->topk_idx[(size_t)t * K + k];
      double g = c->topk_gate[(size_t)t * K + k];
      expert_output(p, c->in, e, c->in->u, u_off, act, ytmp, y);
      for (int j = 0; j < d; ++j) o[j] += g * y[j];
    }
    if (p->n_shared > 0) {
      expert_output(p, c->in, -1, c->in->u, u_off, act, ytmp, y);
      for (int j = 0; j < d; ++j) o[j] += y[j];
    }
  }
  free(act);
  free(ytmp);
  free(y);
}

void oracle_layer_rows(const oracle_problem* p, const oracle_inputs* in,
                       const int32_t* topk_idx, const double* topk_gate,
                       const int32_t* row_of, int32_t n_tokens,
                       const int32_t* tokens, double* out, int nthreads) {
  layer_ctx c = {p, in, topk_idx, topk_gate, row_of, tokens, out};
  parallel_for(n_tokens, nthreads, layer_range, &c);
}

void oracle_combine(const oracle_problem* p, const void* u, const void* y,
                    const int32_t* row_of, const double* gate, const void* y_shared,
                    double* out) {
  const int d = p->d, K = p->K;
  for (int t = 0; t < p->T; ++t) {
    double* o = out + (size_t)t * d;
    for (int j = 0; j < d; ++j) o[j] = load_elem(u, p->dtype, (size_t)t * d + j);
    for (int k = 0; k < K; ++k) {
      const int32_t row = row_of[(size_t)t * K + k];
      if (row < 0) continue;                       /* dropped */
      const double g = gate[(size_t)t * K + k];
      for (int j = 0; j < d; ++j) o[j] += g * load_elem(y, p->dtype, (size_t)row * d + j);
    }
    if (y_shared)
      for (int j = 0; j < d; ++j) o[j] += load_elem(y_shared, p->dtype, (size_t)t * d + j);
  }
}

void oracle_layer_forward(const oracle_problem* p, const oracle_inputs* in,
                          float* H, int32_t* topk_idx, double* topk_gate,
                          double* lse_sq, double* mean_prob,
                          int32_t* expert_counts, int32_t* kept_counts,
                          int32_t* offsets, int32_t* row_of,
                          int32_t* token_of_row, double* out, int nthreads) {
  const size_t T = (size_t)p->T, N = (size_t)p->N, K = (size_t)p->K;
  float* h = H ? H : (float*)malloc(sizeof(float) * (T * N + 1));
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)malloc(sizeof(int32_t) * (T * K + 1));
  double* gate = topk_gate ? topk_gate : (double*)malloc(sizeof(double) * (T * K + 1));
  int32_t* cnt = expert_counts ? expert_counts : (int32_t*)malloc(sizeof(int32_t) * N);
  int32_t* kept = kept_counts ? kept_counts : (int32_t*)malloc(sizeof(int32_t) * N);
  int32_t* off = offsets ? offsets : (int32_t*)malloc(sizeof(int32_t) * (N + 1));
  int32_t* rof = row_of ? row_of : (int32_t*)malloc(sizeof(int32_t) * (T * K + 1));
  int32_t* tor = token_of_row ? token_of_row : (int32_t*)malloc(sizeof(int32_t) * (T * K + 1));

  oracle_router_logits(p, in, h, nthreads);
  oracle_route(p, h, idx, gate, lse_sq, mean_prob, NULL);
  int32_t C = oracle_capacity(p->T, p->K, p->N, p->capacity_factor);
  oracle_dispatch(p, idx, C, cnt, kept, off, rof, tor);
  oracle_layer_rows(p, in, idx, gate, rof, p->T, NULL, out, nthreads);

  if (!H) free(h);
  if (!topk_idx) free(idx);
  if (!topk_gate) free(gate);
  if (!expert_counts) free(cnt);
  if (!kept_counts) free(kept);
  if (!offsets) free(off);
  if (!row_of) free(rof);
  if (!token_of_row) free(tor);
}

/* ------------------------------------------------------------------ */
/* router statistics                                                   */
/* "Mixture of Experts (MoE)" glossary, auxiliary-loss and z-loss       */
/* entries; "Noise Top-k Gating", load-balancing entry: the pages name  */
/* the variance of the expert assignment distribution, the entropy of  */
/* the routing probabilities and a penalty on large router logits.     */
/* ------------------------------------------------------------------ */
void oracle_router_stats(const oracle_problem* p, const int32_t* expert_counts,
                         const double* mean_prob, const double* lse_sq, double* stats) {
  const int N = p->N;
  const double n = (double)N;
  const double tk = (double)p->T * (double)p->K;
  /* variance (population, over the N experts) of the assignment fractions */
  double fv = 0.0;
  for (int i = 0; i < N; ++i) {
    const double f = tk > 0.0 ? (double)expert_counts[i] / tk : 0.0;
    const double dlt = f - 1.0 / n;
    fv += dlt * dlt;
  }
  stats[0] = fv / n;
  /* variance of the mean routing probabilities */
  double pv = 0.0;
  for (int i = 0; i < N; ++i) {
    const double dlt = mean_prob[i] - 1.0 / n;
    pv += dlt * dlt;
  }
  stats[1] = pv / n;
  /* entropy of the mean routing probabilities (natural log; 0 log 0 = 0) */
  double ent = 0.0;
  for (int i = 0; i < N; ++i)
    if (mean_prob[i] > 0.0) ent -= mean_prob[i] * log(mean_prob[i]);
  stats[2] = ent;
  /* z-loss: mean over tokens of the squared log-partition of the logits */
  double z = 0.0;
  for (int t = 0; t < p->T; ++t) z += lse_sq[t];
  stats[3] = p->T > 0 ? z / (double)p->T : 0.0;
}

/* ------------------------------------------------------------------ */
/* expert choice  [Glossary] sparse-MoE entry: experts select the       */
/* top-k tokens; [MoE-notes] affinities s = Softmax_i(u_t^T e_i)        */
/* ------------------------------------------------------------------ */

int32_t oracle_ec_capacity(int32_t T, int32_t K, int32_t N, float cf) {
  return oracle_capacity(T, K, N, cf > 0.0f ? cf : 1.0f);
}

typedef struct { double s; int32_t t; } ec_key;

/* s descending, then token ascending */
static int ec_cmp(const void* a, const void* b) {
  const ec_key* x = (const ec_key*)a;
  const ec_key* y = (const ec_key*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t > y->t) - (x->t < y->t);
}

void oracle_ec_select(const oracle_problem* p, const double* probs, int32_t C,
                      int32_t* expert_tokens, double* expert_gates, int32_t* row_of,
                      double* gate_of) {
  const int T = p->T, N = p->N;
  ec_key* keys = (ec_key*)malloc(sizeof(ec_key) * (size_t)(T > 0 ? T : 1));
  unsigned char* sel = (unsigned char*)malloc((size_t)(T > 0 ? T : 1));
  for (size_t i = 0; i < (size_t)T * N; ++i) {
    row_of[i] = -1;
    gate_of[i] = 0.0;
  }
  for (int e = 0; e < N; ++e) {
    for (int t = 0; t < T; ++t) {
      keys[t].s = probs[(size_t)t * N + e];
      keys[t].t = t;
    }
    qsort(keys, (size_t)T, sizeof(ec_key), ec_cmp);
    memset(sel, 0, (size_t)T);
    for (int j = 0; j < C && j < T; ++j) sel[keys[j].t] = 1;
    /* the expert's rows hold its tokens in ascending token order */
    int j = 0;
    for (int t = 0; t < T; ++t) {
      if (!sel[t]) continue;
      const double g = probs[(size_t)t * N + e];
      expert_tokens[(size_t)e * C + j] = t;
      expert_gates[(size_t)e * C + j] = g;
      row_of[(size_t)t * N + e] = e * C + j;
      gate_of[(size_t)t * N + e] = g;
      ++j;
    }
  }
  free(keys);
  free(sel);
}

/* ------------------------------------------------------------------ */
/* backward pass: the chain rule through the forward definitions above  */
/* (combine, gating, router, expert FFNs), one token or row at a time.   */
/* The pages give the forward pass; its gradient is the plain calculus   */
/* of those definitions with the routing held fixed.                     */
/* ------------------------------------------------------------------ */

void oracle_combine_backward(const oracle_problem* p, const double* d_out, const void* y,
                             const int32_t* row_of, const double* gate, double* dy,
                             double* d_gate) {
  const int d = p->d, K = p->K;
  for (int t = 0; t < p->T; ++t) {
    const double* o = d_out + (size_t)t * d;
    for (int k = 0; k < K; ++k) {
      const int32_t row = row_of[(size_t)t * K + k];
      double acc = 0.0;
      if (row >= 0) {
        const double g = gate[(size_t)t * K + k];
        for (int j = 0; j < d; ++j) {
          dy[(size_t)row * d + j] = g * o[j];
          acc += o[j] * load_elem(y, p->dtype, (size_t)row * d + j);
        }
      }
      d_gate[(size_t)t * K + k] = acc;
    }
  }
}

/* dH for one token */
static void gate_jacobian_row(const oracle_problem* p, const float* h, const int32_t* idx,
                              const double* gate, const double* dg, double* dH) {
  const int N = p->N, K = p->K;
  double gdg = 0.0;
  for (int k = 0; k < K; ++k) gdg += gate[k] * dg[k];
  for (int i = 0; i < N; ++i) dH[i] = 0.0;
  if (p->gating == OR_GATE_SOFTMAX_TOPK) {
    /* g_k = s_{e_k}: ds_i/dH_l = s_i (delta_il - s_l) */
    double m = (double)h[0];
    for (int i = 1; i < N; ++i)
      if ((double)h[i] > m) m = (double)h[i];
    double Z = 0.0;
    for (int i = 0; i < N; ++i) Z += exp((double)h[i] - m);
    for (int i = 0; i < N; ++i) {
      double delta = 0.0;
      for (int k = 0; k < K; ++k)
        if (idx[k] == i) delta = dg[k];
      const double s = exp((double)h[i] - m) / Z;
      dH[i] = s * (delta - gdg);
    }
  } else {
    /* g = softmax over the selected scores: dg_k/dH_{e_m} = g_k (delta_km - g_m) */
    for (int k = 0; k < K; ++k) dH[idx[k]] = gate[k] * (dg[k] - gdg);
  }
}

void oracle_route_backward(const oracle_problem* p, const float* H, const int32_t* topk_idx,
                           const double* topk_gate, const double* d_gate, double* dH) {
  const int N = p->N, K = p->K;
  for (int t = 0; t < p->T; ++t)
    gate_jacobian_row(p, H + (size_t)t * N, topk_idx + (size_t)t * K,
                      topk_gate + (size_t)t * K, d_gate + (size_t)t * K, dH + (size_t)t * N);
}

typedef struct {
  const oracle_problem* p; const oracle_inputs* in; const double* dH;
  double* dw_router; double* du_router;
} router_grad_ctx;

/* dW_router rows i in [i0, i1) */
static void router_dw_range(void* vctx, int i0, int i1) {
  router_grad_ctx* c = (router_grad_ctx*)vctx;
  const oracle_problem* p = c->p;
  for (int i = i0; i < i1; ++i)
    for (int j = 0; j < p->d; ++j) {
      double acc = 0.0;
      for (int t = 0; t < p->T; ++t)
        acc += c->dH[(size_t)t * p->N + i] * load_elem(c->in->u, p->dtype, (size_t)t * p->d + j);
      c->dw_router[(size_t)i * p->d + j] = acc;
    }
}

/* du_router rows t in [t0, t1) */
static void router_du_range(void* vctx, int t0, int t1) {
  router_grad_ctx* c = (router_grad_ctx*)vctx;
  const oracle_problem* p = c->p;
  for (int t = t0; t < t1; ++t)
    for (int j = 0; j < p->d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < p->N; ++i)
        acc += c->dH[(size_t)t * p->N + i] * (double)c->in->w_router[(size_t)i * p->d + j];
      c->du_router[(size_t)t * p->d + j] = acc;
    }
}

void oracle_router_param_grads(const oracle_problem* p, const oracle_inputs* in,
                               const double* dH, double* dw_router, double* db_router,
                               double* du_router, int nthreads) {
  router_grad_ctx c = {p, in, dH, dw_router, du_router};
  if (dw_router) parallel_for(p->N, nthreads, router_dw_range, &c);
  if (db_router)
    for (int i = 0; i < p->N; ++i) {
      double acc = 0.0;
      for (int t = 0; t < p->T; ++t) acc += dH[(size_t)t * p->N + i];
      db_router[i] = acc;
    }
  if (du_router) parallel_for(p->T, nthreads, router_du_range, &c);
}

static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/* weights of a routed expert (e >= 0) or of shared expert s (e = -1-s) */
typedef struct {
  int dff;
  const void *wg, *wu, *wd;
  size_t wg_off, wd_off;
} expert_weights;

static expert_weights weights_of(const oracle_problem* p, const oracle_inputs* in, int e) {
  expert_weights w;
  if (e >= 0) {
    w.dff = p->d_ff;
    w.wg = in->w_gate; w.wu = in->w_up; w.wd = in->w_down;
    w.wg_off = (size_t)e * p->d_ff * p->d;
    w.wd_off = (size_t)e * p->d * p->d_ff;
  } else {
    const int s = -1 - e;
    w.dff = p->d_ff_shared;
    w.wg = in->ws_gate; w.wu = in->ws_up; w.wd = in->ws_down;
    w.wg_off = (size_t)s * p->d_ff_shared * p->d;
    w.wd_off = (size_t)s * p->d * p->d_ff_shared;
  }
  return w;
}

/* hidden unit f of one row: g, v and (from dy) the gradients dG, dU and the
 * stored activation a */
static void unit_backward(const oracle_problem* p, const expert_weights* w, const void* x,
                          size_t x_off, const double* dy, int f, double* dG, double* dU,
                          double* a_stored) {
  const int d = p->d;
  const double g = dot_elems(x, x_off, w->wg, w->wg_off + (size_t)f * d, p->dtype, d);
  double dA = 0.0;
  for (int j = 0; j < d; ++j)
    dA += dy[j] * load_elem(w->wd, p->dtype, w->wd_off + (size_t)j * w->dff + f);
  if (p->act == OR_ACT_SWIGLU) {
    const double v = dot_elems(x, x_off, w->wu, w->wg_off + (size_t)f * d, p->dtype, d);
    const double sg = sigmoid(g);
    const double silu = g * sg;
    *dG = dA * v * sg * (1.0 + g * (1.0 - sg));
    *dU = dA * silu;
    if (a_stored) *a_stored = round_storage(silu * v, p->dtype);
  } else {
    *dG = g > 0.0 ? dA : 0.0;
    *dU = 0.0;
    if (a_stored) *a_stored = round_storage(g > 0.0 ? g : 0.0, p->dtype);
  }
}

/* dx += backward of expert e on one row */
static void expert_backward(const oracle_problem* p, const oracle_inputs* in, int e,
                            const void* x, size_t x_off, const double* dy, double* dx) {
  const expert_weights w = weights_of(p, in, e);
  const int d = p->d;
  for (int f = 0; f < w.dff; ++f) {
    double dG, dU;
    unit_backward(p, &w, x, x_off, dy, f, &dG, &dU, NULL);
    for (int i = 0; i < d; ++i) {
      dx[i] += dG * load_elem(w.wg, p->dtype, w.wg_off + (size_t)f * d + i);
      if (p->act == OR_ACT_SWIGLU)
        dx[i] += dU * load_elem(w.wu, p->dtype, w.wg_off + (size_t)f * d + i);
    }
  }
}

typedef struct {
  const oracle_problem* p; const oracle_inputs* in; const void* x;
  const int32_t* expert_of_row; const double* dy; double* dx;
} ffn_bwd_ctx;

static void ffn_bwd_range(void* vctx, int r0, int r1) {
  ffn_bwd_ctx* c = (ffn_bwd_ctx*)vctx;
  const oracle_problem* p = c->p;
  const int d = p->d;
  for (int r = r0; r < r1; ++r) {
    double* dx = c->dx + (size_t)r * d;
    const double* dy = c->dy + (size_t)r * d;
    for (int i = 0; i < d; ++i) dx[i] = 0.0;
    const int e = c->expert_of_row[r];
    if (e >= 0) {
      expert_backward(p, c->in, e, c->x, (size_t)r * d, dy, dx);
    } else {
      for (int s = 0; s < p->n_shared; ++s)
        expert_backward(p, c->in, -1 - s, c->x, (size_t)r * d, dy, dx);
    }
  }
}

void oracle_ffn_backward_rows(const oracle_problem* p, const oracle_inputs* in, int32_t n_rows,
                              const void* x, const int32_t* expert_of_row, const double* dy,
                              double* dx, int nthreads) {
  ffn_bwd_ctx c = {p, in, x, expert_of_row, dy, dx};
  parallel_for(n_rows, nthreads, ffn_bwd_range, &c);
}

typedef struct {
  const oracle_problem* p; const oracle_inputs* in; int expert; int n_rows;
  const void* x; const double* dy; const int32_t* f_list;
  double *dwg, *dwu, *dwd;
} wgrad_ctx;

static void wgrad_range(void* vctx, int q0, int q1) {
  wgrad_ctx* c = (wgrad_ctx*)vctx;
  const oracle_problem* p = c->p;
  const int d = p->d;
  const expert_weights w = weights_of(p, c->in, c->expert);
  for (int q = q0; q < q1; ++q) {
    const int f = c->f_list[q];
    double* g_row = c->dwg + (size_t)q * d;
    double* u_row = c->dwu ? c->dwu + (size_t)q * d : NULL;
    double* d_col = c->dwd + (size_t)q * d;
    for (int i = 0; i < d; ++i) {
      g_row[i] = 0.0;
      if (u_row) u_row[i] = 0.0;
      d_col[i] = 0.0;
    }
    for (int r = 0; r < c->n_rows; ++r) {
      double dG, dU, a;
      const double* dy = c->dy + (size_t)r * d;
      unit_backward(p, &w, c->x, (size_t)r * d, dy, f, &dG, &dU, &a);
      for (int i = 0; i < d; ++i) {
        const double xi = load_elem(c->x, p->dtype, (size_t)r * d + i);
        g_row[i] += dG * xi;
        if (u_row) u_row[i] += dU * xi;
        d_col[i] += dy[i] * a;
      }
    }
  }
}

void oracle_ffn_weight_grads(const oracle_problem* p, const oracle_inputs* in, int32_t expert,
                             int32_t n_rows, const void* x, const double* dy, int32_t n_f,
                             const int32_t* f_list, double* dw_gate_rows, double* dw_up_rows,
                             double* dw_down_cols, int nthreads) {
  wgrad_ctx c = {p, in, expert, n_rows, x, dy, f_list, dw_gate_rows,
                 p->act == OR_ACT_SWIGLU ? dw_up_rows : NULL, dw_down_cols};
  parallel_for(n_f, nthreads, wgrad_range, &c);
}

typedef struct {
  const oracle_problem* p; const oracle_inputs* in; const float* H;
  const int32_t* topk_idx; const double* topk_gate; const int32_t* row_of;
  const double* d_out; const int32_t* tokens; double *du, *d_gate, *dH;
} layer_bwd_ctx;

static void layer_bwd_range(void* vctx, int r0, int r1) {
  layer_bwd_ctx* c = (layer_bwd_ctx*)vctx;
  const oracle_problem* p = c->p;
  const int d = p->d, K = p->K, N = p->N;
  double* act = (double*)malloc(sizeof(double) * (size_t)max_width(p));
  double* ytmp = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  double* dy = (double*)malloc(sizeof(double) * (size_t)d);
  for (int r = r0; r < r1; ++r) {
    const int t = c->tokens ? c->tokens[r] : r;
    const double* o = c->d_out + (size_t)t * d;
    const size_t u_off = (size_t)t * d;
    double* du = c->du + (size_t)r * d;
    double* dg = c->d_gate + (size_t)r * K;
    double* dH = c->dH + (size_t)r * N;
    for (int j = 0; j < d; ++j) du[j] = o[j];                 /* residual */
    for (int k = 0; k < K; ++k) {
      dg[k] = 0.0;
      if (c->row_of[(size_t)t * K + k] < 0) continue;        /* dropped */
      const int e = c->topk_idx[(size_t)t * K + k];
      const double g = c->topk_gate[(size_t)t * K + k];
      expert_output(p, c->in, e, c->in->u, u_off, act, ytmp, y);
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += o[j] * y[j];
      dg[k] = acc;
      for (int j = 0; j < d; ++j) dy[j] = g * o[j];
      expert_backward(p, c->in, e, c->in->u, u_off, dy, du);
    }
    for (int s = 0; s < p->n_shared; ++s)
      expert_backward(p, c->in, -1 - s, c->in->u, u_off, o, du);
    gate_jacobian_row(p, c->H + (size_t)t * N, c->topk_idx + (size_t)t * K,
                      c->topk_gate + (size_t)t * K, dg, dH);
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < N; ++i) acc += dH[i] * (double)c->in->w_router[(size_t)i * d + j];
      du[j] += acc;
    }
  }
  free(act);
  free(ytmp);
  free(y);
  free(dy);
}

void oracle_layer_backward_rows(const oracle_problem* p, const oracle_inputs* in,
                                const float* H, const int32_t* topk_idx,
                                const double* topk_gate, const int32_t* row_of,
                                const double* d_out, int32_t n_tokens, const int32_t* tokens,
                                double* du, double* d_gate, double* dH, int nthreads) {
  layer_bwd_ctx c = {p, in, H, topk_idx, topk_gate, row_of, d_out, tokens, du, d_gate, dH};
  parallel_for(n_tokens, nthreads, layer_bwd_range, &c);
}
