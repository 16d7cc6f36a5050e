/*
 * moe_oracle.h -- plain CPU reference of the sparse Mixture-of-Experts FFN
 * layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source with the HIP
 * library and includes no HIP header.
 *
 * What it computes (the pages it follows are cited on each function):
 *   h_t = u_t + sum_k g_{k,t} * FFN_{e_k}(u_t) + sum_s FFN_s(u_t)
 * with the router, gating variants, capacity/drop rule, dispatch maps and
 * combine written out as their plain definitions, one token at a time.
 *
 * Precision.  Every dot product and every derived quantity is evaluated in
 * double.  Values that the method materialises at a lower precision are
 * rounded to that precision where they are stored, once:
 *   - router scores H are fp32 (the router runs at fp32);
 *   - the gated activation (act) and each expert output y are rounded to the
 *     storage type of the expert path (bf16 round-to-nearest-even, or fp32);
 *   - the sum of the shared experts' outputs is rounded once.
 * The layer output is returned unrounded, in double.
 *
 * Every function is single-threaded per token; functions taking `nthreads`
 * spread independent tokens (or rows) over that many POSIX threads.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };                        /* storage type */
enum { OR_GATE_SOFTMAX_TOPK = 0, OR_GATE_TOPK_SOFTMAX = 1 };
enum { OR_ACT_SWIGLU = 0, OR_ACT_RELU = 1 };
enum { OR_DROP_TOKEN_ORDER = 0, OR_DROP_CHOICE_RANK = 1 };   /* capacity priority */

typedef struct {
  int32_t T, d, N, K, d_ff;     /* tokens, hidden width, experts, top-K, expert width */
  int32_t n_shared, d_ff_shared;/* always-on experts and their width            */
  float capacity_factor;        /* <= 0: no capacity limit                      */
  float noise_weight;           /* W_noise scaling the Gaussian noise input     */
  int32_t gating;               /* OR_GATE_*                                    */
  int32_t act;                  /* OR_ACT_*                                     */
  int32_t dtype;                /* OR_F32 / OR_BF16 for u and expert weights    */
  int32_t drop_order;           /* OR_DROP_*: which assignments a full expert keeps */
} oracle_problem;

/* All weights row-major.  Element type of u and of the expert weights is
 * problem.dtype (bf16 passed as its raw 16-bit pattern). */
typedef struct {
  const void*  u;         /* [T][d]                                   */
  const float* w_router;  /* [N][d]   row i is expert i's centroid    */
  const float* b_router;  /* [N] or NULL                              */
  const float* noise;     /* [T][N] or NULL                           */
  const void*  w_gate;    /* [N][d_ff][d]   (W1 for the ReLU FFN)     */
  const void*  w_up;      /* [N][d_ff][d]   (NULL for the ReLU FFN)   */
  const void*  w_down;    /* [N][d][d_ff]   (W2 for the ReLU FFN)     */
  const void*  ws_gate;   /* [n_shared][d_ff_shared][d] or NULL       */
  const void*  ws_up;     /* [n_shared][d_ff_shared][d] or NULL       */
  const void*  ws_down;   /* [n_shared][d][d_ff_shared] or NULL       */
} oracle_inputs;

/* Round a double to the nearest bf16 value, ties to even (bf16 = the upper
 * 16 bits of an IEEE binary32: 8 significant bits, binary32's exponent
 * range).  Exposed so that tests can pin it against an independent
 * conversion. */
double oracle_round_bf16(double v);

/* Router logits, one fp32 rounding of the exact value
 *   H[t][i] = fp32( sum_j u[t][j]*w_router[i][j] + b[i] + W_noise*noise[t][i] ).
 * MoE-layer equation (affinity u_t^T e_i) of the DeepSeekMoE notes; the
 * router as a linear layer and noise added to the logits before selection
 * (Noise Top-k Gating, "Key implementation details"). */
void oracle_router_logits(const oracle_problem* p, const oracle_inputs* in,
                          float* H, int nthreads);

/* Softmax statistics, top-K selection and gates from fp32 scores H[T][N].
 *   topk_idx[T][K]  experts ordered by (H descending, index ascending)
 *   topk_gate[T][K] variant SOFTMAX_TOPK: the full softmax value s_i;
 *                   variant TOPK_SOFTMAX: softmax over the K selected scores
 *   lse_sq[T]       (log sum_i exp H_i)^2            (may be NULL)
 *   mean_prob[N]    (1/T) sum_t s_{i,t}              (may be NULL)
 *   probs[T][N]     s_{i,t}                          (may be NULL)        */
void oracle_route(const oracle_problem* p, const float* H, int32_t* topk_idx,
                  double* topk_gate, double* lse_sq, double* mean_prob,
                  double* probs);

/* Expert capacity ceil(cf*T*K/N) evaluated in double, capped at T (an expert
 * can hold each token at most once); -1 when cf <= 0 (no limit). */
int32_t oracle_capacity(int32_t T, int32_t K, int32_t N, float cf);

/* Dispatch maps.  Which assignments an expert keeps when more than C choose
 * it (p->drop_order):
 *   OR_DROP_TOKEN_ORDER  the first C in ascending token order
 *   OR_DROP_CHOICE_RANK  the first C in order of (choice rank k, token):
 *                        every token's first choice before any second
 *                        choice, and so on
 * Kept assignments occupy the expert's rows in ascending token order.
 *   expert_counts[N]   assignments per expert before capacity
 *   kept_counts[N]     min(count, C)
 *   offsets[N+1]       exclusive prefix sum of kept_counts
 *   row_of[T][K]       offsets[e] + position among the kept, or -1 if dropped
 *   token_of_row[T*K]  inverse map; -1 past offsets[N]                   */
void oracle_dispatch(const oracle_problem* p, const int32_t* topk_idx,
                     int32_t capacity, int32_t* expert_counts,
                     int32_t* kept_counts, int32_t* offsets, int32_t* row_of,
                     int32_t* token_of_row);

/* Expert FFN outputs for n rows.  Row r applies expert expert_of_row[r]
 * (0..N-1: routed expert; -1: the sum of all shared experts) to the vector
 * x + r*d (element type p->dtype).  y[r][d] receives the materialised
 * output, i.e. rounded once to the storage type. */
void oracle_ffn_rows(const oracle_problem* p, const oracle_inputs* in,
                     int32_t n_rows, const void* x, const int32_t* expert_of_row,
                     double* y, int nthreads);

/* Layer outputs for a list of tokens, given routing and dispatch:
 *   out[r][j] = u[t][j] + sum_{k kept} gate[t][k]*y_{t,k}[j] + y_shared[t][j]
 * with t = tokens[r] (tokens == NULL: every token, n_tokens == T). */
void oracle_layer_rows(const oracle_problem* p, const oracle_inputs* in,
                       const int32_t* topk_idx, const double* topk_gate,
                       const int32_t* row_of, int32_t n_tokens,
                       const int32_t* tokens, double* out, int nthreads);

/* Combine alone, from given expert outputs:
 *   out[t][j] = u[t][j] + sum_{k: row_of[t][k] >= 0} gate[t][k]*y[row_of[t][k]][j]
 *               + y_shared[t][j]
 * y [T*K][d] and y_shared [T][d] (or NULL) in the problem's element type. */
void oracle_combine(const oracle_problem* p, const void* u, const void* y,
                    const int32_t* row_of, const double* gate, const void* y_shared,
                    double* out);

/* The whole forward pass: logits, routing, capacity and dispatch, then the
 * layer output of every token.  Outputs as above; any side output may be
 * NULL except out. */
void oracle_layer_forward(const oracle_problem* p, const oracle_inputs* in,
                          float* H, int32_t* topk_idx, double* topk_gate,
                          double* lse_sq, double* mean_prob,
                          int32_t* expert_counts, int32_t* kept_counts,
                          int32_t* offsets, int32_t* row_of,
                          int32_t* token_of_row, double* out, int nthreads);

/* Router statistics from the side outputs of a forward pass:
 *   stats[0] = (1/N) sum_i (f_i - 1/N)^2,  f_i = expert_counts[i] / (T*K)
 *   stats[1] = (1/N) sum_i (P_i - 1/N)^2,  P_i = mean_prob[i]
 *   stats[2] = -sum_i P_i ln P_i
 *   stats[3] = (1/T) sum_t lse_sq[t]
 * The pages name these quantities (variance of the expert assignment
 * distribution, entropy of the routing probabilities, a penalty on large
 * router logits) without fixing a loss formula; combining them into a loss
 * is the caller's choice. */
void oracle_router_stats(const oracle_problem* p, const int32_t* expert_counts,
                         const double* mean_prob, const double* lse_sq, double* stats);

/* Expert choice ("Mixture of Experts (MoE)" glossary, sparse-MoE entry:
 * experts select their top-k tokens).  Capacity C per expert: the token-
 * choice capacity ceil(cf*T*K/N) capped at T, with cf <= 0 read as 1. */
int32_t oracle_ec_capacity(int32_t T, int32_t K, int32_t N, float cf);

/* Each expert e takes the C tokens with the largest probs[t][e] (ties: the
 * lower token index); its rows e*C .. e*C+C-1 hold them in ascending token
 * order.  probs [T][N] are the affinities s (as double; the GPU's fp32
 * values may be passed widened, so that both sides decide on the same
 * numbers).  C <= T.
 *   expert_tokens [N][C], expert_gates [N][C]: token and gate s of each row
 *   row_of [T][N]: row of (t, e) or -1;  gate_of [T][N]: s or 0          */
void oracle_ec_select(const oracle_problem* p, const double* probs, int32_t C,
                      int32_t* expert_tokens, double* expert_gates, int32_t* row_of,
                      double* gate_of);

/* ------------------------------------------------------------------ */
/* Backward pass.  The gradient of the layer output with respect to u,   */
/* the router weights and bias and the expert weights, given d_out =      */
/* dL/dh.  The routing (Top-K sets, capacity drops) is held fixed, as it  */
/* is piecewise constant in the inputs; gradients reach the router        */
/* through the gates.  Everything in double; the forward values that the  */
/* method materialises (H in fp32, act and y in the storage type) enter   */
/* as stored.                                                             */
/* ------------------------------------------------------------------ */

/* Combine backward:
 *   dy[row][j]   = gate[t][k] * d_out[t][j]       for kept (t, k), row = row_of[t][k]
 *   d_gate[t][k] = sum_j d_out[t][j] * y[row][j]  (0 for a dropped assignment)
 * y [T*K][d] elem, d_out [T][d]; rows of dy that no kept assignment
 * references are left untouched. */
void oracle_combine_backward(const oracle_problem* p, const double* d_out, const void* y,
                             const int32_t* row_of, const double* gate, double* dy,
                             double* d_gate);

/* Gating Jacobian, dH [T][N] from d_gate [T][K]:
 *   SOFTMAX_TOPK (g_k = s_{e_k}, s = softmax over all N of H):
 *     dH_i = s_i (delta_i - sum_k g_k dg_k),  delta_i = dg_k if i = e_k, else 0
 *   TOPK_SOFTMAX (g = softmax over the K selected scores):
 *     dH_{e_k} = g_k (dg_k - sum_m g_m dg_m), every other dH_i = 0 */
void oracle_route_backward(const oracle_problem* p, const float* H, const int32_t* topk_idx,
                           const double* topk_gate, const double* d_gate, double* dH);

/* Router parameters:  dw_router[i][j] = sum_t dH[t][i] u[t][j];
 * db_router[i] = sum_t dH[t][i];  du_router[t][j] = sum_i dH[t][i] w_router[i][j].
 * Any output may be NULL. */
void oracle_router_param_grads(const oracle_problem* p, const oracle_inputs* in,
                               const double* dH, double* dw_router, double* db_router,
                               double* du_router, int nthreads);

/* Expert FFN backward for n rows: row r is the input x + r*d of expert
 * expert_of_row[r] (0..N-1 routed; -1: every shared expert, each receiving
 * the same dy), dy [n][d] the gradient of its output, dx [n][d] the
 * gradient of its input.  With g = W_gate x, v = W_up x, a = SiLU(g) v:
 *   dA = W_down^T dy,  dG = dA v SiLU'(g),  dU = dA SiLU(g),
 *   dx = W_gate^T dG + W_up^T dU
 * (ReLU FFN: dG = dA [g > 0], dx = W_1^T dG). */
void oracle_ffn_backward_rows(const oracle_problem* p, const oracle_inputs* in, int32_t n_rows,
                              const void* x, const int32_t* expert_of_row, const double* dy,
                              double* dx, int nthreads);

/* Weight gradients of one expert for selected hidden units f = f_list[q]:
 *   dw_gate_rows[q][:] = sum_r dG[r][f] x[r][:]     (row f of dW_gate)
 *   dw_up_rows[q][:]   = sum_r dU[r][f] x[r][:]     (row f of dW_up; NULL for ReLU)
 *   dw_down_cols[q][:] = sum_r dy[r][:] a[r][f]     (column f of dW_down)
 * over the n rows of x (elem) and dy (double) that the expert processed;
 * a is the stored activation (rounded to the storage type).  expert =
 * 0..N-1 for a routed expert, -1-s for shared expert s. */
void oracle_ffn_weight_grads(const oracle_problem* p, const oracle_inputs* in, int32_t expert,
                             int32_t n_rows, const void* x, const double* dy, int32_t n_f,
                             const int32_t* f_list, double* dw_gate_rows, double* dw_up_rows,
                             double* dw_down_cols, int nthreads);

/* Whole-layer backward for a list of tokens (tokens == NULL: all T),
 * from the routing of a forward pass:
 *   d_gate[r][k] = <d_out_t, y_{t,k}>, y recomputed and rounded as stored
 *   dH[r][:]     the gating Jacobian applied to d_gate
 *   du[r][:]     = d_out_t + sum_{k kept} dx_{e_k}(g_k d_out_t)
 *                  + dx_shared(d_out_t) + W_router^T dH[r]
 * with t = tokens[r].  d_out [T][d]. */
void oracle_layer_backward_rows(const oracle_problem* p, const oracle_inputs* in,
                                const float* H, const int32_t* topk_idx,
                                const double* topk_gate, const int32_t* row_of,
                                const double* d_out, int32_t n_tokens, const int32_t* tokens,
                                double* du, double* d_gate, double* dH, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
