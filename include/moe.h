/*
 * moe.h -- C ABI of libmoe: the forward pass of one sparse Mixture-of-Experts
 * FFN layer on an AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * The layer (MoE-layer equation of the "Mixture-of-Experts (MoE)" ML notes,
 * which quote DeepSeekMoE):
 *     h_t = sum_{i=1..N} g_{i,t} FFN_i(u_t) + u_t,
 *     g_{i,t} = s_{i,t} if s_{i,t} is among the K largest affinities, else 0,
 *     s_{i,t} = Softmax_i(u_t^T e_i)
 * computed in four stages, one entry point each, plus the chained pass:
 *     moe_route        router GEMM (fp32), softmax, top-K, gates, statistics
 *     moe_dispatch     per-expert histogram, capacity, prefix sum, stable
 *                      permutation of token rows into expert-contiguous rows
 *     moe_grouped_ffn  every expert's FFN over its ragged group of rows
 *     moe_combine      gate-weighted un-permute and sum, plus the residual
 *     moe_layer_forward  the four stages in order on one stream
 *     moe_router_stats   load-balance and z statistics from the side outputs
 *     moe_ec_*           expert-choice routing (experts select their tokens)
 *     moe_layer_backward the gradients of the layer (training)
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller (for example
 *     a torch allocation).  Row-major, densely packed, 16-byte aligned.
 *     The library allocates nothing and keeps no state between calls; it is
 *     re-entrant.  Scratch memory is the caller's workspace `ws` of
 *     `ws_bytes` bytes, at least moe_workspace_size(p) (256-byte aligned).
 *   - `stream` is a hipStream_t (NULL: the null stream).  All work is
 *     enqueued on it; nothing synchronises the host, and the host never reads
 *     data back (ragged sizes stay on the device).
 *   - Outputs are fully overwritten, never accumulated.
 *   - "elem" is the problem's element type: fp32 for MOE_F32, bf16 (raw
 *     16-bit pattern) for MOE_BF16.  It types u, the expert weights, x_perm,
 *     y_perm, y_shared and out.  The router always runs in fp32 (router
 *     weights, bias, noise, scores, gates, probabilities).
 *   - Return value: MOE_OK or an error code.  Every argument check happens
 *     before the first HIP call, so checks are testable without a GPU.
 *     T == 0 returns MOE_OK and touches nothing (pointers are not checked).
 *     NaN or Inf inside the data is undefined behaviour (results unspecified,
 *     never a fault).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* NULL required pointer, bad size or enum, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,  /* valid problem outside what the library implements */
  MOE_ERR_WORKSPACE = 3,    /* ws NULL or ws_bytes below moe_workspace_size() */
  MOE_ERR_HIP = 4           /* a HIP launch failed (hipGetLastError) */
} moe_status_t;

/* Gating variant.
 * MOE_GATE_SOFTMAX_TOPK: softmax over all N experts, the K largest kept with
 *   their softmax values as gates, not renormalised (MoE-layer equation of
 *   the DeepSeekMoE notes).
 * MOE_GATE_TOPK_SOFTMAX: top-K of the scores, then softmax over the K
 *   selected scores only; gates sum to 1 ("Router: Selecting Experts and
 *   Computing Weights", Figure 2 of "MoE: Choosing Which MLPs to Use for
 *   Each Token"). */
enum { MOE_GATE_SOFTMAX_TOPK = 0, MOE_GATE_TOPK_SOFTMAX = 1 };

/* Expert FFN.  Weights use the [out][in] layout, no biases.
 * MOE_ACT_SWIGLU: y = W_down (SiLU(W_gate x) * (W_up x)), SiLU(z) = z/(1+e^-z)
 *   (the gated MLP with Gate, Up and Down weights, Figure 1 of "MoE:
 *   Choosing Which MLPs to Use for Each Token").
 * MOE_ACT_RELU:   y = W_down ReLU(W_gate x)  (w_up unused, NULL). */
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU = 1 };

enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Which assignments an expert keeps when more than C choose it.
 * MOE_DROP_TOKEN_ORDER: the first C in ascending token order (first come,
 *   first served; "Switch Transformers explained", "Making it work").
 * MOE_DROP_CHOICE_RANK: the first C in order of (choice rank k, token):
 *   every token's first choice before any second choice, and so on, the
 *   priority of top-2 gating at scale (the GShard entry of the "Mixture of
 *   Experts (MoE)" glossary).
 * In both, the kept assignments take the expert's rows in token order. */
enum { MOE_DROP_TOKEN_ORDER = 0, MOE_DROP_CHOICE_RANK = 1 };

typedef struct moe_problem {
  int32_t T;            /* tokens (rows of u), >= 0                           */
  int32_t d;            /* hidden width, multiple of 64                       */
  int32_t N;            /* routed experts, 1..256                             */
  int32_t K;            /* experts per token, 1..min(N, 16)                   */
  int32_t d_ff;         /* routed expert width, multiple of 64                */
  int32_t n_shared;     /* always-on shared experts, >= 0                     */
  int32_t d_ff_shared;  /* shared expert width (multiple of 64 if n_shared)   */
  float capacity_factor;/* > 0: capacity C = moe_capacity(T,K,N,cf); <= 0: none */
  float noise_weight;   /* W_noise: scores = logits + W_noise * noise         */
  int32_t gating;       /* MOE_GATE_*                                         */
  int32_t act;          /* MOE_ACT_*                                          */
  int32_t dtype;        /* MOE_F32 or MOE_BF16                                */
  int32_t drop_order;   /* MOE_DROP_*: priority under capacity                */
} moe_problem_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* Bytes of workspace that suffice for every entry point on problem p
 * (0 when p is invalid or T == 0). */
size_t moe_workspace_size(const moe_problem_t* p);

/* Expert capacity: ceil(cf * (T*K) / N) evaluated in double in that order,
 * capped at T (an expert holds each token at most once); -1 when cf <= 0 or
 * cf is NaN (no limit).  Expert capacity = (tokens per batch / experts) *
 * capacity factor, "Mixture of Experts (MoE)" glossary, expert-capacity
 * entry; the K factor counts each (token, expert) assignment. */
int32_t moe_capacity(int32_t T, int32_t K, int32_t N, float cf);

/* Row-tile height of the grouped expert GEMMs (moe_grouped_ffn, the
 * forward and backward passes) over `rows` rows of x_perm split into
 * `groups` expert groups: rows = T*K and groups = N for the routed experts of
 * token choice, rows = N*C for expert choice, rows = T and groups = 1 for the
 * shared experts.  bf16 problems: 256 when the mean group has at least 1024
 * rows (a group's last tile then grows to 320 rows when the group ends at
 * most 64 rows past a multiple of 256, and a group of at most 64 rows gets a
 * 64-row tile), 128 from 128 rows, else 32; fp32 problems: 32.  A planning
 * query with no device work: callers and tests use it to know which kernel
 * a shape reaches.  Returns -1 for rows < 0, groups <= 0 or an unknown dtype. */
int32_t moe_ffn_row_tile(int32_t rows, int32_t groups, int32_t dtype);

/* Stage 1 -- router.
 * scores H[t][i] = fp32(sum_j u[t][j] w_router[i][j] + b_router[i]) then
 *   H = fmaf(W_noise, noise[t][i], H) if noise != NULL ("Noise Top-k
 *   Gating": Gaussian noise scaled by W_noise is added to the logits before
 *   the top-k selection; W_noise = 0 or noise == NULL: plain logits).
 * topk_idx[t][k]: the K experts with the largest H, ordered by (H desc,
 *   index asc); equal scores (+0 == -0) go to the lower index.
 * topk_gate[t][k]: per p->gating (see above).
 * lse_sq[t] = (log sum_i exp H[t][i])^2   (router z-loss term per token)
 * mean_prob[i] = (1/T) sum_t softmax_i(H[t])  (load-balancing statistic P_i)
 * In:  u [T][d] elem; w_router [N][d] fp32 (row i = centroid e_i);
 *      b_router [N] fp32 or NULL; noise [T][N] fp32 or NULL.
 * Out: scores [T][N] fp32 or NULL; topk_idx [T][K] int32; topk_gate [T][K]
 *      fp32; mean_prob [N] fp32; lse_sq [T] fp32.
 * Errors: INVALID_ARG for a NULL required pointer or a NaN W_noise with noise. */
int moe_route(const moe_problem_t* p, const void* u, const float* w_router,
              const float* b_router, const float* noise, float* scores,
              int32_t* topk_idx, float* topk_gate, float* mean_prob,
              float* lse_sq, void* ws, size_t ws_bytes, void* stream);

/* Stage 2 -- dispatch ("From Router to Combine", Figure 3 of "MoE: Choosing
 * Which MLPs to Use for Each Token": inputs are grouped by expert, the same
 * token vector appearing in each of its experts' groups).
 * expert_counts[e]: assignments (t,k) with topk_idx[t][k] == e (before
 *   capacity).
 * Capacity ("Mixture of Experts (MoE)" glossary and "Switch Transformers
 *   explained", "Making it work": overflow is dropped and the token keeps only
 *   the residual): an assignment is kept iff its rank among expert e's
 *   assignments in ascending token order is below C = moe_capacity(...).
 * kept_counts[e] = min(expert_counts[e], C); offsets[0..N] exclusive prefix
 *   sum of kept_counts (offsets[N] = kept rows R).
 * row_of[t][k] = offsets[e] + rank, or -1 when dropped; token_of_row[r] = t
 *   for r < R and -1 for R <= r < T*K.  Rows of one expert ascend in t.
 * x_perm[r] = u[token_of_row[r]] for r < R (rows >= R unspecified).
 * In:  u [T][d] elem; topk_idx [T][K] int32 (each row K distinct experts in
 *      0..N-1; otherwise results are unspecified).
 * Out: expert_counts [N], kept_counts [N], offsets [N+1], row_of [T][K],
 *      token_of_row [T*K] int32; x_perm [T*K][d] elem. */
int moe_dispatch(const moe_problem_t* p, const void* u, const int32_t* topk_idx,
                 int32_t* expert_counts, int32_t* kept_counts, int32_t* offsets,
                 int32_t* row_of, int32_t* token_of_row, void* x_perm, void* ws,
                 size_t ws_bytes, void* stream);

/* Stage 3 -- expert FFNs as grouped GEMMs over ragged groups: rows
 * [offsets[e], offsets[e+1]) of x_perm through expert e ("each expert
 * applies its MLP to the tokens assigned to it ... values of tokens are not
 * mixed", "From Router to Combine").  Shared experts ("Shared Expert",
 * Figure 4): every token u[t] through all n_shared experts, outputs summed.
 * The gated activation is materialised in elem in the workspace; y is
 * rounded to elem once (the shared experts' sum once).
 * In:  x_perm [T*K][d] elem; offsets [N+1] int32 (as from moe_dispatch);
 *      w_gate, w_up [N][d_ff][d] elem (w_up NULL for ReLU);
 *      w_down [N][d][d_ff] elem; u [T][d] elem (shared experts' input, may
 *      be NULL when n_shared == 0); ws_gate, ws_up [n_shared][d_ff_shared][d]
 *      and ws_down [n_shared][d][d_ff_shared] elem (NULL when n_shared == 0).
 * Out: y_perm [T*K][d] elem (rows >= offsets[N] unspecified);
 *      y_shared [T][d] elem (NULL when n_shared == 0). */
int moe_grouped_ffn(const moe_problem_t* p, const void* x_perm,
                    const int32_t* offsets, const void* w_gate, const void* w_up,
                    const void* w_down, const void* u, const void* ws_gate,
                    const void* ws_up, const void* ws_down, void* y_perm,
                    void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* Stage 4 -- combine: out[t] = u[t] + sum_k [row_of[t][k] >= 0]
 *   topk_gate[t][k] * y_perm[row_of[t][k]] + y_shared[t], summed in fp32 in
 *   that order and rounded to elem once ("Combine gathers each expert's
 *   results by the original token", "From Router to Combine"; residual of the
 *   MoE-layer equation; dropped assignments add nothing).
 * In:  u [T][d], y_perm [T*K][d], y_shared [T][d] or NULL (elem);
 *      row_of [T][K] int32; topk_gate [T][K] fp32.
 * Out: out [T][d] elem. */
int moe_combine(const moe_problem_t* p, const void* u, const void* y_perm,
                const int32_t* row_of, const float* topk_gate,
                const void* y_shared, void* out, void* ws, size_t ws_bytes,
                void* stream);

/* Router statistics of one forward pass, from its side outputs, into
 * stats[4] fp32 (device memory):
 *   stats[0]  variance over the N experts of the assignment fractions
 *             f_i = expert_counts[i] / (T*K)  (counts before capacity)
 *   stats[1]  variance over the experts of the mean probabilities mean_prob
 *   stats[2]  entropy -sum_i P_i ln P_i of the mean probabilities
 *   stats[3]  mean over the tokens of lse_sq (the squared log-partition of
 *             the router logits)
 * The "Mixture of Experts (MoE)" glossary (auxiliary-loss entry) names the
 * variance of the expert assignment distribution and the entropy of the
 * routing probabilities as what a load-balancing loss acts on, "Noise Top-k
 * Gating" the variance of routing probability across experts, and the
 * glossary's z-loss entry a penalty on large router logits; the pages fix no
 * loss formula, so forming a loss from these is the caller's.  Variances are
 * population variances (divided by N).  Sums run in double, in a fixed
 * order.  No workspace.
 * In:  expert_counts [N] int32, mean_prob [N] fp32, lse_sq [T] fp32, as
 *      from moe_dispatch and moe_route. */
int moe_router_stats(const moe_problem_t* p, const int32_t* expert_counts,
                     const float* mean_prob, const float* lse_sq, float* stats, void* stream);

/* The weights of one layer (all device pointers, layouts as above). */
typedef struct moe_weights {
  const float* w_router;  /* [N][d] fp32                          */
  const float* b_router;  /* [N] fp32 or NULL                     */
  const void* w_gate;     /* [N][d_ff][d] elem                    */
  const void* w_up;       /* [N][d_ff][d] elem, NULL for ReLU     */
  const void* w_down;     /* [N][d][d_ff] elem                    */
  const void* ws_gate;    /* [n_shared][d_ff_shared][d] or NULL   */
  const void* ws_up;      /* [n_shared][d_ff_shared][d] or NULL   */
  const void* ws_down;    /* [n_shared][d][d_ff_shared] or NULL   */
} moe_weights_t;

/* Every output and intermediate of the chained pass (device pointers).
 * scores may be NULL; y_shared must be non-NULL iff n_shared > 0. */
typedef struct moe_layer_outputs {
  float* scores;          /* [T][N] fp32 or NULL */
  int32_t* topk_idx;      /* [T][K]              */
  float* topk_gate;       /* [T][K]              */
  float* mean_prob;       /* [N]                 */
  float* lse_sq;          /* [T]                 */
  int32_t* expert_counts; /* [N]                 */
  int32_t* kept_counts;   /* [N]                 */
  int32_t* offsets;       /* [N+1]               */
  int32_t* row_of;        /* [T][K]              */
  int32_t* token_of_row;  /* [T*K]               */
  void* x_perm;           /* [T*K][d] elem       */
  void* y_perm;           /* [T*K][d] elem       */
  void* y_shared;         /* [T][d] elem or NULL */
  /* Optional, for training (NULL: not kept; bf16 problems only, else
   * MOE_ERR_UNSUPPORTED): GEMM-1's fp32 pre-activations, which
   * moe_layer_backward then takes instead of recomputing GEMM-1.  Row r of
   * pre holds g = x_perm[r] W_gate^T in columns 0..d_ff-1 and, for SwiGLU,
   * v = x_perm[r] W_up^T in columns d_ff..2*d_ff-1 (ReLU: g only); rows
   * >= offsets[N] unspecified.  pre_shared is the same for the shared
   * experts over every token (width n_shared*d_ff_shared per half), used
   * iff n_shared > 0.  Keeping them adds their writes to the forward pass;
   * the forward's other outputs do not change. */
  float* pre;             /* [T*K][gu*d_ff] fp32 or NULL, gu = 2 (SwiGLU) or 1 */
  float* pre_shared;      /* [T][gu*n_shared*d_ff_shared] fp32 or NULL */
} moe_layer_outputs_t;

/* The whole forward pass: moe_route, moe_dispatch, moe_grouped_ffn and
 * moe_combine in order on `stream`, out [T][d] elem. */
int moe_layer_forward(const moe_problem_t* p, const void* u, const float* noise,
                      const moe_weights_t* w, moe_layer_outputs_t* o, void* out,
                      void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * moe_layer_forward; its scratch memory is instead a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from load until
 * the process ends.  The call allocates and frees nothing.
 *   - Problems whose moe_workspace_size() exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     return MOE_ERR_UNSUPPORTED (before any HIP call); use
 *     moe_layer_forward for them.
 *   - `stream` must belong to the current device (MOE_ERR_INVALID_ARG
 *     otherwise).  The first call on a device looks up that device's copy of
 *     the array (MOE_ERR_HIP if the lookup fails).
 *   - Every call on one GPU shares that GPU's array, and nothing in it needs
 *     to start cleared: each kernel writes the scratch it reads.  Calls that
 *     overlap on one GPU (other streams, other host threads) race on it;
 *     serialise them. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_problem_t* p, const void* u, const float* noise,
                              const moe_weights_t* w, moe_layer_outputs_t* o, void* out,
                              void* stream);

/* ------------------------------------------------------------------ */
/* Backward pass.  The gradient of the layer output h (MoE-layer equation
 * of "Mixture-of-Experts (MoE)", ML notes, through the stages of "From
 * Router to Combine") with respect to u, the router weights and bias and
 * the routed and shared expert weights, given d_out = dL/dh, for bf16
 * problems.  The Top-K sets and capacity decisions of the forward pass are
 * held fixed (they are piecewise constant in the inputs); gradients reach
 * the router through the gates:
 *   dY[row]      = g_{t,k} d_out_t                          (kept (t, k))
 *   d_gate[t][k] = <d_out_t, y_perm[row]>                   (0 if dropped)
 *   d_scores     = the gating variant's Jacobian applied to d_gate
 *                  SOFTMAX_TOPK: dH_i = s_i (delta_i - sum_k g_k dg_k)
 *                  TOPK_SOFTMAX: dH_{e_k} = g_k (dg_k - sum_m g_m dg_m)
 *   dA = dY W_down,  dG = dA v SiLU'(g),  dU = dA SiLU(g)
 *                  g, v: the forward's saved fp32 pre-activations when given
 *                  (moe_saved_t.pre), else recomputed by GEMM-1 with the
 *                  same kernels, so both ways give bit-identical gradients
 *   dX = W_gate^T dG + W_up^T dU;   dW_down = sum_rows dY a^T,
 *   dW_gate = sum_rows dG x^T,  dW_up = sum_rows dU x^T
 *   dW_router = sum_t dH_t u_t^T,  db = sum_t dH_t
 *   du_t = d_out_t + sum_k dX[row_of[t][k]] + dX_shared_t + W_router^T dH_t
 * Shared experts: the same with dY = d_out over every token.  The noise
 * input gets no gradient.
 * Precision: dY, dA, a, dG, dU and dX are stored in bf16; every GEMM and
 * every sum accumulates in fp32 in a fixed order; du and the expert weight
 * gradients are rounded once to bf16; router gradients are fp32.
 * Results are bit-identical run to run. */

/* What the backward needs from the forward pass (its outputs). */
typedef struct moe_saved {
  const float* scores;      /* [T][N] fp32; may be NULL for MOE_GATE_TOPK_SOFTMAX */
  const int32_t* topk_idx;  /* [T][K] */
  const float* topk_gate;   /* [T][K] */
  const int32_t* row_of;    /* [T][K] */
  const int32_t* offsets;   /* [N+1] */
  const void* x_perm;       /* [T*K][d] elem */
  const void* y_perm;       /* [T*K][d] elem */
  const float* pre;         /* moe_layer_outputs_t.pre, or NULL: recompute GEMM-1 */
  const float* pre_shared;  /* moe_layer_outputs_t.pre_shared, or NULL (used iff n_shared > 0) */
} moe_saved_t;

/* Gradients (device pointers, all written).  Weight gradients have the
 * shapes of the weights in moe_weights_t; dw_up (and dws_up) NULL for ReLU;
 * the dws_* are required iff n_shared > 0.  The last four are optional
 * intermediates (NULL: kept in the workspace). */
typedef struct moe_grads {
  void* du;                 /* [T][d] elem  */
  float* dw_router;         /* [N][d] fp32  */
  float* db_router;         /* [N] fp32 or NULL */
  void* dw_gate;
  void* dw_up;
  void* dw_down;
  void* dws_gate;
  void* dws_up;
  void* dws_down;
  float* d_gate;            /* [T][K] fp32 or NULL */
  float* d_scores;          /* [T][N] fp32 or NULL */
  void* dy_perm;            /* [T*K][d] elem or NULL (rows past offsets[N] unspecified) */
  void* dx_perm;            /* [T*K][d] elem or NULL (rows past offsets[N] unspecified) */
} moe_grads_t;

/* Workspace bytes of moe_layer_backward (0 for T == 0 or an invalid p). */
size_t moe_backward_workspace_size(const moe_problem_t* p);

/* The backward pass on `stream`.  In: u, the weights, the forward's saved
 * outputs and d_out [T][d] elem.  Errors: UNSUPPORTED for fp32 problems;
 * INVALID_ARG for a missing required pointer (scores with SOFTMAX_TOPK
 * gating); WORKSPACE if ws_bytes < moe_backward_workspace_size(p). */
int moe_layer_backward(const moe_problem_t* p, const void* u, const moe_weights_t* w,
                       const moe_saved_t* s, const void* d_out, moe_grads_t* g, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Expert choice ("Mixture of Experts (MoE)" glossary, sparse-MoE entry:
 * expert choice lets the experts select their top-k tokens).
 *   affinities  s[t][i] = Softmax over the N experts of token t's router
 *               scores H (the same H as moe_route: fp32 router, bias,
 *               noise), as in the MoE-layer equation;
 *   selection   expert i takes the C tokens of largest s[.][i] (ties: the
 *               lower token index), C = moe_ec_capacity(T, K, N, cf);
 *   rows        expert i owns rows i*C .. i*C+C-1 of x_perm / y_perm, its
 *               tokens in ascending token order;
 *   output      out_t = u_t + sum over the experts i that chose t, in
 *               ascending i, of s[t][i] * FFN_i(u_t), + sum of the shared
 *               experts; fp32 accumulation, one rounding to elem.
 * A token may be chosen by no expert (out_t = u_t + shared) or by several;
 * every expert processes exactly C rows.  Problem fields as for token
 * choice (K only sets C; gating is unused). */

/* C = ceil(cf*T*K/N) capped at T, with cf <= 0 read as 1. */
int32_t moe_ec_capacity(int32_t T, int32_t K, int32_t N, float cf);

/* Workspace bytes of the expert-choice calls (0 for T == 0). */
size_t moe_ec_workspace_size(const moe_problem_t* p);

/* Router scores, affinities and the experts' selections.
 * In:  u [T][d] elem; w_router [N][d], b_router [N] or NULL, noise [T][N]
 *      or NULL (fp32), as for moe_route.
 * Out: scores [T][N] fp32 or NULL; probs [N][T] fp32 (expert-major s);
 *      expert_tokens [N][C] int32; expert_gates [N][C] fp32;
 *      row_of [T][N] int32 (row of (t, i) or -1); gate_of [T][N] fp32
 *      (s[t][i] or 0); offsets [N+1] int32 (i*C); mean_prob [N];
 *      lse_sq [T] (as moe_route). */
int moe_ec_route(const moe_problem_t* p, const void* u, const float* w_router,
                 const float* b_router, const float* noise, float* scores, float* probs,
                 int32_t* expert_tokens, float* expert_gates, int32_t* row_of, float* gate_of,
                 int32_t* offsets, float* mean_prob, float* lse_sq, void* ws, size_t ws_bytes,
                 void* stream);

/* x_perm[i*C + j] = u[expert_tokens[i][j]]: x_perm [N*C][d] elem. */
int moe_ec_dispatch(const moe_problem_t* p, const void* u, const int32_t* expert_tokens,
                    void* x_perm, void* stream);

/* out [T][d] elem from y_perm [N*C][d], row_of / gate_of [T][N] and y_shared
 * [T][d] or NULL (as described above). */
int moe_ec_combine(const moe_problem_t* p, const void* u, const void* y_perm,
                   const int32_t* row_of, const float* gate_of, const void* y_shared, void* out,
                   void* stream);

/* Outputs and intermediates of the chained expert-choice pass. */
typedef struct moe_ec_outputs {
  float* scores;          /* [T][N] fp32 or NULL */
  float* probs;           /* [N][T] fp32         */
  int32_t* expert_tokens; /* [N][C]              */
  float* expert_gates;    /* [N][C]              */
  int32_t* row_of;        /* [T][N]              */
  float* gate_of;         /* [T][N]              */
  int32_t* offsets;       /* [N+1]               */
  float* mean_prob;       /* [N]                 */
  float* lse_sq;          /* [T]                 */
  void* x_perm;           /* [N*C][d] elem       */
  void* y_perm;           /* [N*C][d] elem       */
  void* y_shared;         /* [T][d] elem or NULL */
} moe_ec_outputs_t;

/* moe_ec_route, moe_ec_dispatch, the grouped expert FFN over the N groups
 * of C rows (and the shared experts), and moe_ec_combine, in order on
 * `stream`; ws of at least moe_ec_workspace_size(p) bytes. */
int moe_ec_layer_forward(const moe_problem_t* p, const void* u, const float* noise,
                         const moe_weights_t* w, moe_ec_outputs_t* o, void* out, void* ws,
                         size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
