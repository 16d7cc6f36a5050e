// libmoe C ABI: argument checks, workspace layout and launch sequencing.
// Every check runs before the first HIP call, so a bad argument never
// reaches the device; all work is enqueued on the caller's stream.
#include <math.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

Workspace workspace_layout(const moe_problem_t& p) {
  Workspace w{};
  const size_t T = (size_t)p.T, N = (size_t)p.N, K = (size_t)p.K;
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int rt = route_tokens_per_block(p);
  w.route_blocks = (int)((T + rt - 1) / rt);
  w.disp_blocks = (int)((T + kDispatchTok - 1) / kDispatchTok);
  size_t off = 0;
  w.route_part = off;
  off = align_up(off + (size_t)w.route_blocks * N * 4, kAlign);
  w.route_pre = off;
  off = align_up(off + route_pre_bytes(p), kAlign);
  w.disp_count = off;
  off = align_up(off + (size_t)w.disp_blocks * K * N * 4, kAlign);
  w.disp_base = off;
  off = align_up(off + (size_t)w.disp_blocks * K * N * 4, kAlign);
  w.disp_q = off;
  off = align_up(off + K * N * 4, kAlign);
  w.tiles = off;
  off = align_up(off + gemm_plan_bytes(N), kAlign);
  w.act = off;
  off = align_up(off + T * K * (size_t)p.d_ff * es, kAlign);
  w.act_shared = off;
  if (p.n_shared > 0) off = align_up(off + T * (size_t)p.n_shared * p.d_ff_shared * es, kAlign);
  const bool bf16 = p.dtype == MOE_BF16;
  w.has_split = bf16 && (ffn_row_tile(p.T * p.K, p.N, true) == 256 ||
                         (p.n_shared > 0 && ffn_row_tile(p.T, 1, true) == 256));
  w.split = off;
  if (w.has_split) off = align_up(off + kSplitBytes, kAlign);
  w.total = off;
  return w;
}

static int32_t ec_capacity_of(int32_t T, int32_t K, int32_t N, float cf) {
  const float c = cf > 0.0f ? cf : 1.0f;
  double v = ceil((double)c * (double)((int64_t)T * K) / (double)N);
  if (v > (double)T) v = (double)T;
  return (int32_t)v;
}

EcWorkspace ec_workspace_layout(const moe_problem_t& p) {
  EcWorkspace w{};
  const size_t T = (size_t)p.T, N = (size_t)p.N, K = (size_t)p.K;
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int rt = route_tokens_per_block(p);
  w.route_blocks = (int)((T + rt - 1) / rt);
  w.C = ec_capacity_of(p.T, p.K, p.N, p.capacity_factor);
  size_t off = 0;
  w.route_part = off;
  off = align_up(off + (size_t)w.route_blocks * N * 4, kAlign);
  w.route_pre = off;
  off = align_up(off + route_pre_bytes(p), kAlign);
  w.scores = off;
  off = align_up(off + T * N * 4, kAlign);
  w.tk_idx = off;
  off = align_up(off + T * K * 4, kAlign);
  w.tk_gate = off;
  off = align_up(off + T * K * 4, kAlign);
  w.sel = off;
  off = align_up(off + ec_select_bytes(p.T, p.N), kAlign);
  w.tiles = off;
  off = align_up(off + gemm_plan_bytes(N), kAlign);
  w.act = off;
  off = align_up(off + N * (size_t)w.C * (size_t)p.d_ff * es, kAlign);
  w.act_shared = off;
  if (p.n_shared > 0) off = align_up(off + T * (size_t)p.n_shared * p.d_ff_shared * es, kAlign);
  w.total = off;
  return w;
}

BwdWorkspace bwd_workspace_layout(const moe_problem_t& p) {
  BwdWorkspace w{};
  const size_t T = (size_t)p.T, N = (size_t)p.N, K = (size_t)p.K, d = (size_t)p.d;
  const size_t rows = T * K, dff = (size_t)p.d_ff, es = 2;
  const size_t gu = p.act == MOE_ACT_SWIGLU ? 2 : 1;
  const size_t wsw = (size_t)p.n_shared * p.d_ff_shared;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, kAlign);
    return at;
  };
  w.tiles = take(2 * (N + 2) * 4);
  w.dy_perm = take(rows * d * es);
  w.dA = take(rows * dff * es);
  w.act = take(rows * dff * es);
  w.dgu = take(rows * gu * dff * es);
  w.dx_perm = take(rows * d * es);
  w.d_gate = take(T * K * 4);
  w.dH = take(T * N * 4);
  w.partial = take((size_t)router_grad_slices(p.T, N) * N * (d + 1) * 4);
  if (p.n_shared > 0) {
    w.dA_s = take(T * wsw * es);
    w.act_s = take(T * wsw * es);
    w.dgu_s = take(T * gu * wsw * es);
    w.dx_shared = take(T * d * es);
  }
  w.ldt = wgrad_transposed_ld(p);
  if (w.ldt > 0) {
    w.kpad = take((N + 1) * 4);
    w.dyT = take(d * (size_t)w.ldt * es);
    w.xT = take(d * (size_t)w.ldt * es);
    // the shared experts join the transposed launches while their operands
    // stay within one 32-bit buffer descriptor each
    const long long ts = (long long)(T + 63) / 64 * 64;
    if (p.n_shared > 0 && ts <= (1LL << 22) && (long long)T * gu * wsw * 2 < (1LL << 31)) {
      w.ldts = (int)ts;
      w.dOT = take(d * (size_t)ts * es);
      w.uT = take(d * (size_t)ts * es);
    }
  }
  w.total = off;
  return w;
}

int wgrad_transposed_ld(const moe_problem_t& p) {
  const long long rows = (long long)p.T * p.K;
  if (rows < 512LL * p.N) return 0;            // short groups: the direct kernel
  const long long ld = (rows + 63LL * p.N + 63) / 64 * 64;
  // a 256-row tile of the transposed operand is addressed through one buffer
  // descriptor, whose size is 32-bit: 256 * ld * 2 bytes stays below 2 GiB;
  // so is each group's k-major operand, at most rows x 2 d_ff elements
  const long long gu = p.act == MOE_ACT_SWIGLU ? 2 : 1;
  if (rows * gu * p.d_ff * 2 >= (1LL << 31)) return 0;
  return ld <= (1LL << 22) ? (int)ld : 0;
}

}  // namespace moe

using moe::Workspace;
using moe::EcWorkspace;

namespace {

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Structural checks of the problem descriptor.
int check_problem(const moe_problem_t* p) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  if (p->T < 0 || p->d <= 0 || p->N <= 0 || p->K <= 0 || p->d_ff <= 0 || p->n_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (p->K > p->N) return MOE_ERR_INVALID_ARG;
  if (p->n_shared > 0 && p->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_GATE_SOFTMAX_TOPK && p->gating != MOE_GATE_TOPK_SOFTMAX)
    return MOE_ERR_INVALID_ARG;
  if (p->act != MOE_ACT_SWIGLU && p->act != MOE_ACT_RELU) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (isnan(p->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (p->drop_order != MOE_DROP_TOKEN_ORDER && p->drop_order != MOE_DROP_CHOICE_RANK)
    return MOE_ERR_INVALID_ARG;
  // valid, but outside what the kernels implement
  if (p->N > 256 || p->K > 16) return MOE_ERR_UNSUPPORTED;
  if (p->d % 64 != 0 || p->d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (p->n_shared > 0 && p->d_ff_shared % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const long long rows = (long long)p->T * p->K;
  if (rows > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
  if ((long long)p->n_shared * p->d_ff_shared > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
  if ((long long)p->d * p->d_ff > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  // the grouped GEMMs address a row tile (at most 320 rows) of an operand
  // through a buffer descriptor whose size field is 32 bits
  long long ld = p->d;
  const long long gu = p->act == MOE_ACT_SWIGLU ? 2 : 1;
  if (gu * p->d_ff > ld) ld = gu * p->d_ff;
  if (gu * p->n_shared * (long long)p->d_ff_shared > ld) ld = gu * p->n_shared * (long long)p->d_ff_shared;
  if (320LL * ld * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Required device buffers: non-null and aligned (16 bytes for anything read
// or written in 16-byte vectors, 4 bytes otherwise).
int need(const void* ptr, size_t align) {
  if (ptr == nullptr) return MOE_ERR_INVALID_ARG;
  return aligned(ptr, align) ? MOE_OK : MOE_ERR_INVALID_ARG;
}
int maybe(const void* ptr, size_t align) {
  return (ptr == nullptr || aligned(ptr, align)) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

#define MOE_TRY(x)                 \
  do {                             \
    const int moe_s_ = (x);        \
    if (moe_s_ != MOE_OK) return moe_s_; \
  } while (0)

int check_ws(void* ws, size_t ws_bytes, size_t required) {
  if (required == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < required || !aligned(ws, moe::kAlign)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int check_route(const moe_problem_t* p, const void* u, const float* w_router,
                const float* b_router, const float* noise, const float* scores,
                const int32_t* topk_idx, const float* topk_gate, const float* mean_prob,
                const float* lse_sq) {
  MOE_TRY(need(u, 16));
  MOE_TRY(need(w_router, 16));
  MOE_TRY(maybe(b_router, 4));
  MOE_TRY(maybe(noise, 4));
  MOE_TRY(maybe(scores, 4));
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(topk_gate, 4));
  MOE_TRY(need(mean_prob, 4));
  MOE_TRY(need(lse_sq, 4));
  if (noise != nullptr && !isfinite(p->noise_weight)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_dispatch(const void* u, const int32_t* topk_idx, const int32_t* expert_counts,
                   const int32_t* kept_counts, const int32_t* offsets, const int32_t* row_of,
                   const int32_t* token_of_row, const void* x_perm) {
  MOE_TRY(need(u, 16));
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(need(kept_counts, 4));
  MOE_TRY(need(offsets, 4));
  MOE_TRY(need(row_of, 4));
  MOE_TRY(need(token_of_row, 4));
  MOE_TRY(need(x_perm, 16));
  return MOE_OK;
}

int check_ffn(const moe_problem_t* p, const void* x_perm, const int32_t* offsets,
              const void* w_gate, const void* w_up, const void* w_down, const void* u,
              const void* ws_gate, const void* ws_up, const void* ws_down, const void* y_perm,
              const void* y_shared) {
  MOE_TRY(need(x_perm, 16));
  MOE_TRY(need(offsets, 4));
  MOE_TRY(need(w_gate, 16));
  if (p->act == MOE_ACT_SWIGLU) MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(y_perm, 16));
  if (p->n_shared > 0) {
    MOE_TRY(need(u, 16));
    MOE_TRY(need(ws_gate, 16));
    if (p->act == MOE_ACT_SWIGLU) MOE_TRY(need(ws_up, 16));
    MOE_TRY(need(ws_down, 16));
    MOE_TRY(need(y_shared, 16));
  }
  return MOE_OK;
}

int check_combine(const moe_problem_t* p, const void* u, const void* y_perm,
                  const int32_t* row_of, const float* topk_gate, const void* y_shared,
                  const void* out) {
  MOE_TRY(need(u, 16));
  MOE_TRY(need(y_perm, 16));
  MOE_TRY(need(row_of, 4));
  MOE_TRY(need(topk_gate, 4));
  MOE_TRY(need(out, 16));
  if (p->n_shared > 0) MOE_TRY(need(y_shared, 16));
  else MOE_TRY(maybe(y_shared, 16));
  return MOE_OK;
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: problem outside the implemented range";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe status";
  }
}

size_t moe_workspace_size(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK || p->T == 0) return 0;
  return moe::workspace_layout(*p).total;
}

int32_t moe_capacity(int32_t T, int32_t K, int32_t N, float cf) {
  if (!(cf > 0.0f) || N <= 0 || T < 0 || K < 0) return -1;
  double c = ceil((double)cf * (double)((int64_t)T * K) / (double)N);
  if (c > (double)T) c = (double)T;
  return (int32_t)c;
}

int32_t moe_ffn_row_tile(int32_t rows, int32_t groups, int32_t dtype) {
  if (rows < 0 || groups <= 0 || (dtype != MOE_F32 && dtype != MOE_BF16)) return -1;
  return moe::ffn_row_tile(rows, groups, dtype == MOE_BF16);
}

int moe_route(const moe_problem_t* p, const void* u, const float* w_router,
              const float* b_router, const float* noise, float* scores, int32_t* topk_idx,
              float* topk_gate, float* mean_prob, float* lse_sq, void* ws, size_t ws_bytes,
              void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_route(p, u, w_router, b_router, noise, scores, topk_idx, topk_gate, mean_prob,
                      lse_sq));
  const Workspace w = moe::workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.disp_count));
  return hip_status(moe::launch_route(*p, u, w_router, b_router, noise, scores, topk_idx,
                                      topk_gate, mean_prob, lse_sq,
                                      reinterpret_cast<float*>(ws_at(ws, w.route_part)),
                                      w.route_blocks,
                                      reinterpret_cast<float*>(ws_at(ws, w.route_pre)),
                                      static_cast<hipStream_t>(stream)));
}

int moe_dispatch(const moe_problem_t* p, const void* u, const int32_t* topk_idx,
                 int32_t* expert_counts, int32_t* kept_counts, int32_t* offsets, int32_t* row_of,
                 int32_t* token_of_row, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_dispatch(u, topk_idx, expert_counts, kept_counts, offsets, row_of, token_of_row,
                         x_perm));
  const Workspace w = moe::workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.tiles));
  const int32_t C = moe_capacity(p->T, p->K, p->N, p->capacity_factor);
  return hip_status(moe::launch_dispatch(
      *p, u, topk_idx, C, expert_counts, kept_counts, offsets, row_of, token_of_row, x_perm,
      reinterpret_cast<int32_t*>(ws_at(ws, w.disp_count)),
      reinterpret_cast<int32_t*>(ws_at(ws, w.disp_base)),
      reinterpret_cast<int32_t*>(ws_at(ws, w.disp_q)), w.disp_blocks,
      static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn(const moe_problem_t* p, const void* x_perm, const int32_t* offsets,
                    const void* w_gate, const void* w_up, const void* w_down, const void* u,
                    const void* ws_gate, const void* ws_up, const void* ws_down, void* y_perm,
                    void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_ffn(p, x_perm, offsets, w_gate, w_up, w_down, u, ws_gate, ws_up, ws_down, y_perm,
                    y_shared));
  const Workspace w = moe::workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.total));
  return hip_status(moe::launch_grouped_ffn(
      *p, p->T * p->K, x_perm, offsets, w_gate, w_up, w_down, u, ws_gate, ws_up, ws_down, y_perm,
      p->n_shared > 0 ? y_shared : nullptr, reinterpret_cast<int32_t*>(ws_at(ws, w.tiles)),
      ws_at(ws, w.act), ws_at(ws, w.act_shared),
      w.has_split ? reinterpret_cast<float*>(ws_at(ws, w.split)) : nullptr,
      static_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_problem_t* p, const void* u, const void* y_perm, const int32_t* row_of,
                const float* topk_gate, const void* y_shared, void* out, void* ws,
                size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_combine(p, u, y_perm, row_of, topk_gate, y_shared, out));
  return hip_status(moe::launch_combine(*p, u, y_perm, row_of, topk_gate,
                                        p->n_shared > 0 ? y_shared : nullptr, out,
                                        static_cast<hipStream_t>(stream)));
}

int moe_router_stats(const moe_problem_t* p, const int32_t* expert_counts,
                     const float* mean_prob, const float* lse_sq, float* stats, void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(need(mean_prob, 4));
  MOE_TRY(need(lse_sq, 4));
  MOE_TRY(need(stats, 4));
  return hip_status(moe::launch_router_stats(*p, expert_counts, mean_prob, lse_sq, stats,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of moe_layer_forward's arguments other than the workspace.
int check_layer(const moe_problem_t* p, const void* u, const float* noise,
                const moe_weights_t* wt, const moe_layer_outputs_t* o, const void* out) {
  if (wt == nullptr || o == nullptr) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_route(p, u, wt->w_router, wt->b_router, noise, o->scores, o->topk_idx,
                      o->topk_gate, o->mean_prob, o->lse_sq));
  MOE_TRY(check_dispatch(u, o->topk_idx, o->expert_counts, o->kept_counts, o->offsets,
                         o->row_of, o->token_of_row, o->x_perm));
  MOE_TRY(check_ffn(p, o->x_perm, o->offsets, wt->w_gate, wt->w_up, wt->w_down, u, wt->ws_gate,
                    wt->ws_up, wt->ws_down, o->y_perm, o->y_shared));
  MOE_TRY(check_combine(p, u, o->y_perm, o->row_of, o->topk_gate, o->y_shared, out));
  const bool keep_shared = p->n_shared > 0 && o->pre_shared != nullptr;
  if (o->pre != nullptr || keep_shared) {
    if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const long long gu = p->act == MOE_ACT_SWIGLU ? 2 : 1;
    // the tiles address their fp32 rows through 32-bit buffer sizes
    long long ldp = gu * p->d_ff;
    if (gu * p->n_shared * (long long)p->d_ff_shared > ldp) ldp = gu * p->n_shared * (long long)p->d_ff_shared;
    if (320LL * ldp * 4 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(maybe(o->pre, 16));
    if (keep_shared) MOE_TRY(need(o->pre_shared, 16));
  }
  return MOE_OK;
}

// The four stages of the layer on stream s, scratch in ws (layout w).
int launch_layer(const moe_problem_t* p, const void* u, const float* noise,
                 const moe_weights_t* wt, moe_layer_outputs_t* o, void* out, void* ws,
                 const Workspace& w, hipStream_t s) {
  hipError_t e = moe::launch_route(*p, u, wt->w_router, wt->b_router, noise, o->scores,
                                   o->topk_idx, o->topk_gate, o->mean_prob, o->lse_sq,
                                   reinterpret_cast<float*>(ws_at(ws, w.route_part)),
                                   w.route_blocks, reinterpret_cast<float*>(ws_at(ws, w.route_pre)),
                                   s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int32_t C = moe_capacity(p->T, p->K, p->N, p->capacity_factor);
  e = moe::launch_dispatch(*p, u, o->topk_idx, C, o->expert_counts, o->kept_counts, o->offsets,
                           o->row_of, o->token_of_row, o->x_perm,
                           reinterpret_cast<int32_t*>(ws_at(ws, w.disp_count)),
                           reinterpret_cast<int32_t*>(ws_at(ws, w.disp_base)),
                           reinterpret_cast<int32_t*>(ws_at(ws, w.disp_q)), w.disp_blocks, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  void* ysh = p->n_shared > 0 ? o->y_shared : nullptr;
  e = moe::launch_grouped_ffn(*p, p->T * p->K, o->x_perm, o->offsets, wt->w_gate, wt->w_up, wt->w_down, u,
                              wt->ws_gate, wt->ws_up, wt->ws_down, o->y_perm, ysh,
                              reinterpret_cast<int32_t*>(ws_at(ws, w.tiles)), ws_at(ws, w.act),
                              ws_at(ws, w.act_shared),
                              w.has_split ? reinterpret_cast<float*>(ws_at(ws, w.split)) : nullptr, s,
                              o->pre, p->n_shared > 0 ? o->pre_shared : nullptr);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_combine(*p, u, o->y_perm, o->row_of, o->topk_gate, ysh, out, s);
  return hip_status(e);
}

// ------------------------------------------- allocation-free layer forward
// Scratch memory of moe_layer_forward_noalloc: a file-scope device array,
// one copy per GPU, held from module load until the process ends.  In host
// code `scratch` names only a host-side handle of the symbol; its device
// address on each GPU comes from hipGetSymbolAddress with that GPU current,
// looked up once per device and kept in scratch_dev.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's scratch array, for a launch on stream
// s (which must belong to the current GPU).
int scratch_for(hipStream_t s, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if (sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return MOE_ERR_HIP;
    scratch_dev[dev] = a;
  }
  *ptr = scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward(const moe_problem_t* p, const void* u, const float* noise,
                      const moe_weights_t* wt, moe_layer_outputs_t* o, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_layer(p, u, noise, wt, o, out));
  const Workspace w = moe::workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.total));
  return launch_layer(p, u, noise, wt, o, out, ws, w, static_cast<hipStream_t>(stream));
}

int moe_layer_forward_noalloc(const moe_problem_t* p, const void* u, const float* noise,
                              const moe_weights_t* wt, moe_layer_outputs_t* o, void* out,
                              void* stream) {
  MOE_TRY(check_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_layer(p, u, noise, wt, o, out));
  const Workspace w = moe::workspace_layout(*p);
  if (w.total > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  MOE_TRY(scratch_for(s, &ws));
  return launch_layer(p, u, noise, wt, o, out, ws, w, s);
}

// ------------------------------------------------------------ backward

namespace {

// backward-specific limits: bf16 only; every operand a buffer descriptor
// addresses (a group's rows of the widest row-major operand) under 4 GB
int check_backward_problem(const moe_problem_t* p) {
  MOE_TRY(check_problem(p));
  if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  long long ld = p->d;
  const long long gu = p->act == MOE_ACT_SWIGLU ? 2 : 1;
  if (gu * p->d_ff > ld) ld = gu * p->d_ff;
  if (gu * p->n_shared * (long long)p->d_ff_shared > ld) ld = gu * p->n_shared * (long long)p->d_ff_shared;
  if ((long long)p->T * ld * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

size_t moe_backward_workspace_size(const moe_problem_t* p) {
  if (check_backward_problem(p) != MOE_OK || p->T == 0) return 0;
  return moe::bwd_workspace_layout(*p).total;
}

int moe_layer_backward(const moe_problem_t* p, const void* u, const moe_weights_t* w,
                       const moe_saved_t* sv, const void* d_out, moe_grads_t* g, void* ws,
                       size_t ws_bytes, void* stream) {
  MOE_TRY(check_backward_problem(p));
  if (p->T == 0) return MOE_OK;
  if (w == nullptr || sv == nullptr || g == nullptr) return MOE_ERR_INVALID_ARG;
  const bool swiglu = p->act == MOE_ACT_SWIGLU;
  const bool shared = p->n_shared > 0;
  MOE_TRY(need(u, 16));
  MOE_TRY(need(d_out, 16));
  MOE_TRY(need(w->w_router, 16));
  MOE_TRY(need(w->w_gate, 16));
  MOE_TRY(need(w->w_down, 16));
  if (swiglu) MOE_TRY(need(w->w_up, 16));
  if (p->gating == MOE_GATE_SOFTMAX_TOPK) MOE_TRY(need(sv->scores, 4));
  else MOE_TRY(maybe(sv->scores, 4));
  MOE_TRY(need(sv->topk_idx, 4));
  MOE_TRY(need(sv->topk_gate, 4));
  MOE_TRY(need(sv->row_of, 4));
  MOE_TRY(need(sv->offsets, 4));
  MOE_TRY(need(sv->x_perm, 16));
  MOE_TRY(need(sv->y_perm, 16));
  MOE_TRY(need(g->du, 16));
  MOE_TRY(need(g->dw_router, 4));
  MOE_TRY(maybe(g->db_router, 4));
  MOE_TRY(need(g->dw_gate, 16));
  MOE_TRY(need(g->dw_down, 16));
  if (swiglu) MOE_TRY(need(g->dw_up, 16));
  if (shared) {
    MOE_TRY(need(w->ws_gate, 16));
    MOE_TRY(need(w->ws_down, 16));
    MOE_TRY(need(g->dws_gate, 16));
    MOE_TRY(need(g->dws_down, 16));
    if (swiglu) {
      MOE_TRY(need(w->ws_up, 16));
      MOE_TRY(need(g->dws_up, 16));
    }
  }
  MOE_TRY(maybe(g->d_gate, 4));
  MOE_TRY(maybe(g->d_scores, 4));
  MOE_TRY(maybe(g->dy_perm, 16));
  MOE_TRY(maybe(g->dx_perm, 16));
  MOE_TRY(maybe(sv->pre, 16));
  if (shared) MOE_TRY(maybe(sv->pre_shared, 16));
  const moe::BwdWorkspace L = moe::bwd_workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, L.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* d_gate = g->d_gate ? g->d_gate : reinterpret_cast<float*>(ws_at(ws, L.d_gate));
  float* dH = g->d_scores ? g->d_scores : reinterpret_cast<float*>(ws_at(ws, L.dH));
  void* dy = g->dy_perm ? g->dy_perm : ws_at(ws, L.dy_perm);
  void* dx = g->dx_perm ? g->dx_perm : ws_at(ws, L.dx_perm);

  hipError_t e = moe::launch_combine_backward(*p, d_out, sv->y_perm, sv->row_of, sv->topk_gate,
                                               dy, d_gate, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_route_backward(*p, sv->scores, sv->topk_idx, sv->topk_gate, d_gate, dH, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_router_param_grads(*p, u, dH, reinterpret_cast<float*>(ws_at(ws, L.partial)),
                                     g->dw_router, g->db_router, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::FfnBwdBuffers b{};
  b.offsets = sv->offsets;
  b.x_perm = sv->x_perm;
  b.dy_perm = dy;
  b.w_gate = w->w_gate;
  b.w_up = w->w_up;
  b.w_down = w->w_down;
  b.tiles = reinterpret_cast<int32_t*>(ws_at(ws, L.tiles));
  b.dA = ws_at(ws, L.dA);
  b.act = ws_at(ws, L.act);
  b.dgu = ws_at(ws, L.dgu);
  b.dx_perm = dx;
  b.dw_gate = g->dw_gate;
  b.dw_up = g->dw_up;
  b.dw_down = g->dw_down;
  b.pre = sv->pre;
  b.pre_shared = shared ? sv->pre_shared : nullptr;
  if (L.ldt > 0) {
    b.kpad = reinterpret_cast<int32_t*>(ws_at(ws, L.kpad));
    b.dyT = ws_at(ws, L.dyT);
    b.xT = ws_at(ws, L.xT);
    b.ldt = L.ldt;
    if (L.ldts > 0) {
      b.dOT = ws_at(ws, L.dOT);
      b.uT = ws_at(ws, L.uT);
      b.ldts = L.ldts;
    }
  }
  if (shared) {
    b.u = u;
    b.d_out = d_out;
    b.ws_gate = w->ws_gate;
    b.ws_up = w->ws_up;
    b.ws_down = w->ws_down;
    b.dA_s = ws_at(ws, L.dA_s);
    b.act_s = ws_at(ws, L.act_s);
    b.dgu_s = ws_at(ws, L.dgu_s);
    b.dx_shared = ws_at(ws, L.dx_shared);
    b.dws_gate = g->dws_gate;
    b.dws_up = g->dws_up;
    b.dws_down = g->dws_down;
  }
  e = moe::launch_grouped_ffn_backward(*p, p->T * p->K, b, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_du(*p, dH, w->w_router, d_out, dx, sv->row_of,
                                   shared ? b.dx_shared : nullptr, g->du, s));
}

// ------------------------------------------------------------ expert choice

int32_t moe_ec_capacity(int32_t T, int32_t K, int32_t N, float cf) {
  if (N <= 0 || T < 0 || K < 0) return -1;
  return moe::ec_capacity_of(T, K, N, cf);
}

size_t moe_ec_workspace_size(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK || p->T == 0) return 0;
  return moe::ec_workspace_layout(*p).total;
}

namespace {

int check_ec_problem(const moe_problem_t* p) {
  MOE_TRY(check_problem(p));
  const int64_t C = moe::ec_capacity_of(p->T, p->K, p->N, p->capacity_factor);
  if ((int64_t)p->N * C > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_ec_route(const moe_problem_t* p, const void* u, const float* w_router,
                   const float* b_router, const float* noise, const float* scores,
                   const float* probs, const int32_t* expert_tokens, const float* expert_gates,
                   const int32_t* row_of, const float* gate_of, const int32_t* offsets,
                   const float* mean_prob, const float* lse_sq) {
  MOE_TRY(need(u, 16));
  MOE_TRY(need(w_router, 16));
  MOE_TRY(maybe(b_router, 4));
  MOE_TRY(maybe(noise, 4));
  MOE_TRY(maybe(scores, 4));
  MOE_TRY(need(probs, 4));
  MOE_TRY(need(expert_tokens, 4));
  MOE_TRY(need(expert_gates, 4));
  MOE_TRY(need(row_of, 4));
  MOE_TRY(need(gate_of, 4));
  MOE_TRY(need(offsets, 4));
  MOE_TRY(need(mean_prob, 4));
  MOE_TRY(need(lse_sq, 4));
  if (noise != nullptr && !isfinite(p->noise_weight)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

hipError_t ec_route_launch(const moe_problem_t* p, const void* u, const float* w_router,
                           const float* b_router, const float* noise, float* scores,
                           float* probs, int32_t* expert_tokens, float* expert_gates,
                           int32_t* row_of, float* gate_of, int32_t* offsets, float* mean_prob,
                           float* lse_sq, void* ws, const EcWorkspace& w, hipStream_t s) {
  float* sc = scores != nullptr ? scores : reinterpret_cast<float*>(ws_at(ws, w.scores));
  hipError_t e = moe::launch_route(*p, u, w_router, b_router, noise, sc,
                                   reinterpret_cast<int32_t*>(ws_at(ws, w.tk_idx)),
                                   reinterpret_cast<float*>(ws_at(ws, w.tk_gate)), mean_prob,
                                   lse_sq, reinterpret_cast<float*>(ws_at(ws, w.route_part)),
                                   w.route_blocks, reinterpret_cast<float*>(ws_at(ws, w.route_pre)),
                                   s);
  if (e != hipSuccess) return e;
  return moe::launch_ec_select(*p, sc, w.C, probs, expert_tokens, expert_gates, row_of, gate_of,
                               offsets, ws_at(ws, w.sel), s);
}

}  // namespace

int moe_ec_route(const moe_problem_t* p, const void* u, const float* w_router,
                 const float* b_router, const float* noise, float* scores, float* probs,
                 int32_t* expert_tokens, float* expert_gates, int32_t* row_of, float* gate_of,
                 int32_t* offsets, float* mean_prob, float* lse_sq, void* ws, size_t ws_bytes,
                 void* stream) {
  MOE_TRY(check_ec_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(check_ec_route(p, u, w_router, b_router, noise, scores, probs, expert_tokens,
                         expert_gates, row_of, gate_of, offsets, mean_prob, lse_sq));
  const EcWorkspace w = moe::ec_workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.tiles));
  return hip_status(ec_route_launch(p, u, w_router, b_router, noise, scores, probs,
                                    expert_tokens, expert_gates, row_of, gate_of, offsets,
                                    mean_prob, lse_sq, ws, w, static_cast<hipStream_t>(stream)));
}

int moe_ec_dispatch(const moe_problem_t* p, const void* u, const int32_t* expert_tokens,
                    void* x_perm, void* stream) {
  MOE_TRY(check_ec_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(need(u, 16));
  MOE_TRY(need(expert_tokens, 4));
  MOE_TRY(need(x_perm, 16));
  const int32_t C = moe::ec_capacity_of(p->T, p->K, p->N, p->capacity_factor);
  return hip_status(moe::launch_ec_gather(*p, u, expert_tokens, p->N * C, x_perm,
                                          static_cast<hipStream_t>(stream)));
}

int moe_ec_combine(const moe_problem_t* p, const void* u, const void* y_perm,
                   const int32_t* row_of, const float* gate_of, const void* y_shared, void* out,
                   void* stream) {
  MOE_TRY(check_ec_problem(p));
  if (p->T == 0) return MOE_OK;
  MOE_TRY(need(u, 16));
  MOE_TRY(need(y_perm, 16));
  MOE_TRY(need(row_of, 4));
  MOE_TRY(need(gate_of, 4));
  MOE_TRY(need(out, 16));
  if (p->n_shared > 0) MOE_TRY(need(y_shared, 16));
  return hip_status(moe::launch_ec_combine(*p, u, y_perm, row_of, gate_of,
                                           p->n_shared > 0 ? y_shared : nullptr, out,
                                           static_cast<hipStream_t>(stream)));
}

int moe_ec_layer_forward(const moe_problem_t* p, const void* u, const float* noise,
                         const moe_weights_t* wt, moe_ec_outputs_t* o, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
  MOE_TRY(check_ec_problem(p));
  if (p->T == 0) return MOE_OK;
  if (wt == nullptr || o == nullptr) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ec_route(p, u, wt->w_router, wt->b_router, noise, o->scores, o->probs,
                         o->expert_tokens, o->expert_gates, o->row_of, o->gate_of, o->offsets,
                         o->mean_prob, o->lse_sq));
  MOE_TRY(check_ffn(p, o->x_perm, o->offsets, wt->w_gate, wt->w_up, wt->w_down, u, wt->ws_gate,
                    wt->ws_up, wt->ws_down, o->y_perm, o->y_shared));
  MOE_TRY(need(out, 16));
  const EcWorkspace w = moe::ec_workspace_layout(*p);
  MOE_TRY(check_ws(ws, ws_bytes, w.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = ec_route_launch(p, u, wt->w_router, wt->b_router, noise, o->scores, o->probs,
                                 o->expert_tokens, o->expert_gates, o->row_of, o->gate_of,
                                 o->offsets, o->mean_prob, o->lse_sq, ws, w, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int rows = p->N * w.C;
  e = moe::launch_ec_gather(*p, u, o->expert_tokens, rows, o->x_perm, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  void* ysh = p->n_shared > 0 ? o->y_shared : nullptr;
  e = moe::launch_grouped_ffn(*p, rows, o->x_perm, o->offsets, wt->w_gate, wt->w_up, wt->w_down,
                              u, wt->ws_gate, wt->ws_up, wt->ws_down, o->y_perm, ysh,
                              reinterpret_cast<int32_t*>(ws_at(ws, w.tiles)), ws_at(ws, w.act),
                              ws_at(ws, w.act_shared), nullptr, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_ec_combine(*p, u, o->y_perm, o->row_of, o->gate_of, ysh, out, s));
}

}  // extern "C"
