// Internal declarations shared by the libmoe translation units (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
// bf16 is the upper half of an IEEE binary32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return static_cast<uint16_t>(x >> 16);
}

// Row buffers of the grouped FFN (x_perm, y_perm) larger than this many
// bytes do not stay in the 256 MB Infinity Cache between the stage that
// writes them and the one that reads them: dispatch stores x_perm and
// combine loads y_perm with non-temporal accesses, which stream them
// without evicting what the cache still holds.  Below it the cache serves
// the reads.
constexpr size_t kStreamRowsBytes = (size_t)192 << 20;

// ------------------------------------------------------------- layout
constexpr size_t kAlign = 256;
__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Router launch shape: each block owns `tok` tokens (16, 32 or 64).
int route_tokens_per_block(const moe_problem_t& p);
// Few-token batches: d-slices of the split-k logits (0: fused path) and the
// workspace they need ([slices][T][N] fp32).
int route_pre_splits(const moe_problem_t& p);
size_t route_pre_bytes(const moe_problem_t& p);
constexpr int kDispatchTok = 256;   // tokens per dispatch block

// Grouped-GEMM plan: full- and tail-tile prefixes ([2][N+2] int32), then
// the work-queue counters of the persistent GEMM launches (kQueueSets sets
// of kQueueInts, zeroed by the plan kernel before each grouped FFN).
constexpr int kQueueInts = 16;
constexpr int kQueueSets = 4;
// Split-K of the persistent plain GEMM's tail tiles: at most kSplitSlots
// pieces, each with 64 KB of fp32 partial sums, and one counter per tail
// tile (after the queue counters, zeroed with them).
constexpr int kSplitSlots = 256;
constexpr size_t kSplitBytes = (size_t)kSplitSlots * 64 * 256 * 4;
inline size_t gemm_plan_bytes(size_t N) {
  return (2 * (N + 2) + kQueueSets * kQueueInts + kSplitSlots) * 4;
}

struct Workspace {
  size_t route_part;   // fp32 [route_blocks][N]   per-block softmax sums
  size_t route_pre;    // fp32 [slices][T][N]       split-k logits (few tokens)
  size_t disp_count;   // int32 [disp_blocks][K][N]  per-block expert counts (per choice rank)
  size_t disp_base;    // int32 [disp_blocks][K][N]  per-block rank base
  size_t disp_q;       // int32 [K][N]               kept per choice rank
  size_t tiles;        // int32 gemm_plan_bytes(N)  grouped-GEMM tile prefixes, queue counters
  size_t act;          // elem [T*K][d_ff]        gated activations
  size_t act_shared;   // elem [T][n_shared*d_ff_shared]
  size_t split;        // fp32 kSplitBytes: split-K partial sums of the persistent
                       // down GEMMs' tail tiles (only when a 256-row GEMM runs)
  bool has_split;
  size_t total;
  int route_blocks;
  int disp_blocks;
};
Workspace workspace_layout(const moe_problem_t& p);

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments are pre-validated.
hipError_t launch_route(const moe_problem_t& p, const void* u, const float* w_router,
                        const float* b_router, const float* noise, float* scores,
                        int32_t* topk_idx, float* topk_gate, float* mean_prob,
                        float* lse_sq, float* part, int route_blocks, float* pre,
                        hipStream_t s);

hipError_t launch_router_stats(const moe_problem_t& p, const int32_t* expert_counts,
                               const float* mean_prob, const float* lse_sq, float* stats,
                               hipStream_t s);

hipError_t launch_dispatch(const moe_problem_t& p, const void* u, const int32_t* topk_idx,
                           int32_t capacity, int32_t* expert_counts, int32_t* kept_counts,
                           int32_t* offsets, int32_t* row_of, int32_t* token_of_row,
                           void* x_perm, int32_t* blk_count, int32_t* blk_base,
                           int32_t* level_q, int disp_blocks, hipStream_t s);

// Row-tile height of the grouped GEMMs over `rows` rows in `groups` groups
// (the mean group size picks the kernel family).
int ffn_row_tile(int rows, int groups, bool bf16);

// rows_alloc: rows of x_perm / y_perm / act (T*K for token choice).
hipError_t launch_grouped_ffn(const moe_problem_t& p, int rows_alloc, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, const void* u, const void* ws_gate,
                              const void* ws_up, const void* ws_down, void* y_perm,
                              void* y_shared, int32_t* tiles, void* act, void* act_shared,
                              float* split, hipStream_t s, float* pre = nullptr,
                              float* pre_shared = nullptr);

hipError_t launch_combine(const moe_problem_t& p, const void* u, const void* y_perm,
                          const int32_t* row_of, const float* topk_gate,
                          const void* y_shared, void* out, hipStream_t s);

// backward of the expert FFNs (grouped_gemm.hip); every pointer is device
// memory, elem typed unless noted, shapes per the layer's problem
struct FfnBwdBuffers {
  const int32_t* offsets;   // [N+1] expert row offsets of the forward
  const void* x_perm;       // [rows][d]     forward rows
  const void* dy_perm;      // [rows][d]     gradients of the expert outputs
  const void *w_gate, *w_up, *w_down;
  int32_t* tiles;           // [2][N+2] workspace
  void* dA;                 // [rows][d_ff]  workspace
  void* act;                // [rows][d_ff]  workspace
  void* dgu;                // [rows][2*d_ff] workspace (ReLU: [rows][d_ff])
  void* dx_perm;            // [rows][d]     gradients of the rows
  void *dw_gate, *dw_up, *dw_down;
  // weight gradients in transposed form (null kpad: the direct k-major kernel)
  int32_t* kpad;            // [N+1] workspace
  void* dyT;                // [d][ldt] workspace
  void* xT;                 // [d][ldt] workspace
  int ldt;
  // shared experts' weight gradients in the same launches (null dOT: by the
  // direct kernel): d_out and u transposed, [d][ldts] workspace each
  void* dOT;
  void* uT;
  int ldts;
  // shared experts (n_shared > 0)
  const void* u;            // [T][d]
  const void* d_out;        // [T][d]
  const void *ws_gate, *ws_up, *ws_down;
  void* dA_s;               // [T][n_shared*d_ff_shared] workspace
  void* act_s;              // [T][n_shared*d_ff_shared] workspace
  void* dgu_s;              // [T][2*n_shared*d_ff_shared] workspace
  void* dx_shared;          // [T][d]
  void *dws_gate, *dws_up, *dws_down;
  // the forward's fp32 pre-activations (null: recomputed by GEMM-1)
  const float* pre;         // [rows][gu*d_ff]
  const float* pre_shared;  // [T][gu*n_shared*d_ff_shared]
};
hipError_t launch_grouped_ffn_backward(const moe_problem_t& p, int rows_alloc,
                                       const FfnBwdBuffers& b, hipStream_t s);

// backward, apart from the expert GEMMs (backward.hip)
int router_grad_slices(int T, int N);
hipError_t launch_combine_backward(const moe_problem_t& p, const void* d_out, const void* y_perm,
                                   const int32_t* row_of, const float* gate, void* dy_perm,
                                   float* d_gate, hipStream_t s);
hipError_t launch_route_backward(const moe_problem_t& p, const float* scores,
                                 const int32_t* topk_idx, const float* gate, const float* d_gate,
                                 float* dH, hipStream_t s);
hipError_t launch_router_param_grads(const moe_problem_t& p, const void* u, const float* dH,
                                     float* partial, float* dw_router, float* db_router,
                                     hipStream_t s);
hipError_t launch_du(const moe_problem_t& p, const float* dH, const float* w_router,
                     const void* d_out, const void* dx_perm, const int32_t* row_of,
                     const void* dx_shared, void* du, hipStream_t s);

struct BwdWorkspace {
  size_t tiles;        // int32 [2][N+2]
  size_t dy_perm;      // elem [T*K][d]
  size_t dA;           // elem [T*K][d_ff]
  size_t act;          // elem [T*K][d_ff]
  size_t dgu;          // elem [T*K][2*d_ff] (ReLU: d_ff)
  size_t dx_perm;      // elem [T*K][d]
  size_t d_gate;       // fp32 [T][K]
  size_t dH;           // fp32 [T][N]
  size_t partial;      // fp32 [slices][N][d+1]
  size_t dA_s, act_s;  // elem [T][n_shared*d_ff_shared]
  size_t dgu_s;        // elem [T][2*n_shared*d_ff_shared]
  size_t dx_shared;    // elem [T][d]
  size_t kpad;         // int32 [N+1]         (transposed weight gradients only)
  size_t dyT;          // elem [d][ldt]
  size_t xT;           // elem [d][ldt]
  int ldt;             // 0: weight gradients by the direct k-major kernel
  size_t dOT, uT;      // elem [d][ldts] (transposed form with shared experts)
  int ldts;            // 0: shared experts' weight gradients by the direct kernel
  size_t total;
};
BwdWorkspace bwd_workspace_layout(const moe_problem_t& p);
// Leading dimension of the transposed weight-gradient operands (rows padded
// per expert to a multiple of 64), or 0 when the experts' groups are too
// short on average for the transposed form to pay.
int wgrad_transposed_ld(const moe_problem_t& p);

// expert choice (expert_choice.hip)
// 64-token words of the per-expert selection masks; sel holds
// uint64 [N][words] masks then int32 [N][words] chosen-before counts
inline int ec_select_words(int T) { return (T + 63) / 64; }
inline size_t ec_select_bytes(int T, int N) { return (size_t)N * ec_select_words(T) * 12; }
hipError_t launch_ec_select(const moe_problem_t& p, const float* scores, int32_t C,
                            float* probsT, int32_t* expert_tokens, float* expert_gates,
                            int32_t* row_of, float* gate_of, int32_t* offsets, void* sel,
                            hipStream_t s);
hipError_t launch_ec_gather(const moe_problem_t& p, const void* u, const int32_t* tokens,
                            int rows, void* x_perm, hipStream_t s);
hipError_t launch_ec_combine(const moe_problem_t& p, const void* u, const void* y_perm,
                             const int32_t* row_of, const float* gate_of, const void* y_shared,
                             void* out, hipStream_t s);

struct EcWorkspace {
  size_t route_part;   // fp32 [route_blocks][N]
  size_t route_pre;    // fp32 [slices][T][N]
  size_t scores;       // fp32 [T][N]      router scores when the caller keeps none
  size_t tk_idx;       // int32 [T][K]     token-choice top-K of the router (unused)
  size_t tk_gate;      // fp32 [T][K]
  size_t sel;          // selection masks and counts (ec_select_bytes)
  size_t tiles;        // int32 [2][N+2]
  size_t act;          // elem [N*C][d_ff]
  size_t act_shared;   // elem [T][n_shared*d_ff_shared]
  size_t total;
  int route_blocks;
  int C;
};
EcWorkspace ec_workspace_layout(const moe_problem_t& p);

}  // namespace moe
