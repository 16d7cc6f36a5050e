// Stage 2 -- dispatch: per-expert histogram, capacity, prefix sum and a
// stable permutation of token rows into expert-contiguous rows.
//
// "MoE: Choosing Which MLPs to Use for Each Token", "From Router to Combine"
// (Figure 3): dispatch groups the original token vectors by expert; a token
// with K experts appears in K groups.  Capacity ("Mixture of Experts (MoE)"
// glossary, expert-capacity entry; "Switch Transformers explained", "Making
// it work"): past an expert's capacity, tokens are dropped and keep only the
// residual.  First come, first served in ascending token order.
//
// Stable ranks without ordering races: each block owns 256 tokens and builds,
// per expert, a 256-bit LDS mask of the tokens that chose it (atomicOr sets
// bits, so the mask does not depend on thread timing).  A token's rank inside
// the block is the popcount of the mask bits below it; block bases come from
// a fixed-order scan.  No floating point, no order-dependent atomics: the
// maps are bit-identical run to run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTok = kDispatchTok;     // tokens per block (one per thread)
constexpr int kWords = kTok / 32;

// build masks[N][kWords] for tokens [blk*kTok, +kTok)
__device__ __forceinline__ void build_masks(uint32_t* mask, const int32_t* topk_idx, int T,
                                            int N, int K, int t_local, int t) {
  for (int i = threadIdx.x; i < N * kWords; i += kTok) mask[i] = 0u;
  __syncthreads();
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[(size_t)t * K + k];
      if (e >= 0 && e < N) atomicOr(&mask[e * kWords + (t_local >> 5)], 1u << (t_local & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTok) void dispatch_count_kernel(const int32_t* topk_idx, int T,
                                                              int N, int K, int32_t* blk_count) {
  __shared__ uint32_t mask[256 * kWords];
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kTok + tl;
  build_masks(mask, topk_idx, T, N, K, tl, t);
  for (int e = tl; e < N; e += kTok) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popc(mask[e * kWords + w]);
    blk_count[(size_t)blockIdx.x * N + e] = c;
  }
}

// One block: per-expert running sums over blocks in block order, capacity,
// then the exclusive scan over experts.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(const int32_t* blk_count,
                                                            int32_t* blk_base, int blocks, int N,
                                                            int32_t capacity,
                                                            int32_t* expert_counts,
                                                            int32_t* kept_counts,
                                                            int32_t* offsets) {
  __shared__ int32_t s[256];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < N) {
    // 16 block counts in flight at a time, then their running sums
    constexpr int kChunk = 16;
    int run = 0;
    for (int b0 = 0; b0 < blocks; b0 += kChunk) {
      int c[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        c[i] = b0 + i < blocks ? blk_count[(size_t)(b0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (b0 + i < blocks) blk_base[(size_t)(b0 + i) * N + e] = run;
        run += c[i];
      }
    }
    expert_counts[e] = run;
    kept = (capacity >= 0 && run > capacity) ? capacity : run;
    kept_counts[e] = kept;
  }
  s[e] = kept;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < N) offsets[e + 1] = s[e];
  if (e == 0) offsets[0] = 0;
}

// Ranks, maps and the row copy in one pass.  Block b owns kRowTok tokens
// inside one 256-token mask chunk; it rebuilds that chunk's masks (the same
// bits as dispatch_count_kernel's), computes the rows of its tokens, writes
// row_of and token_of_row, then copies each token row (read once, 16-byte
// vectors) to every kept row.
constexpr int kRowTok = 16;                 // tokens per block
constexpr int kVecPerLane = 8;              // 16-byte vectors in flight per lane
static_assert(kTok % kRowTok == 0, "blocks tile the mask chunks");

__global__ __launch_bounds__(256) void dispatch_permute_kernel(
    const int32_t* topk_idx, const int32_t* blk_base, const int32_t* offsets, int T, int N, int K,
    int32_t capacity, int32_t* row_of, int32_t* token_of_row, const u32x4* u, u32x4* x_perm,
    int vec_per_row) {
  __shared__ uint32_t mask[256 * kWords];
  __shared__ int32_t srow[kRowTok * 16];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRowTok;           // first token of this block
  const int chunk = t0 / kTok;
  build_masks(mask, topk_idx, T, N, K, tid, chunk * kTok + tid);
  if (tid < kRowTok) {
    const int t = t0 + tid;
    if (t < T) {
      const int tl = t - chunk * kTok;
      const int w0 = tl >> 5;
      const uint32_t below = (1u << (tl & 31)) - 1u;
      for (int k = 0; k < K; ++k) {
        const int e = topk_idx[(size_t)t * K + k];
        int32_t row = -1;
        if (e >= 0 && e < N) {
          int r = __popc(mask[e * kWords + w0] & below);
          for (int w = 0; w < w0; ++w) r += __popc(mask[e * kWords + w]);
          const int rank = blk_base[(size_t)chunk * N + e] + r;
          if (capacity < 0 || rank < capacity) {
            row = offsets[e] + rank;
            token_of_row[row] = t;
          }
        }
        row_of[(size_t)t * K + k] = row;
        srow[tid * 16 + k] = row;
      }
    }
  }
  // rows past the kept total hold no token
  const int64_t total = (int64_t)T * K;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t r = offsets[N] + (int64_t)blockIdx.x * 256 + tid; r < total; r += stride)
    token_of_row[r] = -1;
  __syncthreads();

  // copy: wave w takes tokens w, w+4, ... of the block
  const int lane = tid & 63;
  for (int j = tid >> 6; j < kRowTok; j += 4) {
    const int t = t0 + j;
    if (t >= T) break;
    const u32x4* src = u + (size_t)t * vec_per_row;
    for (int v0 = 0; v0 < vec_per_row; v0 += 64 * kVecPerLane) {
      u32x4 q[kVecPerLane];
#pragma unroll
      for (int i = 0; i < kVecPerLane; ++i) {
        const int v = v0 + i * 64 + lane;
        if (v < vec_per_row) q[i] = src[v];
      }
      for (int k = 0; k < K; ++k) {
        const int row = srow[j * 16 + k];
        if (row < 0) continue;
        u32x4* dst = x_perm + (size_t)row * vec_per_row;
#pragma unroll
        for (int i = 0; i < kVecPerLane; ++i) {
          const int v = v0 + i * 64 + lane;
          if (v < vec_per_row) dst[v] = q[i];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_dispatch(const moe_problem_t& p, const void* u, const int32_t* topk_idx,
                           int32_t capacity, int32_t* expert_counts, int32_t* kept_counts,
                           int32_t* offsets, int32_t* row_of, int32_t* token_of_row,
                           void* x_perm, int32_t* blk_count, int32_t* blk_base,
                           int disp_blocks, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(disp_blocks), dim3(kTok), 0, s, topk_idx, p.T,
                     p.N, p.K, blk_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, s, (const int32_t*)blk_count,
                     blk_base, disp_blocks, p.N, capacity, expert_counts, kept_counts, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = (int)((size_t)p.d * es / 16);
  const unsigned blocks = (unsigned)((p.T + kRowTok - 1) / kRowTok);
  hipLaunchKernelGGL(dispatch_permute_kernel, dim3(blocks), dim3(256), 0, s, topk_idx,
                     (const int32_t*)blk_base, (const int32_t*)offsets, p.T, p.N, p.K, capacity,
                     row_of, token_of_row, static_cast<const u32x4*>(u),
                     static_cast<u32x4*>(x_perm), vec_per_row);
  return hipGetLastError();
}

}  // namespace moe
