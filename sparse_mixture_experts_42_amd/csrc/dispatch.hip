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
//
// SCAN: when all chunk counts fit in LDS (chunks x N <= kScanInBlock), every
// block runs the scan itself on the chunk counts -- the per-expert running
// sums over the chunks before its own, the capacity and the expert offsets
// (the same fixed-order integer sums as dispatch_scan_kernel) -- and block 0
// writes expert_counts, kept_counts and offsets.  That saves a launch of the
// one-block scan kernel, whose cost is mostly launch latency.  Otherwise the
// scan kernel has written blk_base and offsets.
constexpr int kRowTok = 16;                 // tokens per block
constexpr int kVecPerLane = 8;              // 16-byte vectors in flight per lane
constexpr int kScanInBlock = 4096;          // chunk counts one block scans itself (16 KB)
static_assert(kTok % kRowTok == 0, "blocks tile the mask chunks");

// Copy each token row of the block (read once, 16-byte vectors, kVecPerLane
// per lane in flight) to every kept row srow[j*16 + k]; wave w takes tokens
// w, w+4, ... of the block.
template <bool NT>
__device__ __forceinline__ void copy_rows(int t0, int T, int K, const int32_t* srow,
                                          const u32x4* u, u32x4* x_perm, int vec_per_row) {
  const int lane = threadIdx.x & 63;
  for (int j = threadIdx.x >> 6; j < kRowTok; j += 4) {
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
          if (v >= vec_per_row) continue;
          if constexpr (NT) __builtin_nontemporal_store(q[i], &dst[v]);
          else dst[v] = q[i];
        }
      }
    }
  }
}

template <bool SCAN, bool NT>
__global__ __launch_bounds__(256) void dispatch_permute_kernel(
    const int32_t* topk_idx, const int32_t* blk_count, int chunks, const int32_t* blk_base,
    int32_t* offsets, int32_t* expert_counts, int32_t* kept_counts, int T, int N, int K,
    int32_t capacity, int32_t* row_of, int32_t* token_of_row, const u32x4* u, u32x4* x_perm,
    int vec_per_row) {
  __shared__ uint32_t mask[256 * kWords];
  __shared__ int32_t srow[kRowTok * 16];
  __shared__ int32_t s_cnt[SCAN ? kScanInBlock : 1];
  __shared__ int32_t s_base[SCAN ? 256 : 1];
  __shared__ int32_t s_off[SCAN ? 257 : 1];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRowTok;           // first token of this block
  const int chunk = t0 / kTok;
  if constexpr (SCAN) {
    for (int i = tid; i < chunks * N; i += 256) s_cnt[i] = blk_count[i];
    __syncthreads();
    int kept = 0;
    if (tid < N) {
      int run = 0, mine = 0;
      for (int c = 0; c < chunks; ++c) {
        if (c == chunk) mine = run;
        run += s_cnt[c * N + tid];
      }
      s_base[tid] = mine;
      kept = (capacity >= 0 && run > capacity) ? capacity : run;
      if (blockIdx.x == 0) {
        expert_counts[tid] = run;
        kept_counts[tid] = kept;
      }
    }
    // inclusive scan of the kept counts over the experts (s_cnt is free now)
    __syncthreads();
    s_cnt[tid] = kept;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? s_cnt[tid - o] : 0;
      __syncthreads();
      s_cnt[tid] += v;
      __syncthreads();
    }
    if (tid < N) s_off[tid + 1] = s_cnt[tid];
    if (tid == 0) s_off[0] = 0;
    __syncthreads();
    if (blockIdx.x == 0) {
      if (tid < N) offsets[tid] = s_off[tid];
      if (tid == 0) offsets[N] = s_off[N];      // N may be 256: past the last thread
    }
  }
  auto base_of = [&](int e) -> int32_t {
    if constexpr (SCAN) return s_base[e];
    else return blk_base[(size_t)chunk * N + e];
  };
  auto off_of = [&](int e) -> int32_t {
    if constexpr (SCAN) return s_off[e];
    else return offsets[e];
  };
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
          const int rank = base_of(e) + r;
          if (capacity < 0 || rank < capacity) {
            row = off_of(e) + rank;
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
  for (int64_t r = off_of(N) + (int64_t)blockIdx.x * 256 + tid; r < total; r += stride)
    token_of_row[r] = -1;
  __syncthreads();

  copy_rows<NT>(t0, T, K, srow, u, x_perm, vec_per_row);
}

// ---------------------------------------------------------------------
// Capacity by choice rank: a full expert keeps the first C of its
// assignments in order of (choice rank k, token), and the kept ones take its
// rows in token order.  With q[k][e] = min(max(C - sum_{k'<k} n[k'][e], 0),
// n[k][e]) kept at level k (n = level-k assignments to e), the kept level-k
// assignments are the first q[k][e] of that level in token order, and the
// row of a kept (t, k) is offsets[e] + sum_k' min(q[k'][e], rank_k'(t, e)),
// rank_k'(t, e) = level-k' assignments to e of tokens before t.  Per-chunk
// level masks give those ranks with the same popcounts as above.

// level-k masks of a chunk: bit t of mask[e] set iff topk_idx[t][k] == e
__device__ __forceinline__ void build_level_mask(uint32_t* mask, const int32_t* topk_idx, int T,
                                                 int N, int K, int k, int t_local, int t) {
  for (int i = threadIdx.x; i < N * kWords; i += kTok) mask[i] = 0u;
  __syncthreads();
  if (t < T) {
    const int e = topk_idx[(size_t)t * K + k];
    if (e >= 0 && e < N) atomicOr(&mask[e * kWords + (t_local >> 5)], 1u << (t_local & 31));
  }
  __syncthreads();
}

// cnt[chunk][k][e]: level-k assignments to e in the chunk
__global__ __launch_bounds__(kTok) void dispatch_count_levels_kernel(const int32_t* topk_idx, int T,
                                                                     int N, int K, int32_t* cnt) {
  __shared__ uint32_t mask[256 * kWords];
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kTok + tl;
  for (int k = 0; k < K; ++k) {
    build_level_mask(mask, topk_idx, T, N, K, k, tl, t);
    for (int e = tl; e < N; e += kTok) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kWords; ++w) c += __popc(mask[e * kWords + w]);
      cnt[((size_t)blockIdx.x * K + k) * N + e] = c;
    }
    __syncthreads();
  }
}

// One block: per (level, expert) running sums over the chunks, the kept
// counts per level q, and the expert offsets.
__global__ __launch_bounds__(256) void dispatch_scan_levels_kernel(
    const int32_t* cnt, int32_t* base, int32_t* q, int chunks, int N, int K, int32_t capacity,
    int32_t* expert_counts, int32_t* kept_counts, int32_t* offsets) {
  __shared__ int32_t tot[16 * 256];
  __shared__ int32_t sc[256];
  const int tid = threadIdx.x;
  for (int pk = tid; pk < K * N; pk += 256) {
    int run = 0;
    for (int c = 0; c < chunks; ++c) {
      const size_t at = (size_t)c * K * N + pk;
      const int v = cnt[at];
      base[at] = run;
      run += v;
    }
    tot[pk] = run;
  }
  __syncthreads();
  int kept = 0;
  if (tid < N) {
    int cum = 0;
    for (int k = 0; k < K; ++k) {
      const int n = tot[k * N + tid];
      int room = capacity - cum;
      room = room < 0 ? 0 : room;
      const int qk = n < room ? n : room;
      q[k * N + tid] = qk;
      kept += qk;
      cum += n;
    }
    expert_counts[tid] = cum;
    kept_counts[tid] = kept;
  }
  sc[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < N) offsets[tid + 1] = sc[tid];
  if (tid == 0) offsets[0] = 0;
}

template <bool NT>
__global__ __launch_bounds__(256) void dispatch_permute_levels_kernel(
    const int32_t* topk_idx, const int32_t* base, const int32_t* q, const int32_t* offsets, int T,
    int N, int K, int32_t* row_of, int32_t* token_of_row, const u32x4* u, u32x4* x_perm,
    int vec_per_row) {
  __shared__ uint32_t mask[256 * kWords];
  __shared__ int32_t srow[kRowTok * 16];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRowTok;
  const int chunk = t0 / kTok;
  const int t = t0 + tid;                       // token of thread tid < kRowTok
  const bool mine = tid < kRowTok && t < T;
  const int tl = mine ? t - chunk * kTok : 0;
  int e_of[16], pos[16];
  bool kept[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    e_of[k] = (mine && k < K) ? topk_idx[(size_t)t * K + k] : 0;
    pos[k] = 0;
    kept[k] = false;
  }
  for (int lvl = 0; lvl < K; ++lvl) {
    build_level_mask(mask, topk_idx, T, N, K, lvl, tid, chunk * kTok + tid);
    if (mine) {
      const int w0 = tl >> 5;
      const uint32_t below = (1u << (tl & 31)) - 1u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k >= K) break;
        const int e = e_of[k];
        if (e < 0 || e >= N) continue;           // no such expert: never kept
        int r = __popc(mask[e * kWords + w0] & below);
        for (int w = 0; w < w0; ++w) r += __popc(mask[e * kWords + w]);
        r += base[((size_t)chunk * K + lvl) * N + e];
        const int qv = q[lvl * N + e];
        pos[k] += r < qv ? r : qv;
        if (k == lvl) kept[k] = r < qv;
      }
    }
    __syncthreads();
  }
  if (mine) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k >= K) break;
      int32_t row = -1;
      if (kept[k]) {
        row = offsets[e_of[k]] + pos[k];
        token_of_row[row] = t;
      }
      row_of[(size_t)t * K + k] = row;
      srow[tid * 16 + k] = row;
    }
  }
  const int64_t total = (int64_t)T * K;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t r = offsets[N] + (int64_t)blockIdx.x * 256 + tid; r < total; r += stride)
    token_of_row[r] = -1;
  __syncthreads();
  copy_rows<NT>(t0, T, K, srow, u, x_perm, vec_per_row);
}

}  // namespace

hipError_t launch_dispatch(const moe_problem_t& p, const void* u, const int32_t* topk_idx,
                           int32_t capacity, int32_t* expert_counts, int32_t* kept_counts,
                           int32_t* offsets, int32_t* row_of, int32_t* token_of_row,
                           void* x_perm, int32_t* blk_count, int32_t* blk_base,
                           int32_t* level_q, int disp_blocks, hipStream_t s) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = (int)((size_t)p.d * es / 16);
  const unsigned blocks = (unsigned)((p.T + kRowTok - 1) / kRowTok);
  const bool nt = (size_t)p.T * p.K * p.d * es > kStreamRowsBytes;
  if (p.drop_order == MOE_DROP_CHOICE_RANK && capacity >= 0 && p.K > 1) {
    // (K = 1 or no capacity: both orders keep the same assignments)
    hipLaunchKernelGGL(dispatch_count_levels_kernel, dim3(disp_blocks), dim3(kTok), 0, s, topk_idx,
                       p.T, p.N, p.K, blk_count);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dispatch_scan_levels_kernel, dim3(1), dim3(256), 0, s,
                       (const int32_t*)blk_count, blk_base, level_q, disp_blocks, p.N, p.K,
                       capacity, expert_counts, kept_counts, offsets);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nt)
      hipLaunchKernelGGL(dispatch_permute_levels_kernel<true>, dim3(blocks), dim3(256), 0, s, topk_idx,
                         (const int32_t*)blk_base, (const int32_t*)level_q, (const int32_t*)offsets,
                         p.T, p.N, p.K, row_of, token_of_row, static_cast<const u32x4*>(u),
                         static_cast<u32x4*>(x_perm), vec_per_row);
    else
      hipLaunchKernelGGL(dispatch_permute_levels_kernel<false>, dim3(blocks), dim3(256), 0, s, topk_idx,
                         (const int32_t*)blk_base, (const int32_t*)level_q, (const int32_t*)offsets,
                         p.T, p.N, p.K, row_of, token_of_row, static_cast<const u32x4*>(u),
                         static_cast<u32x4*>(x_perm), vec_per_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(disp_blocks), dim3(kTok), 0, s, topk_idx, p.T,
                     p.N, p.K, blk_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool scan_in_block = (int64_t)disp_blocks * p.N <= kScanInBlock;
  if (!scan_in_block) {
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, s, (const int32_t*)blk_count,
                       blk_base, disp_blocks, p.N, capacity, expert_counts, kept_counts, offsets);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto permute = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, topk_idx, (const int32_t*)blk_count,
                       disp_blocks, (const int32_t*)blk_base, offsets, expert_counts, kept_counts, p.T,
                       p.N, p.K, capacity, row_of, token_of_row, static_cast<const u32x4*>(u),
                       static_cast<u32x4*>(x_perm), vec_per_row);
  };
  if (scan_in_block) {
    if (nt) permute(dispatch_permute_kernel<true, true>);
    else permute(dispatch_permute_kernel<true, false>);
  } else {
    if (nt) permute(dispatch_permute_kernel<false, true>);
    else permute(dispatch_permute_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace moe
