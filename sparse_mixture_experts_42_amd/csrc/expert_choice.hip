// Expert-choice routing: each expert selects its top-C tokens.
//
// "Mixture of Experts (MoE)" glossary, sparse-MoE entry: expert choice
// inverts the routing, letting the experts select the top-k tokens.  The
// affinities are those of the MoE-layer equation ("Mixture-of-Experts (MoE)"
// ML notes): s_{i,t} = Softmax_i over the experts of token t's router
// scores.  Expert i takes the C tokens of largest s_{i,t} (ties: the lower
// token index) and holds them in rows i*C .. i*C+C-1 in ascending token
// order; the gate of a chosen pair is s_{i,t}; a token's output adds the
// gated outputs of every expert that chose it, in ascending expert order.
//
// Kernels:
//   ec_probs_kernel    s from the router scores, written expert-major [N][T]
//   ec_select_kernel   one block per expert: radix select of the C-th
//                      largest affinity (four 8-bit digits of the fp32 bit
//                      pattern, which orders non-negative floats), then an
//                      in-order compaction with a fixed block scan
//   ec_gather_kernel   x_perm[i*C + j] = u[token j of expert i]
//   ec_combine_kernel  out_t = u_t + sum_i g_{i,t} y[row_{i,t}] (+ shared)
// Integer counts only (LDS histograms with integer atomics, fixed-order
// scans): the selection is bit-identical run to run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSelThreads = 1024;

// one thread per token: s_i = exp(H_i - m) / sum_j exp(H_j - m)
__global__ __launch_bounds__(256) void ec_probs_kernel(const float* scores, int T, int N,
                                                       float* probsT) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* h = scores + (size_t)t * N;
  float m = h[0];
  for (int i = 1; i < N; ++i) m = fmaxf(m, h[i]);
  float z = 0.0f;
  for (int i = 0; i < N; ++i) z += expf(h[i] - m);
  for (int i = 0; i < N; ++i) probsT[(size_t)i * T + t] = expf(h[i] - m) / z;
}

// exclusive prefix sum over the block's threads (fixed order), and the total
__device__ __forceinline__ int block_excl_scan(int v, int* s, int& total) {
  const int tid = threadIdx.x;
  s[tid] = v;
  __syncthreads();
  for (int o = 1; o < kSelThreads; o <<= 1) {
    const int w = tid >= o ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += w;
    __syncthreads();
  }
  total = s[kSelThreads - 1];
  const int r = s[tid] - v;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(
    const float* probsT, int T, int N, int C, int32_t* expert_tokens, float* expert_gates,
    int32_t* row_of, float* gate_of, int32_t* offsets) {
  __shared__ int hist[256];
  __shared__ int scan[kSelThreads];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_need;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(probsT + (size_t)e * T);
  if (tid == 0) {
    offsets[e] = e * C;
    if (e == 0) offsets[N] = N * C;
    sh_prefix = 0u;
    sh_need = C;
  }
  // radix select, most significant digit first: after the four passes
  // sh_prefix is the key of the C-th largest affinity and sh_need the
  // number of tokens with exactly that key to take (the first ones)
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh_prefix;
    if (C > 0) {
      for (int t = tid; t < T; t += kSelThreads) {
        const uint32_t k = key[t];
        const bool match = pass == 0 || (k >> (shift + 8)) == prefix;
        if (match) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (tid == 0 && C > 0) {
      int need = sh_need, above = 0, dig = 0;
      for (int dd = 255; dd >= 0; --dd) {
        if (above + hist[dd] >= need) {
          dig = dd;
          break;
        }
        above += hist[dd];
      }
      sh_need = need - above;
      sh_prefix = (prefix << 8) | (uint32_t)dig;
    }
    __syncthreads();
  }
  const uint32_t kstar = sh_prefix;
  const int need_eq = C > 0 ? sh_need : 0;

  // compaction in token order: thread tid owns tokens [t0, t1)
  const int chunk = (T + kSelThreads - 1) / kSelThreads;
  const int t0 = tid * chunk < T ? tid * chunk : T;
  const int t1 = t0 + chunk < T ? t0 + chunk : T;
  int n_gt = 0, n_eq = 0;
  if (C > 0) {
    for (int t = t0; t < t1; ++t) {
      const uint32_t k = key[t];
      n_gt += k > kstar;
      n_eq += k == kstar;
    }
  }
  int tot;
  const int eq_before = block_excl_scan(n_eq, scan, tot);
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  const int pos0 = block_excl_scan(n_gt + take_eq, scan, tot);
  int pos = pos0, eq_seen = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t k = key[t];
    bool sel = false;
    if (C > 0) {
      if (k > kstar) sel = true;
      else if (k == kstar) sel = eq_seen++ < take_eq;
    }
    if (sel) {
      const int row = e * C + pos;
      const float g = __uint_as_float(k);
      expert_tokens[row] = t;
      expert_gates[row] = g;
      row_of[(size_t)t * N + e] = row;
      gate_of[(size_t)t * N + e] = g;
      ++pos;
    } else {
      row_of[(size_t)t * N + e] = -1;
      gate_of[(size_t)t * N + e] = 0.0f;
    }
  }
}

// x_perm[r] = u[expert_tokens[r]]: one wave per row, 16-byte vectors, eight
// per lane loaded before any is stored
__global__ __launch_bounds__(256) void ec_gather_kernel(const u32x4* u, const int32_t* tokens,
                                                        u32x4* x_perm, int rows,
                                                        int vec_per_row) {
  constexpr int CH = 8;
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += nw) {
    const u32x4* src = u + (size_t)tokens[r] * vec_per_row;
    u32x4* dst = x_perm + (size_t)r * vec_per_row;
    for (int v0 = lane; v0 < vec_per_row; v0 += 64 * CH) {
      u32x4 q[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (v0 + 64 * c < vec_per_row) q[c] = src[v0 + 64 * c];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (v0 + 64 * c < vec_per_row) dst[v0 + 64 * c] = q[c];
    }
  }
}

__device__ __forceinline__ void unpack(const u32x4& q, float* f, bool bf16) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  if (bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// One wave per token: the experts that chose the token are compacted, in
// ascending expert order, into an LDS list of (row, gate); the token's
// vectors then accumulate in fp32 in the order u, list, shared, and are
// rounded once.
constexpr int kChunk = 8;    // 16-byte vectors per lane in flight

template <bool BF16>
__global__ __launch_bounds__(256) void ec_combine_kernel(const u32x4* u, const u32x4* y_perm,
                                                         const int32_t* row_of,
                                                         const float* gate_of,
                                                         const u32x4* y_shared, u32x4* out, int T,
                                                         int N, int vec_per_row) {
  constexpr int EV = BF16 ? 8 : 4;
  __shared__ int32_t lrow[4][256];
  __shared__ float lgate[4][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + wv; t < T; t += nw) {
    int n = 0;
    for (int i0 = 0; i0 < N; i0 += 64) {
      const int i = i0 + lane;
      const int32_t row = i < N ? row_of[(size_t)t * N + i] : -1;
      const uint64_t m = __ballot(row >= 0);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (row >= 0) {
        lrow[wv][n + before] = row;
        lgate[wv][n + before] = gate_of[(size_t)t * N + i];
      }
      n += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // each lane issues the loads of kChunk vectors of one source row before
    // using any of them (8 KB per wave in flight per source row)
    const size_t tb = (size_t)t * vec_per_row;
    for (int v0 = lane; v0 < vec_per_row; v0 += 64 * kChunk) {
      float acc[kChunk][EV];
      u32x4 q[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int v = v0 + 64 * c;
        q[c] = v < vec_per_row ? u[tb + v] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kChunk; ++c) unpack(q[c], acc[c], BF16);
      for (int j = 0; j < n; ++j) {
        const size_t rb = (size_t)lrow[wv][j] * vec_per_row;
        const float g = lgate[wv][j];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int v = v0 + 64 * c;
          q[c] = v < vec_per_row ? y_perm[rb + v] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          float tmp[EV];
          unpack(q[c], tmp, BF16);
#pragma unroll
          for (int i = 0; i < EV; ++i) acc[c][i] = fmaf(g, tmp[i], acc[c][i]);
        }
      }
      if (y_shared != nullptr) {
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int v = v0 + 64 * c;
          q[c] = v < vec_per_row ? y_shared[tb + v] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          float tmp[EV];
          unpack(q[c], tmp, BF16);
#pragma unroll
          for (int i = 0; i < EV; ++i) acc[c][i] += tmp[i];
        }
      }
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int v = v0 + 64 * c;
        if (v >= vec_per_row) continue;
        u32x4 o;
        if constexpr (BF16) {
          uint32_t w[4];
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
            w[q2] = (uint32_t)f32_to_bf16(acc[c][2 * q2]) |
                    ((uint32_t)f32_to_bf16(acc[c][2 * q2 + 1]) << 16);
          o = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          o = u32x4{__float_as_uint(acc[c][0]), __float_as_uint(acc[c][1]),
                    __float_as_uint(acc[c][2]), __float_as_uint(acc[c][3])};
        }
        out[tb + v] = o;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_ec_select(const moe_problem_t& p, const float* scores, int32_t C,
                            float* probsT, int32_t* expert_tokens, float* expert_gates,
                            int32_t* row_of, float* gate_of, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(ec_probs_kernel, dim3((p.T + 255) / 256), dim3(256), 0, s, scores, p.T, p.N,
                     probsT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ec_select_kernel, dim3(p.N), dim3(kSelThreads), 0, s, (const float*)probsT,
                     p.T, p.N, C, expert_tokens, expert_gates, row_of, gate_of, offsets);
  return hipGetLastError();
}

hipError_t launch_ec_gather(const moe_problem_t& p, const void* u, const int32_t* tokens,
                            int rows, void* x_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = (int)((size_t)p.d * es / 16);
  long long blocks = (rows + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ec_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(u), tokens, static_cast<u32x4*>(x_perm), rows,
                     vec_per_row);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const moe_problem_t& p, const void* u, const void* y_perm,
                             const int32_t* row_of, const float* gate_of, const void* y_shared,
                             void* out, hipStream_t s) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = (int)((size_t)p.d * es / 16);
  long long blocks = (p.T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(ec_combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(u), static_cast<const u32x4*>(y_perm), row_of,
                       gate_of, static_cast<const u32x4*>(y_shared), static_cast<u32x4*>(out),
                       p.T, p.N, vec_per_row);
  else
    hipLaunchKernelGGL(ec_combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(u), static_cast<const u32x4*>(y_perm), row_of,
                       gate_of, static_cast<const u32x4*>(y_shared), static_cast<u32x4*>(out),
                       p.T, p.N, vec_per_row);
  return hipGetLastError();
}

}  // namespace moe
