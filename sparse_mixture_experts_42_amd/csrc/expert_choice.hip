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
//                      largest affinity (8-bit digits of the fp32 bit
//                      pattern, which orders non-negative floats), then an
//                      in-order compaction from ballots and a fixed-order
//                      scan of per-wave counts
//   ec_rows_kernel     the token-major maps row_of / gate_of from the
//                      per-word selections
//   ec_gather_kernel   x_perm[i*C + j] = u[token j of expert i]
//   ec_combine_kernel  out_t = u_t + sum_i g_{i,t} y[row_{i,t}] (+ shared)
// Integer counts only (LDS histograms with integer atomics, fixed-order
// scans): the selection is bit-identical run to run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelRounds = 8;   // rounds of kSelThreads tokens held per thread at once

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

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

// hist[d] += 1 for every active lane.  With ROUNDS > 0 the first digits met
// in the wave are counted with one atomic each from a leader lane, so that a
// digit most tokens share (the exponent byte of the affinities, in the first
// pass) does not serialise 64 same-address LDS atomics.
template <int ROUNDS>
__device__ __forceinline__ void hist_add(int* hist, uint32_t d, bool active, int lane) {
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const uint64_t act = __ballot(active);
    if (act == 0ull) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
    const bool same = active && d == dl;
    const uint64_t m = __ballot(same);
    if (lane == leader) atomicAdd(&hist[dl], (int)__popcll(m));
    active = active && !same;
  }
  if (active) atomicAdd(&hist[d], 1);
}

// One block per expert.  Radix select, most significant 8-bit digit first:
// each pass histograms the digit of the keys that match the prefix found so
// far, and one wave finds the digit holding the C-th largest key with a
// scan over the 256 bins in descending order.  The passes stop early once
// every key with the current prefix is taken.  The selection is then: key
// prefix above P, or equal to P among the first `need` such tokens in token
// order.  A token's row is (tokens above P before it) + min(tokens equal to
// P before it, need), from ballots and one fixed-order scan of per-wave
// counts, so every expert's rows come out in ascending token order.
//
// Outputs: the expert-major rows (expert_tokens, expert_gates), and per
// 64-token word w of the expert the mask of chosen tokens sel_mask[e][w] and
// the number chosen before the word sel_pre[e][w], from which
// ec_rows_kernel writes the token-major maps.  The first kSelRounds *
// kSelThreads keys stay in registers across the passes.
__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(
    const float* probsT, int T, int C, int W, int32_t* expert_tokens, float* expert_gates,
    uint64_t* sel_mask, int32_t* sel_pre) {
  __shared__ int hist2[2][256];
  __shared__ int cnt[2][kSelRounds * kSelWaves];
  __shared__ int base[2];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_need, sh_done;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t* key = reinterpret_cast<const uint32_t*>(probsT + (size_t)e * T);
  uint32_t k0[kSelRounds];
#pragma unroll
  for (int j = 0; j < kSelRounds; ++j) {
    const int t = j * kSelThreads + tid;
    k0[j] = t < T ? key[t] : 0u;
  }
  if (tid < 256) hist2[0][tid] = 0;
  if (tid == 0) {
    sh_prefix = 0u;
    sh_need = C;
    sh_done = C <= 0;
    base[0] = 0;
    base[1] = 0;
  }
  __syncthreads();
  // hist2[pass & 1] is this pass's histogram; the other one, last read by
  // wave 0 before the previous pass's closing barrier, is cleared for the next
  int shift = 32;
  for (int pass = 0; pass < 4; ++pass) {
    if (sh_done) break;
    shift -= 8;
    int* hist = hist2[pass & 1];
    if (tid < 256) hist2[(pass & 1) ^ 1][tid] = 0;
    const uint32_t prefix = sh_prefix;
    for (int c0 = 0; c0 < T; c0 += kSelRounds * kSelThreads) {
      uint32_t k[kSelRounds];
      if (c0 == 0) {
#pragma unroll
        for (int j = 0; j < kSelRounds; ++j) k[j] = k0[j];
      } else {
#pragma unroll
        for (int j = 0; j < kSelRounds; ++j) {
          const int t = c0 + j * kSelThreads + tid;
          k[j] = t < T ? key[t] : 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < kSelRounds; ++j) {
        const int t = c0 + j * kSelThreads + tid;
        const uint32_t d = (k[j] >> shift) & 255u;
        if (pass == 0) hist_add<1>(hist, d, t < T, lane);
        else hist_add<0>(hist, d, t < T && (k[j] >> shift >> 8) == prefix, lane);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255-4l .. 252-4l, descending
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        sum += c[q];
      }
      const int incl = wave_incl_scan(sum, lane);
      const int need = sh_need;
      int above = incl - sum;
      if (above < need && incl >= need) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + c[q] >= need) {
            sh_prefix = (prefix << 8) | (uint32_t)(255 - 4 * lane - q);
            sh_need = need - above;
            sh_done = need - above == c[q];
            break;
          }
          above += c[q];
        }
      }
    }
    __syncthreads();
  }
  const uint32_t P = sh_prefix;
  const int need = C > 0 ? sh_need : 0;
  const bool none = C <= 0;

  for (int c0 = 0; c0 < T; c0 += kSelRounds * kSelThreads) {
    uint32_t k[kSelRounds];
    uint64_t bh[kSelRounds], be[kSelRounds];
    if (c0 == 0) {
#pragma unroll
      for (int j = 0; j < kSelRounds; ++j) k[j] = k0[j];
    } else {
#pragma unroll
      for (int j = 0; j < kSelRounds; ++j) {
        const int t = c0 + j * kSelThreads + tid;
        k[j] = t < T ? key[t] : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < kSelRounds; ++j) {
      const int t = c0 + j * kSelThreads + tid;
      const uint32_t kp = shift < 32 ? k[j] >> shift : 0u;
      bh[j] = __ballot(!none && t < T && kp > P);
      be[j] = __ballot(!none && t < T && kp == P);
      if (lane == 0) {
        cnt[0][j * kSelWaves + wave] = (int)__popcll(bh[j]);
        cnt[1][j * kSelWaves + wave] = (int)__popcll(be[j]);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // exclusive prefix over (round, wave), i.e. token order, plus the
      // totals of the earlier chunks; lane l holds entries 2l and 2l+1
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int x0 = cnt[a][2 * lane], x1 = cnt[a][2 * lane + 1];
        const int b = base[a];
        const int incl = wave_incl_scan(x0 + x1, lane);
        const int ex = b + incl - x0 - x1;
        cnt[a][2 * lane] = ex;
        cnt[a][2 * lane + 1] = ex + x0;
        const int total = __shfl(incl, 63, 64);
        if (lane == 0) base[a] = b + total;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelRounds; ++j) {
      const int t = c0 + j * kSelThreads + tid;
      const int w = (c0 >> 6) + j * kSelWaves + wave;   // this wave's 64-token word
      if (w >= W) continue;                               // wave-uniform
      const bool hi = (bh[j] >> lane) & 1ull, eq = (be[j] >> lane) & 1ull;
      const int hb0 = cnt[0][j * kSelWaves + wave], eb0 = cnt[1][j * kSelWaves + wave];
      const int hb = hb0 + lanes_below(bh[j]);
      const int eb = eb0 + lanes_below(be[j]);
      const int pos = hb + (eb < need ? eb : need);
      const bool sel = (hi || (eq && eb < need)) && pos < C;
      const uint64_t m = __ballot(sel);
      if (sel) {
        expert_tokens[e * C + pos] = t;
        expert_gates[e * C + pos] = __uint_as_float(k[j]);
      }
      if (lane == 0) {
        sel_mask[(size_t)e * W + w] = m;
        sel_pre[(size_t)e * W + w] = hb0 + (eb0 < need ? eb0 : need);
      }
    }
    __syncthreads();
  }
}

// Token-major maps from the per-word selections: one thread per token,
// row_of[t][e] = e*C + (chosen tokens of e before t), gate_of[t][e] = its
// affinity; -1 and 0 where e did not choose t.  Four experts per 16-byte
// store when N is a multiple of 4 and both maps are 16-byte aligned (vec4).
__global__ __launch_bounds__(256) void ec_rows_kernel(const float* probsT, int T, int N, int C,
                                                      int W, const uint64_t* sel_mask,
                                                      const int32_t* sel_pre, int32_t* row_of,
                                                      float* gate_of, int32_t* offsets, bool vec4) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= N; i += 256) offsets[i] = i * C;
  // the wave's word: its masks and counts are wave-uniform loads
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  if (w >= W) return;
  const int lane = threadIdx.x & 63;
  const bool in = t < T;
  auto one = [&](int e, float p, int32_t& r, float& g) {
    const uint64_t m = sel_mask[(size_t)e * W + w];
    const int pre = sel_pre[(size_t)e * W + w];
    const bool sel = in && ((m >> lane) & 1ull);
    r = sel ? e * C + pre + lanes_below(m) : -1;
    g = sel ? p : 0.0f;
  };
  if (vec4) {
    for (int e = 0; e < N; e += 4) {
      float p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = in ? probsT[(size_t)(e + q) * T + t] : 0.0f;
      int32_t r[4];
      float g[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) one(e + q, p[q], r[q], g[q]);
      if (in) {
        *reinterpret_cast<int4*>(row_of + (size_t)t * N + e) = int4{r[0], r[1], r[2], r[3]};
        *reinterpret_cast<float4*>(gate_of + (size_t)t * N + e) = float4{g[0], g[1], g[2], g[3]};
      }
    }
  } else {
    for (int e = 0; e < N; ++e) {
      const float p = in ? probsT[(size_t)e * T + t] : 0.0f;
      int32_t r;
      float g;
      one(e, p, r, g);
      if (in) {
        row_of[(size_t)t * N + e] = r;
        gate_of[(size_t)t * N + e] = g;
      }
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
                            int32_t* row_of, float* gate_of, int32_t* offsets, void* sel,
                            hipStream_t s) {
  const int W = ec_select_words(p.T);
  uint64_t* sel_mask = static_cast<uint64_t*>(sel);
  int32_t* sel_pre = reinterpret_cast<int32_t*>(sel_mask + (size_t)p.N * W);
  hipLaunchKernelGGL(ec_probs_kernel, dim3((p.T + 255) / 256), dim3(256), 0, s, scores, p.T, p.N,
                     probsT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ec_select_kernel, dim3(p.N), dim3(kSelThreads), 0, s, (const float*)probsT,
                     p.T, C, W, expert_tokens, expert_gates, sel_mask, sel_pre);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ec_rows_kernel, dim3((p.T + 255) / 256), dim3(256), 0, s,
                     (const float*)probsT, p.T, p.N, C, W, (const uint64_t*)sel_mask,
                     (const int32_t*)sel_pre, row_of, gate_of, offsets,
                     (p.N & 3) == 0 && (((uintptr_t)row_of | (uintptr_t)gate_of) & 15u) == 0);
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
