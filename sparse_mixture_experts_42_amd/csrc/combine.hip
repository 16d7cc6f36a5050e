// Stage 4 -- combine: gate-weighted un-permute and sum, plus the residual.
//
// "MoE: Choosing Which MLPs to Use for Each Token", "From Router to Combine":
// combine gathers each expert's results by the original token and sums them
// weighted by the router's gates; "Shared Expert" (Figure 4): the shared
// path is added, y = S(x) + R(x).  MoE-layer equation of the "Mixture-of-
// Experts (MoE)" ML notes: the residual u_t is added.  Dropped assignments
// (capacity overflow, "Mixture of Experts (MoE)" glossary) add nothing.
//
// One wave per token; each lane streams 16-byte vectors of the token's K
// expert rows, accumulates in fp32 in the order u, k = 0..K-1, shared, and
// rounds once to the element type.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8(const u32x4& q, float* f) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ void unpack(const u32x4& q, float* f, bool bf16) {
  if (bf16) {
    unpack8(q, f);
  } else {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
}

// Each lane owns kChunk vectors of a row at a time and issues all their
// loads of one source row (u, then each expert row, then the shared row)
// before using any: 8 KB per wave in flight per source instead of 1 KB,
// which is what keeps HBM busy when nothing is cached.
constexpr int kChunk = 8;

template <bool BF16, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* u, const u32x4* y_perm,
                                                      const int32_t* row_of, const float* gate,
                                                      const u32x4* y_shared, u32x4* out, int T,
                                                      int K, int vec_per_row) {
  constexpr int EV = BF16 ? 8 : 4;   // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int wave_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  for (int t = wave_id; t < T; t += nwaves) {
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
      for (int k = 0; k < K; ++k) {
        const int row = row_of[(size_t)t * K + k];
        if (row < 0) continue;
        const float g = gate[(size_t)t * K + k];
        const size_t rb = (size_t)row * vec_per_row;
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int v = v0 + 64 * c;
          if constexpr (NT)
            q[c] = v < vec_per_row ? __builtin_nontemporal_load(&y_perm[rb + v]) : u32x4{0u, 0u, 0u, 0u};
          else
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
        if constexpr (BF16)
          out[tb + v] = pack8(acc[c]);
        else
          out[tb + v] = u32x4{__float_as_uint(acc[c][0]), __float_as_uint(acc[c][1]),
                              __float_as_uint(acc[c][2]), __float_as_uint(acc[c][3])};
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const void* u, const void* y_perm,
                          const int32_t* row_of, const float* topk_gate,
                          const void* y_shared, void* out, hipStream_t s) {
  const size_t es = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = (int)((size_t)p.d * es / 16);
  long long blocks = ((long long)p.T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  const bool nt = (size_t)p.T * p.K * p.d * es > kStreamRowsBytes;
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const u32x4*>(u),
                       static_cast<const u32x4*>(y_perm), row_of, topk_gate,
                       static_cast<const u32x4*>(y_shared), static_cast<u32x4*>(out), p.T, p.K,
                       vec_per_row);
  };
  if (p.dtype == MOE_BF16) {
    if (nt) run(combine_kernel<true, true>);
    else run(combine_kernel<true, false>);
  } else {
    if (nt) run(combine_kernel<false, true>);
    else run(combine_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace moe
