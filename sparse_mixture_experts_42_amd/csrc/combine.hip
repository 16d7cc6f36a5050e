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

constexpr int kMaxK = 16;

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

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* u, const u32x4* y_perm,
                                                      const int32_t* row_of, const float* gate,
                                                      const u32x4* y_shared, u32x4* out, int T,
                                                      int K, int vec_per_row) {
  constexpr int EV = BF16 ? 8 : 4;   // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int wave_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  for (int t = wave_id; t < T; t += nwaves) {
    int rows[kMaxK];
    float g[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      rows[k] = -1;
      g[k] = 0.0f;
      if (k < K) {
        rows[k] = row_of[(size_t)t * K + k];
        g[k] = gate[(size_t)t * K + k];
      }
    }
    for (int v = lane; v < vec_per_row; v += 64) {
      float acc[EV], tmp[EV];
      const u32x4 qu = u[(size_t)t * vec_per_row + v];
      if constexpr (BF16) unpack8(qu, acc);
      else {
        acc[0] = __uint_as_float(qu.x);
        acc[1] = __uint_as_float(qu.y);
        acc[2] = __uint_as_float(qu.z);
        acc[3] = __uint_as_float(qu.w);
      }
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        if (k < K && rows[k] >= 0) {
          const u32x4 qy = y_perm[(size_t)rows[k] * vec_per_row + v];
          if constexpr (BF16) unpack8(qy, tmp);
          else {
            tmp[0] = __uint_as_float(qy.x);
            tmp[1] = __uint_as_float(qy.y);
            tmp[2] = __uint_as_float(qy.z);
            tmp[3] = __uint_as_float(qy.w);
          }
#pragma unroll
          for (int i = 0; i < EV; ++i) acc[i] = fmaf(g[k], tmp[i], acc[i]);
        }
      }
      if (y_shared != nullptr) {
        const u32x4 qs = y_shared[(size_t)t * vec_per_row + v];
        if constexpr (BF16) unpack8(qs, tmp);
        else {
          tmp[0] = __uint_as_float(qs.x);
          tmp[1] = __uint_as_float(qs.y);
          tmp[2] = __uint_as_float(qs.z);
          tmp[3] = __uint_as_float(qs.w);
        }
#pragma unroll
        for (int i = 0; i < EV; ++i) acc[i] += tmp[i];
      }
      u32x4 o;
      if constexpr (BF16) o = pack8(acc);
      else o = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3])};
      out[(size_t)t * vec_per_row + v] = o;
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
  if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(u), static_cast<const u32x4*>(y_perm), row_of,
                       topk_gate, static_cast<const u32x4*>(y_shared), static_cast<u32x4*>(out),
                       p.T, p.K, vec_per_row);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(u), static_cast<const u32x4*>(y_perm), row_of,
                       topk_gate, static_cast<const u32x4*>(y_shared), static_cast<u32x4*>(out),
                       p.T, p.K, vec_per_row);
  return hipGetLastError();
}

}  // namespace moe
