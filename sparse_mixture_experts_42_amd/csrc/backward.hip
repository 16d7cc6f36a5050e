// Backward pass of the layer, apart from the expert GEMMs (grouped_gemm.hip).
//
// The gradient of the MoE-layer equation h_t = u_t + sum_k g_{k,t}
// FFN_{e_k}(u_t) + sum_s FFN_s(u_t) ("Mixture-of-Experts (MoE)" ML notes)
// through the stages of "MoE: Choosing Which MLPs to Use for Each Token"
// ("From Router to Combine"), with the Top-K sets and capacity decisions of
// the forward pass held fixed:
//   combine    dY[row] = g * d_out_t,   d_gate[t][k] = <d_out_t, y[row]>
//   gates      dH = Jacobian of the gating variant applied to d_gate
//   router     dW_router = dH^T u,  db = sum_t dH[t],  du_router = dH W_router
//   dispatch   du_t = d_out_t + sum_k dX[row_of[t][k]] + dX_shared_t + du_router_t
// Every sum runs in a fixed order: results are bit-identical run to run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kChunk = 8;       // 16-byte vectors per lane in flight
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

// One wave per token: dY rows of its kept assignments and the gate
// gradients (lanes accumulate in fp32, then a fixed butterfly over the wave).
__global__ __launch_bounds__(256) void combine_bwd_kernel(const u32x4* d_out, const u32x4* y_perm,
                                                          const int32_t* row_of, const float* gate,
                                                          u32x4* dy_perm, float* d_gate, int T,
                                                          int K, int vec_per_row) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    const size_t tb = (size_t)t * vec_per_row;
    float part[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) part[k] = 0.0f;
    for (int v0 = lane; v0 < vec_per_row; v0 += 64 * kChunk) {
      float o[kChunk][8];
      u32x4 q[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int v = v0 + 64 * c;
        q[c] = v < vec_per_row ? d_out[tb + v] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kChunk; ++c) unpack8(q[c], o[c]);
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) break;
        const int row = row_of[(size_t)t * K + k];
        if (row < 0) continue;
        const float g = gate[(size_t)t * K + k];
        const size_t rb = (size_t)row * vec_per_row;
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int v = v0 + 64 * c;
          q[c] = v < vec_per_row ? y_perm[rb + v] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          float y[8], dy[8];
          unpack8(q[c], y);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            part[k] = fmaf(o[c][i], y[i], part[k]);
            dy[i] = g * o[c][i];
          }
          const int v = v0 + 64 * c;
          if (v < vec_per_row) dy_perm[rb + v] = pack8(dy);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= K) break;
      float x = part[k];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
      if (lane == 0) d_gate[(size_t)t * K + k] = row_of[(size_t)t * K + k] >= 0 ? x : 0.0f;
    }
  }
}

// One thread per token: dH from d_gate through the gating variant.
//   SOFTMAX_TOPK: dH_i = s_i (delta_i - sum_k g_k dg_k), delta_i = dg_k if i = e_k
//   TOPK_SOFTMAX: dH_{e_k} = g_k (dg_k - sum_m g_m dg_m), 0 elsewhere
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* scores, const int32_t* topk_idx,
                                                        const float* gate, const float* d_gate,
                                                        float* dH, int T, int N, int K,
                                                        int softmax_all) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* idx = topk_idx + (size_t)t * K;
  const float* g = gate + (size_t)t * K;
  const float* dg = d_gate + (size_t)t * K;
  float* out = dH + (size_t)t * N;
  float gdg = 0.0f;
  for (int k = 0; k < K; ++k) gdg = fmaf(g[k], dg[k], gdg);
  if (softmax_all) {
    const float* h = scores + (size_t)t * N;
    float m = h[0];
    for (int i = 1; i < N; ++i) m = fmaxf(m, h[i]);
    float z = 0.0f;
    for (int i = 0; i < N; ++i) z += expf(h[i] - m);
    const float rz = 1.0f / z;
    for (int i = 0; i < N; ++i) {
      float delta = 0.0f;
      for (int k = 0; k < K; ++k)
        if (idx[k] == i) delta = dg[k];
      out[i] = expf(h[i] - m) * rz * (delta - gdg);
    }
  } else {
    for (int i = 0; i < N; ++i) out[i] = 0.0f;
    for (int k = 0; k < K; ++k) out[idx[k]] = g[k] * (dg[k] - gdg);
  }
}

// Router parameter gradients, first level: for a slice of kRouterTok tokens,
// partial[s][i][j] = sum_t dH[t][i] u'[t][j] over the columns j of [u | 1]
// (u'[t][d] = 1 gives the bias gradient).  A 64-expert x 64-column tile per
// block, 4x4 per thread; dH and u' go through LDS 32 tokens at a time.
constexpr int kRouterTok = 512;

__global__ __launch_bounds__(256) void router_dw_partial_kernel(const uint16_t* u, const float* dH,
                                                                float* partial, int T, int d,
                                                                int N) {
  __shared__ float sH[32][65];
  __shared__ float sU[32][64];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int j0 = blockIdx.x * 64, e0 = blockIdx.z * 64, s = blockIdx.y;
  const int t_begin = s * kRouterTok;
  const int t_end = t_begin + kRouterTok < T ? t_begin + kRouterTok : T;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    __syncthreads();
    for (int i = threadIdx.x; i < 32 * 64; i += 256) {
      const int tt = i >> 6, cc = i & 63;
      const int t = t0 + tt, e = e0 + cc, j = j0 + cc;
      sH[tt][cc] = (t < t_end && e < N) ? dH[(size_t)t * N + e] : 0.0f;
      float v = 0.0f;
      if (t < t_end) v = j < d ? bf16_to_f32(u[(size_t)t * d + j]) : (j == d ? 1.0f : 0.0f);
      sU[tt][cc] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int tt = 0; tt < 32; ++tt) {
      float hv[4], uv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) hv[a] = sH[tt][4 * ty + a];
#pragma unroll
      for (int b = 0; b < 4; ++b) uv[b] = sU[tt][4 * tx + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(hv[a], uv[b], acc[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int e = e0 + 4 * ty + a;
    if (e >= N) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + 4 * tx + b;
      if (j <= d) partial[((size_t)s * N + e) * (d + 1) + j] = acc[a][b];
    }
  }
}

// Second level: the slices summed in slice order.
__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float* partial, int slices,
                                                               int d, int N, float* dw_router,
                                                               float* db_router) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)N * (d + 1)) return;
  const int e = (int)(idx / (d + 1)), j = (int)(idx - (long long)e * (d + 1));
  float acc = 0.0f;
  for (int s = 0; s < slices; ++s) acc += partial[((size_t)s * N + e) * (d + 1) + j];
  if (j < d) dw_router[(size_t)e * d + j] = acc;
  else if (db_router != nullptr) db_router[e] = acc;
}

// du = d_out + sum_k dX[row_of[t][k]] + dX_shared + dH W_router, one
// rounding.  64 tokens x 64 columns per block, 4x4 per thread; dH and
// W_router go through LDS 32 experts at a time.
__global__ __launch_bounds__(256) void du_kernel(const float* dH, const float* w_router,
                                                 const uint16_t* d_out, const uint16_t* dx_perm,
                                                 const int32_t* row_of, const uint16_t* dx_shared,
                                                 uint16_t* du, int T, int d, int N, int K) {
  __shared__ float sH[64][33];
  __shared__ float sW[32][64];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int e0 = 0; e0 < N; e0 += 32) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      const int tt = i >> 5, ee = i & 31;
      const int t = t0 + tt, e = e0 + ee;
      sH[tt][ee] = (t < T && e < N) ? dH[(size_t)t * N + e] : 0.0f;
    }
    for (int i = threadIdx.x; i < 32 * 64; i += 256) {
      const int ee = i >> 6, jj = i & 63;
      const int e = e0 + ee, j = j0 + jj;
      sW[ee][jj] = (e < N && j < d) ? w_router[(size_t)e * d + j] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int ee = 0; ee < 32; ++ee) {
      float hv[4], wv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) hv[a] = sH[4 * ty + a][ee];
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[b] = sW[ee][4 * tx + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(hv[a], wv[b], acc[a][b]);
    }
  }
  const int j = j0 + 4 * tx;         // d is a multiple of 64: all four columns valid
  if (j >= d) return;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + 4 * ty + a;
    if (t >= T) continue;
    float s[4];
    const uint2 od = *reinterpret_cast<const uint2*>(d_out + (size_t)t * d + j);
    s[0] = __uint_as_float(od.x << 16);
    s[1] = __uint_as_float(od.x & 0xffff0000u);
    s[2] = __uint_as_float(od.y << 16);
    s[3] = __uint_as_float(od.y & 0xffff0000u);
    for (int k = 0; k < K; ++k) {
      const int row = row_of[(size_t)t * K + k];
      if (row < 0) continue;
      const uint2 xv = *reinterpret_cast<const uint2*>(dx_perm + (size_t)row * d + j);
      s[0] += __uint_as_float(xv.x << 16);
      s[1] += __uint_as_float(xv.x & 0xffff0000u);
      s[2] += __uint_as_float(xv.y << 16);
      s[3] += __uint_as_float(xv.y & 0xffff0000u);
    }
    if (dx_shared != nullptr) {
      const uint2 xv = *reinterpret_cast<const uint2*>(dx_shared + (size_t)t * d + j);
      s[0] += __uint_as_float(xv.x << 16);
      s[1] += __uint_as_float(xv.x & 0xffff0000u);
      s[2] += __uint_as_float(xv.y << 16);
      s[3] += __uint_as_float(xv.y & 0xffff0000u);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) s[b] += acc[a][b];
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
    *reinterpret_cast<uint2*>(du + (size_t)t * d + j) = o;
  }
}

}  // namespace

int router_grad_slices(int T) { return (T + kRouterTok - 1) / kRouterTok; }

hipError_t launch_combine_backward(const moe_problem_t& p, const void* d_out, const void* y_perm,
                                   const int32_t* row_of, const float* gate, void* dy_perm,
                                   float* d_gate, hipStream_t s) {
  const int vec_per_row = p.d * 2 / 16;
  long long blocks = ((long long)p.T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(d_out), static_cast<const u32x4*>(y_perm), row_of,
                     gate, static_cast<u32x4*>(dy_perm), d_gate, p.T, p.K, vec_per_row);
  return hipGetLastError();
}

hipError_t launch_route_backward(const moe_problem_t& p, const float* scores,
                                 const int32_t* topk_idx, const float* gate, const float* d_gate,
                                 float* dH, hipStream_t s) {
  hipLaunchKernelGGL(route_bwd_kernel, dim3((p.T + 255) / 256), dim3(256), 0, s, scores, topk_idx,
                     gate, d_gate, dH, p.T, p.N, p.K, p.gating == MOE_GATE_SOFTMAX_TOPK ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_router_param_grads(const moe_problem_t& p, const void* u, const float* dH,
                                     float* partial, float* dw_router, float* db_router,
                                     hipStream_t s) {
  const int slices = router_grad_slices(p.T);
  hipLaunchKernelGGL(router_dw_partial_kernel, dim3((p.d + 1 + 63) / 64, slices, (p.N + 63) / 64),
                     dim3(256), 0, s,
                     static_cast<const uint16_t*>(u), dH, partial, p.T, p.d, p.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)p.N * (p.d + 1);
  hipLaunchKernelGGL(router_dw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const float*)partial, slices, p.d, p.N, dw_router, db_router);
  return hipGetLastError();
}

hipError_t launch_du(const moe_problem_t& p, const float* dH, const float* w_router,
                     const void* d_out, const void* dx_perm, const int32_t* row_of,
                     const void* dx_shared, void* du, hipStream_t s) {
  hipLaunchKernelGGL(du_kernel, dim3((p.T + 63) / 64, p.d / 64), dim3(256), 0, s, dH, w_router,
                     static_cast<const uint16_t*>(d_out), static_cast<const uint16_t*>(dx_perm),
                     row_of, static_cast<const uint16_t*>(dx_shared), static_cast<uint16_t*>(du),
                     p.T, p.d, p.N, p.K);
  return hipGetLastError();
}

}  // namespace moe
