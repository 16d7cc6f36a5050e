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
#include <type_traits>

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

// dH from d_gate through the gating variant:
//   SOFTMAX_TOPK: dH_i = s_i (delta_i - sum_k g_k dg_k), delta_i = dg_k if i = e_k
//   TOPK_SOFTMAX: dH_{e_k} = g_k (dg_k - sum_m g_m dg_m), 0 elsewhere
// One wave per token; lane l writes experts l, l+64, ...  For the softmax
// over all N experts, the max and the sum of exponentials of the logits are
// fixed-order butterflies over the wave.
template <bool kSoftmaxAll>
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* scores,
                                                        const int32_t* topk_idx,
                                                        const float* gate, const float* d_gate,
                                                        float* dH, int T, int N, int K) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int32_t* idx = topk_idx + (size_t)t * K;
  const float* g = gate + (size_t)t * K;
  const float* dg = d_gate + (size_t)t * K;
  float* out = dH + (size_t)t * N;
  float gdg = 0.0f;
  for (int k = 0; k < K; ++k) gdg = fmaf(g[k], dg[k], gdg);
  if constexpr (kSoftmaxAll) {
    const float* h = scores + (size_t)t * N;
    float m = -INFINITY;
    for (int i = lane; i < N; i += 64) m = fmaxf(m, h[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float z = 0.0f;
    for (int i = lane; i < N; i += 64) z += expf(h[i] - m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    const float rz = 1.0f / z;
    for (int i = lane; i < N; i += 64) {
      float delta = 0.0f;
      for (int k = 0; k < K; ++k)
        if (idx[k] == i) delta = dg[k];
      out[i] = expf(h[i] - m) * rz * (delta - gdg);
    }
  } else {
    for (int i = lane; i < N; i += 64) {
      float v = 0.0f;
      for (int k = 0; k < K; ++k)
        if (idx[k] == i) v = g[k] * (dg[k] - gdg);
      out[i] = v;
    }
  }
}

// Router parameter gradients, first level.  A wave owns one slice of
// consecutive tokens, a strip of 64*CPT columns of u and a chunk of NE
// experts; lane l keeps partial[s][e][j] = sum_t dH[t][e] u[t][j] for its CPT
// consecutive columns j and every expert e of the chunk, summed in token
// order.  dH[t][e0 .. e0+NE) is the same for the whole wave.  The waves of
// strip 0 also sum dH itself: the bias gradient, stored as column j = d.
// Tokens go in groups of G.  Slices are short (more waves over the same tokens) unless the
// router is wide and the batch long: the partial array holds
// slices x N x (d+1) floats.
int router_slice_tokens(int T, int N) { return N <= 8 || T <= 1024 ? 32 : 256; }

template <int NE, int CPT, int G>
__global__ __launch_bounds__(256) void router_dw_partial_kernel(const uint16_t* u, const float* dH,
                                                                float* partial, int T, int d,
                                                                int N, int slice_tokens,
                                                                int strips, int chunks,
                                                                int total) {
  using Raw = typename std::conditional<CPT == 8, u32x4, uint2>::type;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= total) return;
  // chunk fastest: the chunks of one (slice, strip) read the same lines of u
  const int c = wave % chunks;
  const int rest = wave / chunks;
  const int strip = rest % strips;
  const int s = rest / strips;
  const int e0 = c * NE;
  const int j = strip * 64 * CPT + lane * CPT;
  const bool colok = j < d;                // d % 64 == 0: a lane's CPT columns are all in or out
  const bool with_bias = strip == 0;
  const int t0 = s * slice_tokens;
  const int t1 = t0 + slice_tokens < T ? t0 + slice_tokens : T;
  float acc[NE][CPT], bias[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    bias[e] = 0.0f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) acc[e][q] = 0.0f;
  }
  const Raw* src = reinterpret_cast<const Raw*>(u + (size_t)t0 * d + (colok ? j : 0));
  const size_t stride = (size_t)d * 2 / sizeof(Raw);
  // dH of a group: lane l loads dH[tg + l / NE][e0 + l % NE], read back per
  // token with readlane; the next group's loads are issued before this
  // group's arithmetic.
  static_assert(G * NE == 64, "one dH element per lane and group");
  const int hl_t = lane / NE, hl_e = e0 + lane % NE;
  auto load = [&](int tg, Raw (&raw)[G], float& hl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      raw[i] = Raw{};
      if (colok && tg + i < t1) raw[i] = src[(size_t)(tg - t0 + i) * stride];
    }
    hl = (tg + hl_t < t1 && hl_e < N) ? dH[(size_t)(tg + hl_t) * N + hl_e] : 0.0f;
  };
  auto compute = [&](int tg, const Raw (&raw)[G], float hl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (tg + i < t1) {
        float hv[NE], uv[CPT];
#pragma unroll
        for (int e = 0; e < NE; ++e)
          hv[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), i * NE + e));
        if constexpr (CPT == 8) {
          unpack8(raw[i], uv);
        } else {
          uv[0] = __uint_as_float(raw[i].x << 16);
          uv[1] = __uint_as_float(raw[i].x & 0xffff0000u);
          uv[2] = __uint_as_float(raw[i].y << 16);
          uv[3] = __uint_as_float(raw[i].y & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int q = 0; q < CPT; ++q) acc[e][q] = fmaf(hv[e], uv[q], acc[e][q]);
        if (with_bias) {
#pragma unroll
          for (int e = 0; e < NE; ++e) bias[e] += hv[e];
        }
      }
    }
  };
  Raw ra[G], rb[G];
  float ha, hb;
  load(t0, ra, ha);
  for (int tg = t0; tg < t1; tg += 2 * G) {
    if (tg + G < t1) load(tg + G, rb, hb);
    compute(tg, ra, ha);
    if (tg + G >= t1) break;
    if (tg + 2 * G < t1) load(tg + 2 * G, ra, ha);
    compute(tg + G, rb, hb);
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    if (e0 + e < N) {
      float* row = partial + ((size_t)s * N + e0 + e) * (d + 1);
      if (colok) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) row[j + q] = acc[e][q];
      }
      if (with_bias && lane == 0) row[d] = bias[e];
    }
  }
}

// Second level: 64 columns of [dW | db] per block.  Four groups of 64
// threads each sum a quarter of the slices in slice order; the four
// quarter sums are then added in quarter order.
__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float* partial, int slices,
                                                               int d, int N, float* dw_router,
                                                               float* db_router) {
  __shared__ float q4[4][64];
  const long long n = (long long)N * (d + 1);
  const long long idx = (long long)blockIdx.x * 64 + (threadIdx.x & 63);
  const int part = threadIdx.x >> 6;
  const int s0 = (int)((long long)slices * part / 4), s1 = (int)((long long)slices * (part + 1) / 4);
  float acc = 0.0f;
  if (idx < n) {
    const float* src = partial + idx;
#pragma unroll 8
    for (int s = s0; s < s1; ++s) acc += src[(size_t)s * n];
  }
  q4[part][threadIdx.x & 63] = acc;
  __syncthreads();
  if (part != 0 || idx >= n) return;
  const int l = threadIdx.x;
  const float v = ((q4[0][l] + q4[1][l]) + q4[2][l]) + q4[3][l];
  const int e = (int)(idx / (d + 1)), j = (int)(idx - (long long)e * (d + 1));
  if (j < d) dw_router[(size_t)e * d + j] = v;
  else if (db_router != nullptr) db_router[e] = v;
}

// du = d_out + sum_k dX[row_of[t][k]] + dX_shared + dH W_router, one
// rounding.  64 tokens x 64 columns per block, 4x4 per thread.  The block's
// row_of entries are staged in LDS first; the gathered rows are then loaded
// four assignments x four tokens at a time, so sixteen loads per thread are
// in flight.  dH and W_router go through LDS 32 experts at a time, and the
// product loop stops at the last expert.
__global__ __launch_bounds__(256) void du_kernel(const float* dH, const float* w_router,
                                                 const uint16_t* d_out, const uint16_t* dx_perm,
                                                 const int32_t* row_of, const uint16_t* dx_shared,
                                                 uint16_t* du, int T, int d, int N, int K) {
  __shared__ float sH[64][33];
  __shared__ float sW[32][64];
  __shared__ int32_t sRow[64 * kMaxK];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int j = j0 + 4 * tx;         // d is a multiple of 64: all four columns valid
  for (int i = threadIdx.x; i < 64 * K; i += 256)
    sRow[i] = t0 + i / K < T ? row_of[(size_t)t0 * K + i] : -1;

  auto add4 = [](float* s, const uint2& v) __attribute__((always_inline)) {
    s[0] += __uint_as_float(v.x << 16);
    s[1] += __uint_as_float(v.x & 0xffff0000u);
    s[2] += __uint_as_float(v.y << 16);
    s[3] += __uint_as_float(v.y & 0xffff0000u);
  };
  float s[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + 4 * ty + a;
    uint2 od = make_uint2(0u, 0u);
    if (t < T) od = *reinterpret_cast<const uint2*>(d_out + (size_t)t * d + j);
    s[a][0] = __uint_as_float(od.x << 16);
    s[a][1] = __uint_as_float(od.x & 0xffff0000u);
    s[a][2] = __uint_as_float(od.y << 16);
    s[a][3] = __uint_as_float(od.y & 0xffff0000u);
  }
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += 4) {
    uint2 xv[4][4];
    bool ok[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = k0 + i < K ? sRow[(4 * ty + a) * K + k0 + i] : -1;
        ok[a][i] = row >= 0;
        xv[a][i] = make_uint2(0u, 0u);
        if (ok[a][i]) xv[a][i] = *reinterpret_cast<const uint2*>(dx_perm + (size_t)row * d + j);
      }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (ok[a][i]) add4(s[a], xv[a][i]);
  }
  if (dx_shared != nullptr) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = t0 + 4 * ty + a;
      if (t < T) add4(s[a], *reinterpret_cast<const uint2*>(dx_shared + (size_t)t * d + j));
    }
  }

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
      const int e = e0 + ee;
      sW[ee][jj] = e < N ? w_router[(size_t)e * d + j0 + jj] : 0.0f;
    }
    __syncthreads();
    const int ne = N - e0 < 32 ? N - e0 : 32;
#pragma unroll 8
    for (int ee = 0; ee < ne; ++ee) {
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
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + 4 * ty + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) s[a][b] += acc[a][b];
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(s[a][0]) | ((uint32_t)f32_to_bf16(s[a][1]) << 16);
    o.y = (uint32_t)f32_to_bf16(s[a][2]) | ((uint32_t)f32_to_bf16(s[a][3]) << 16);
    *reinterpret_cast<uint2*>(du + (size_t)t * d + j) = o;
  }
}

}  // namespace

int router_grad_slices(int T, int N) {
  const int st = router_slice_tokens(T, N);
  return (T + st - 1) / st;
}

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
  const dim3 grid((p.T + 3) / 4);
  if (p.gating == MOE_GATE_SOFTMAX_TOPK)
    hipLaunchKernelGGL(route_bwd_kernel<true>, grid, dim3(256), 0, s, scores, topk_idx, gate,
                       d_gate, dH, p.T, p.N, p.K);
  else
    hipLaunchKernelGGL(route_bwd_kernel<false>, grid, dim3(256), 0, s, scores, topk_idx, gate,
                       d_gate, dH, p.T, p.N, p.K);
  return hipGetLastError();
}

hipError_t launch_router_param_grads(const moe_problem_t& p, const void* u, const float* dH,
                                     float* partial, float* dw_router, float* db_router,
                                     hipStream_t s) {
  const int slices = router_grad_slices(p.T, p.N);
  const int st = router_slice_tokens(p.T, p.N);
  const bool narrow = p.N <= 8;
  const int cols = narrow ? 512 : 256;                   // 64 lanes x CPT columns per wave
  const int strips = (p.d + cols - 1) / cols;
  const int chunks = narrow ? 1 : (p.N + 15) / 16;
  const long long total = (long long)slices * strips * chunks;
  if (total > (1LL << 30)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 3) / 4));
  if (narrow)
    hipLaunchKernelGGL((router_dw_partial_kernel<8, 8, 8>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(u), dH, partial, p.T, p.d, p.N, st, strips,
                       chunks, (int)total);
  else
    hipLaunchKernelGGL((router_dw_partial_kernel<16, 4, 4>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(u), dH, partial, p.T, p.d, p.N, st, strips,
                       chunks, (int)total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)p.N * (p.d + 1);
  hipLaunchKernelGGL(router_dw_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s,
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
