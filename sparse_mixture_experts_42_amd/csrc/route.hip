// Stage 1 -- router: fp32 router GEMM on the matrix cores, then softmax
// statistics, top-K and gates in registers, one 64-lane wave per group of
// tokens.
//
// MoE-layer equation ("Mixture-of-Experts (MoE)" ML notes, quoting
// DeepSeekMoE): s_{i,t} = Softmax_i(u_t^T e_i), g = s on the Top-K, else 0.
// "MoE: Choosing Which MLPs to Use for Each Token", Router section
// (Figure 2): top-K of the scores, then softmax over the selected scores.
// "Noise Top-k Gating", key implementation details: W_noise * N(0,1) noise is
// added to the logits before the selection.  "Switch Transformers explained",
// "Making it work": the router runs at higher precision (fp32 here).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;    // 4 waves

// k-chunk staged in LDS per iteration: wide for narrow routers (few, large
// iterations keep enough bytes in flight for an HBM-bound stream), narrower
// as the padded expert count grows so that the staged weights fit the LDS.
// (at most 512 / NT, and staged u and weights of one chunk within ~80 KB)
template <int TG, int NT>
constexpr int chunk_k() {
  int k = 512 / NT;
  const int fit = 20480 / (16 * TG + 16 * NT) - 4;
  while (k > fit) k /= 2;
  return k < 32 ? 32 : k;
}

struct RouteArgs {
  const void* u;
  const float* w;      // [N][d]
  const float* b;      // [N] or null
  const float* noise;  // [T][N] or null
  float w_noise;
  float* scores;       // [T][N] or null
  int32_t* topk_idx;   // [T][K]
  float* topk_gate;    // [T][K]
  float* lse_sq;       // [T]
  float* part;         // [blocks][N]
  const float* pre;    // [pre_splits][T][N] partial logits (split-k path) or null
  int pre_splits;
  int T, d, N, K, gating;
};

template <typename E> struct Elem;
template <> struct Elem<float> {
  // 4 consecutive values per 16-byte vector
  static constexpr int kPerVec = 4;
};
template <> struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
};

// Order-preserving map of a float to uint32 (larger float -> larger key);
// +0 and -0 are made equal first.
__device__ __forceinline__ uint32_t order_key(float h) {
  if (h == 0.0f) h = 0.0f;
  uint32_t b = __float_as_uint(h);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

template <int G>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <int G>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
template <int G>
__device__ __forceinline__ uint64_t seg_max_u64(uint64_t v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// One block: TOK tokens (TOK = 16 * TG), 4 waves = TG token groups x KS
// k-splits.  NT = experts padded to 16 * NT (NT a power of two, <= 16).
// G = lanes per token in the softmax/top-K phase (power of two, 4..64);
// each lane holds R = max(1, 16*NT/64) expert slots.
// Narrow routers (at most 32 experts) are HBM-bound: DIRECT kernels skip
// the LDS staging and load u and the router weights straight into the
// operand registers of the 16x16x4 MFMA, two 32-wide k-steps ahead.
// The k index of MFMA step m of k-step J on lane group q is 32J + 8q + m for
// both operands, a permutation of k, so the dot products are unchanged.
// PRE: the logits were computed by route_partial_kernel as partial sums over
// pre_splits slices of d; the block sums the slices in slice order instead
// of running the GEMM itself (few-token batches, see launch_route).
template <typename E, int TG, int NT, int G, bool DIRECT, bool PRE = false>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  constexpr int NWV = 4;               // waves per block
  constexpr int TOK = 16 * TG;
  constexpr int KS = NWV / TG;         // waves sharing a token group
  constexpr int NP = 16 * NT;           // padded experts
  constexpr int kDK = chunk_k<TG, NT>();
  constexpr int kLd = kDK + 4;          // padded LDS row (floats): spreads rows over banks
  constexpr int KW = kDK / KS;          // k per wave per chunk
  constexpr int R = (NP + G - 1) / G;   // expert slots per lane
  extern __shared__ float smem[];
  float* sU = smem;                     // [TOK][kLd]
  float* sW = smem + TOK * kLd;         // [NP][kLd]; reused as logits [TOK][NP+1]
  float* sL = (DIRECT || PRE) ? smem : sW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tg = wave / KS;             // token group of this wave
  const int ks = wave % KS;             // k-split of this wave
  const int t0 = blockIdx.x * TOK;
  const int T = a.T, d = a.d, N = a.N;

  constexpr int LdL = NP + 1;
  if constexpr (PRE) {
    static_assert(!DIRECT, "partial logits replace the GEMM");
    for (int i = tid; i < TOK * NP; i += kThreads) {
      const int lt = i / NP, e = i - lt * NP;
      const int t = t0 + lt;
      float v = 0.0f;
      if (t < T && e < N)
        for (int s = 0; s < a.pre_splits; ++s) v += a.pre[((size_t)s * T + t) * N + e];
      sL[lt * LdL + e] = v;
    }
    __syncthreads();
  } else {
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (DIRECT) {
    static_assert(TG == 1 && KS == NWV, "one token group, a k-split per wave");
    constexpr int PD = 2;                 // k-steps in flight per wave
    // lane: token t0 + lane%16, k lanes group q = lane/16; wave ks takes the
    // k-steps J = ks, ks+KS, ... of 32 k each
    const int q = lane >> 4;
    const int t = t0 + (lane & 15);
    const bool t_ok = t < T;
    const E* urow = static_cast<const E*>(a.u) + (size_t)(t_ok ? t : 0) * d + 8 * q;
    const float* wrow[NT];
    bool w_ok[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int e = 16 * j + (lane & 15);
      w_ok[j] = e < N;
      wrow[j] = a.w + (size_t)(w_ok[j] ? e : 0) * d + 8 * q;
    }
    const int nJ = d / 32;
    // one k-step of one lane: 8 u values and 8 weights per expert tile
    struct Step {
      u32x4 u[sizeof(E) == 2 ? 1 : 2];
      float4 w[NT][2];
    };
    auto load = [&](int J, Step& st) {
      const bool ok = J < nJ;
#pragma unroll
      for (int i = 0; i < (sizeof(E) == 2 ? 1 : 2); ++i)
        st.u[i] = (ok && t_ok) ? *reinterpret_cast<const u32x4*>(urow + 32 * J + i * 4)
                               : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          st.w[j][i] = (ok && w_ok[j]) ? *reinterpret_cast<const float4*>(wrow[j] + 32 * J + 4 * i)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto uval = [&](const Step& st, int m) -> float {
      if constexpr (sizeof(E) == 2) {
        const uint32_t w = st.u[0][m >> 1];
        return __uint_as_float((m & 1) ? (w & 0xffff0000u) : (w << 16));
      } else {
        return __uint_as_float(st.u[m >> 2][m & 3]);
      }
    };
    auto wval = [&](const Step& st, int j, int m) -> float {
      const float4 v = st.w[j][m >> 2];
      return (m & 3) == 0 ? v.x : (m & 3) == 1 ? v.y : (m & 3) == 2 ? v.z : v.w;
    };
    auto mul = [&](const Step& st) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float av = uval(st, m);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wval(st, j, m), acc[j], 0, 0, 0);
      }
    };
    // batches of PD k-steps; the next batch is requested before this one
    // is multiplied
    Step cur[PD], nxt[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) load(ks + KS * i, cur[i]);
    for (int J0 = ks; J0 < nJ; J0 += KS * PD) {
#pragma unroll
      for (int i = 0; i < PD; ++i) load(J0 + KS * PD + KS * i, nxt[i]);
#pragma unroll
      for (int i = 0; i < PD; ++i) mul(cur[i]);
#pragma unroll
      for (int i = 0; i < PD; ++i) cur[i] = nxt[i];
    }
  } else {
  // zero padded expert rows once (never overwritten below)
  for (int i = tid; i < (NP - N) * kLd; i += kThreads) sW[N * kLd + i] = 0.0f;

  constexpr int VPR = kDK / Elem<E>::kPerVec;      // 16-byte vectors per u row chunk
  for (int k0 = 0; k0 < d; k0 += kDK) {
    // stage u[t0 .. t0+TOK)[k0 .. k0+kDK) as fp32 and w_router[0..N)[k0 ..
    // k0+kDK): every load of the chunk is issued before any is consumed
    constexpr int UV = (TOK * VPR + kThreads - 1) / kThreads;
    constexpr int WV = (NP * (kDK / 4) + kThreads - 1) / kThreads;
    u32x4 qu[UV];
    float4 qw[WV];
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / VPR, c = v % VPR;
      const int t = t0 + r;
      qu[i] = u32x4{0u, 0u, 0u, 0u};
      if (v < TOK * VPR && t < T && k0 + c * Elem<E>::kPerVec < d)
        qu[i] = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.u) + (size_t)t * d + k0 +
                                                c * Elem<E>::kPerVec);
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / (kDK / 4), c = v % (kDK / 4);
      qw[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < N && k0 + 4 * c < d)
        qw[i] = *reinterpret_cast<const float4*>(a.w + (size_t)r * d + k0 + 4 * c);
    }
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int v = tid + i * kThreads;
      if (v >= TOK * VPR) continue;
      const int r = v / VPR, c = v % VPR;
      float* dst = sU + r * kLd + c * Elem<E>::kPerVec;
      const u32x4 q = qu[i];
      if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[2 * j] = __uint_as_float(q[j] << 16);
          dst[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = __uint_as_float(q[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = tid + i * kThreads;
      const int r = v / (kDK / 4), c = v % (kDK / 4);
      if (r < N) *reinterpret_cast<float4*>(sW + r * kLd + 4 * c) = qw[i];
    }
    __syncthreads();
    // 16x16x4 fp32 MFMA: A row = token (lane%16), B col = expert (lane%16),
    // k = lane/16 within each group of 4
    const float* pa = sU + (tg * 16 + (lane & 15)) * kLd + ks * KW + (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < KW; kk += 4) {
      const float av = pa[kk];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float bv = sW[(j * 16 + (lane & 15)) * kLd + ks * KW + kk + (lane >> 4)];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  }

  // ---- sum the k-split partial logits into sL[TOK][NP+1] (fixed order)
  for (int s = 0; s < KS; ++s) {
    if (ks == s) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float* dst = sL + (tg * 16 + 4 * (lane >> 4) + v) * LdL + j * 16 + (lane & 15);
          *dst = (s == 0) ? acc[j][v] : *dst + acc[j][v];
        }
    }
    __syncthreads();
  }
  }  // !PRE

  // ---- softmax statistics, top-K and gates: each wave takes TOK/4 tokens
  constexpr int TPW = TOK / NWV;            // tokens per wave
  constexpr int TPP = (64 / G) < TPW ? (64 / G) : TPW;  // tokens per pass
  const int seg = lane / G, j = lane % G;
  float pacc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) pacc[r] = 0.0f;

  for (int pass = 0; pass < TPW / TPP; ++pass) {
    const int lt = wave * TPW + pass * TPP + seg;   // token within block
    const int t = t0 + lt;
    const bool tok_ok = (seg < TPP) && (t < T);
    float h[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = j + r * G;
      ok[r] = tok_ok && (i < N);
      float v = -INFINITY;
      if (ok[r]) {
        v = sL[lt * LdL + i];
        if (a.b) v += a.b[i];
        if (a.noise) v = fmaf(a.w_noise, a.noise[(size_t)t * N + i], v);
        if (a.scores) a.scores[(size_t)t * N + i] = v;
      }
      h[r] = v;
    }
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) m = fmaxf(m, h[r]);
    m = seg_max<G>(m);
    float e[R], z = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      e[r] = ok[r] ? expf(h[r] - m) : 0.0f;
      z += e[r];
    }
    z = seg_sum<G>(z);
    const float inv_z = 1.0f / z;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ok[r]) pacc[r] += e[r] / z;
    if (tok_ok && j == 0) {
      const float lse = m + logf(z);
      a.lse_sq[t] = lse * lse;
    }
    (void)inv_z;
    // top-K by K rounds of a segment-wide max of (score, -index) keys
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t i = j + r * G;
      key[r] = ok[r] ? ((uint64_t)order_key(h[r]) << 32) | (uint64_t)(0xffffffffu - i) : 0ull;
    }
    float hk0 = 0.0f, gsum = 0.0f;
    int sel_idx[16];
    float sel_h[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < a.K) {
        uint64_t best = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) best = key[r] > best ? key[r] : best;
        best = seg_max_u64<G>(best);
        const uint32_t idx = 0xffffffffu - (uint32_t)(best & 0xffffffffu);
        const float hk = order_key_inv((uint32_t)(best >> 32));
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (key[r] == best) key[r] = 0ull;
        sel_idx[k] = (int)idx;
        sel_h[k] = hk;
        if (k == 0) hk0 = hk;
        gsum += expf(hk - hk0);
      }
    }
    if (tok_ok && j == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < a.K) {
          float g;
          if (a.gating == MOE_GATE_SOFTMAX_TOPK) g = expf(sel_h[k] - m) / z;
          else g = expf(sel_h[k] - hk0) / gsum;
          a.topk_idx[(size_t)t * a.K + k] = sel_idx[k];
          a.topk_gate[(size_t)t * a.K + k] = g;
        }
      }
    }
  }

  // ---- per-block sums of the softmax probabilities (fixed order)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = pacc[r];
    for (int o = G; o < 64; o <<= 1) v += __shfl_xor(v, o);
    pacc[r] = v;
  }
  __syncthreads();                       // sL no longer read
  float* sP = smem;                      // [NWV][NP]
  if (lane < G) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = lane + r * G;
      if (i < NP) sP[wave * NP + i] = pacc[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += NWV * 64) {
    float v = sP[i];
#pragma unroll
    for (int w = 1; w < NWV; ++w) v += sP[w * NP + i];
    a.part[(size_t)i * gridDim.x + blockIdx.x] = v;
  }
}

// Split-k logits for few-token batches: block (token tile, slice s, expert
// group) computes 16 tokens x 16*NTB experts over d-slice s on the fp32
// 16x16x4 MFMA, register-direct as in the narrow router (k permuted within
// each 32-wide step), the 4 waves on interleaved 32-wide steps, summed over
// the waves in wave order through LDS:  pre[s][t][e] = sum_{k in slice s}.
template <typename E, int NTB>
__global__ __launch_bounds__(kThreads) void route_partial_kernel(const void* u, const float* w, int T,
                                                                 int d, int N, int dk, float* pre) {
  __shared__ float red[4][16][16 * NTB + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, s = blockIdx.y, e0 = blockIdx.z * 16 * NTB;
  const int q = lane >> 4;
  const int t = t0 + (lane & 15);
  const bool t_ok = t < T;
  const E* urow = static_cast<const E*>(u) + (size_t)(t_ok ? t : 0) * d + 8 * q;
  const float* wrow[NTB];
  bool w_ok[NTB];
#pragma unroll
  for (int j = 0; j < NTB; ++j) {
    const int e = e0 + 16 * j + (lane & 15);
    w_ok[j] = e < N;
    wrow[j] = w + (size_t)(w_ok[j] ? e : 0) * d + 8 * q;
  }
  f32x4 acc[NTB];
#pragma unroll
  for (int j = 0; j < NTB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int J0 = s * dk / 32, J1 = J0 + dk / 32;
  for (int J = J0 + wave; J < J1; J += 4) {
    float uv[8];
    if constexpr (sizeof(E) == 2) {
      const u32x4 qu = t_ok ? *reinterpret_cast<const u32x4*>(urow + 32 * J) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < 8; ++m)
        uv[m] = __uint_as_float((m & 1) ? (qu[m >> 1] & 0xffff0000u) : (qu[m >> 1] << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 qu = t_ok ? *reinterpret_cast<const u32x4*>(urow + 32 * J + 4 * i)
                              : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < 4; ++m) uv[4 * i + m] = __uint_as_float(qu[m]);
      }
    }
#pragma unroll
    for (int j = 0; j < NTB; ++j) {
      float wv[8];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 v = w_ok[j] ? *reinterpret_cast<const float4*>(wrow[j] + 32 * J + 4 * i)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
        wv[4 * i] = v.x;
        wv[4 * i + 1] = v.y;
        wv[4 * i + 2] = v.z;
        wv[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(uv[m], wv[m], acc[j], 0, 0, 0);
    }
  }
  // lane holds tokens 4*(lane/16) + v, expert 16*j + lane%16
#pragma unroll
  for (int j = 0; j < NTB; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][16 * j + (lane & 15)] = acc[j][v];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 16 * NTB; i += kThreads) {
    const int tt = i / (16 * NTB), ee = i - tt * 16 * NTB;
    const int tok = t0 + tt, e = e0 + ee;
    if (tok >= T || e >= N) continue;
    const float v = ((red[0][tt][ee] + red[1][tt][ee]) + red[2][tt][ee]) + red[3][tt][ee];
    pre[((size_t)s * T + tok) * N + e] = v;
  }
}

// ------------------------------------------------- bf16 token batches
// The fp32 router weights as three bf16 parts, W = W_hi + W_mid + W_lo:
// W_hi keeps the top 8 significant bits of W (truncation), W_mid the top 8
// of the residual W - W_hi and W_lo the rest.  Each residual is exact in
// fp32 and what is left after W_mid has at most 8 significant bits, so the
// sum is exactly W for every finite |W| >= 2^-90 (below that the last part
// falls into the subnormals and loses less than 2^-133).  A bf16 token value
// times a part is exact in fp32, so the bf16 matrix instruction with fp32
// accumulation evaluates the fp32 router dot product.
__host__ __device__ inline uint16_t bf16_trunc_bits(float f) {
  uint32_t x;
  __builtin_memcpy(&x, &f, 4);
  return (uint16_t)(x >> 16);
}
__host__ __device__ inline float bf16_bits_to_f32(uint16_t h) {
  const uint32_t x = (uint32_t)h << 16;
  float f;
  __builtin_memcpy(&f, &x, 4);
  return f;
}
__host__ __device__ inline void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = bf16_trunc_bits(w);
  const float r1 = w - bf16_bits_to_f32(hi);
  mid = bf16_trunc_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  lo = bf16_trunc_bits(r2);
}

// wp[part][e][k] for e < Np (rows e >= N are zero), four k per thread.
__global__ __launch_bounds__(256) void route_split_kernel(const float* w, int N, int Np, int d,
                                                          uint16_t* wp) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per_part = (long long)Np * d;
  if (i * 4 >= per_part) return;
  const int e = (int)(i * 4 / d), k = (int)(i * 4 - (long long)e * d);
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (e < N) x = *reinterpret_cast<const float4*>(w + (size_t)e * d + k);
  const float v[4] = {x.x, x.y, x.z, x.w};
  uint16_t q[3][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split3(v[j], q[0][j], q[1][j], q[2][j]);
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    uint2 o;
    o.x = (uint32_t)q[p][0] | ((uint32_t)q[p][1] << 16);
    o.y = (uint32_t)q[p][2] | ((uint32_t)q[p][3] << 16);
    *reinterpret_cast<uint2*>(wp + (size_t)p * per_part + (size_t)e * d + k) = o;
  }
}

// Router logits of bf16 tokens on the bf16 matrix cores:
//   pre[s][t][e] = sum over k in d-slice s of u[t][k] * (W_hi + W_mid + W_lo)[e][k]
// Block (token tile, expert tile, slice s): 32*EXP_T experts x TOKB tokens,
// four waves of 32 experts x 32 tokens (v_mfma_f32_32x32x16_bf16, experts as
// the A rows, tokens as the B columns, three instructions per 16-wide k-step,
// one per weight part).  Token rows and weight parts go through LDS in
// 64-wide k chunks, loaded straight from global memory into a ring of three
// stages (1-KB buffer loads, 8 rows of 128 bytes each, so every load reads
// whole cache lines); two chunks are in flight while one is multiplied.
// Rows past the batch or past the experts read zero through the buffer
// descriptors' sizes.  LDS rows hold 8 chunks of 16 bytes, chunk c of row r
// at slot c ^ ((r >> 1) & 7), so the operand reads of 16 lanes hit 16
// different 16-byte bank groups.
typedef __attribute__((address_space(3))) void lds_void;

template <int EXP_T, int NW, int NS>
__global__ __launch_bounds__(64 * NW) void route_logits_kernel(const uint16_t* u, const uint16_t* wp, int T,
                                                               int d, int N, int Np, int dk, float* pre) {
  constexpr int NE = 32 * EXP_T;              // experts per block
  constexpr int TOKB = 32 * NW / EXP_T;       // tokens per block
  constexpr int PD = NS - 1;                  // chunks in flight
  constexpr int UQ = TOKB / 8 / NW;           // 1-KB token loads per wave per chunk
  constexpr int WQ = 3 * NE / 8 / NW;         // 1-KB weight loads per wave per chunk
  constexpr int LPW = UQ + WQ;
  static_assert(UQ * 8 * NW == TOKB && WQ * 8 * NW == 3 * NE, "whole loads per wave");
  __shared__ u32x4 sU[NS][TOKB * 8];
  __shared__ u32x4 sW[NS][3 * NE * 8];        // [part][row][8 slots]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int et = wave % EXP_T, tt = wave / EXP_T;
  const int t0 = blockIdx.x * TOKB, e0 = blockIdx.y * NE, s = blockIdx.z;
  const int kbeg = s * dk, nch = dk / 64;
  const size_t per_part = (size_t)Np * d;

  // buffer descriptors: the block's token rows, each part's expert rows
  const int trows = T - t0 < TOKB ? T - t0 : TOKB;
  const int erows = N - e0 < NE ? N - e0 : NE;
  const __amdgpu_buffer_rsrc_t rU = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(u + (size_t)t0 * d + kbeg), (short)0, (int)((uint32_t)trows * d * 2), 0x00020000);
  __amdgpu_buffer_rsrc_t rW[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
    rW[p] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wp + p * per_part + (size_t)e0 * d + kbeg),
                                              (short)0, (int)((uint32_t)erows * d * 2), 0x00020000);
  // load q of a chunk fills rows 8q .. 8q+7; lane l row 8q + l/8, slot l%8,
  // which holds chunk (l%8) ^ ((8q + l/8) >> 1 & 7)
  const int lrow = lane >> 3;
  const int ch_even = (lane & 7) ^ (lrow >> 1), ch_odd = (lane & 7) ^ (4 + (lrow >> 1));
  auto issue = [&](int c, int buf) {
    const uint32_t kb = (uint32_t)c * 128u;   // bytes into the slice
#pragma unroll
    for (int i = 0; i < UQ; ++i) {
      const int q = wave * UQ + i;
      const uint32_t voff = (uint32_t)((8 * q + lrow) * d) * 2u + kb + (uint32_t)((q & 1) ? ch_odd : ch_even) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rU, (lds_void*)&sU[buf][q * 64], 16, voff, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int q = wave * WQ + i;            // over 3 parts x NE/8 row groups
      const int p = q / (NE / 8), qr = q - p * (NE / 8);
      const uint32_t voff = (uint32_t)((8 * qr + lrow) * d) * 2u + kb + (uint32_t)((qr & 1) ? ch_odd : ch_even) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW[p], (lds_void*)&sW[buf][q * 64], 16, voff, 0, 0, 0);
    }
  };

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  const int arow = et * 32 + (lane & 31), brow = tt * 32 + (lane & 31);
#pragma unroll
  for (int c = 0; c < PD; ++c)
    if (c < nch) issue(c, c);
  for (int c = 0; c < nch; ++c) {
    const int buf = c % NS;
    // chunk c has landed once at most the loads of the chunks after it
    // (up to PD - 1 of them) are pending
    const int later = nch - 1 - c < PD - 1 ? nch - 1 - c : PD - 1;
    if (later >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPW) : "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // every wave is past chunk c-1, whose buffer takes chunk c + PD
    if (c + PD < nch) issue(c + PD, (c + PD) % NS);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      const bf16x8 b = __builtin_bit_cast(bf16x8, sU[buf][brow * 8 + (ch ^ ((brow >> 1) & 7))]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, sW[buf][(p * NE + arow) * 8 + (ch ^ ((arow >> 1) & 7))]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
  }
  // lane: token t0 + brow, experts e0 + et*32 + 8*(v/4) + 4*(lane/32) + v%4
  const int t = t0 + brow;
  if (t >= T) return;
  float* out = pre + ((size_t)s * T + t) * N;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int e = e0 + et * 32 + 8 * g + 4 * (lane >> 5);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (e + v < N) out[e + v] = acc[4 * g + v];
  }
}

// The slices summed in slice order, one thread per (token, expert), eight
// loads in flight: out[t][e] = sum_s pre[s][t][e].
__global__ __launch_bounds__(256) void route_pre_reduce_kernel(const float* pre, int S, long long TN,
                                                               float* out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= TN) return;
  float acc = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = s0 + j < S ? pre[(size_t)(s0 + j) * TN + i] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
  }
  out[i] = acc;
}

// mean_prob[i] = (sum of the per-block sums part[i][*]) / T: one block per
// expert; thread t sums blocks t, t+256, ... in order, then a fixed tree.
__global__ __launch_bounds__(256) void route_finalize_kernel(const float* part, int blocks, int N,
                                                             int T, float* mean_prob) {
  __shared__ float s[256];
  const int i = blockIdx.x;
  const float* p = part + (size_t)i * blocks;
  float acc = 0.0f;
  for (int b = threadIdx.x; b < blocks; b += 256) acc += p[b];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean_prob[i] = s[0] / (float)T;
}

// Router statistics, one block: the variance of the assignment fractions
// f_i = counts_i / (T K), the variance and entropy of the mean probabilities
// and the mean of lse^2.  Double accumulators in a fixed order (strided
// per-thread sums, then a fixed tree), so the result is run-to-run exact.
__device__ __forceinline__ double block_sum(double v, double* s) {
  s[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  const double r = s[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void router_stats_kernel(const int32_t* counts,
                                                           const float* mean_prob,
                                                           const float* lse_sq, int T, int N,
                                                           int K, float* stats) {
  __shared__ double s[256];
  const int i = threadIdx.x;
  double z = 0.0;
  for (int t = i; t < T; t += 256) z += (double)lse_sq[t];
  z = block_sum(z, s);
  const double n = (double)N, tk = (double)T * (double)K;
  double fv = 0.0, pv = 0.0, en = 0.0;
  if (i < N) {
    const double f = (double)counts[i] / tk - 1.0 / n;
    const double pi = (double)mean_prob[i];
    fv = f * f;
    pv = (pi - 1.0 / n) * (pi - 1.0 / n);
    en = pi > 0.0 ? -pi * log(pi) : 0.0;
  }
  fv = block_sum(fv, s);
  pv = block_sum(pv, s);
  en = block_sum(en, s);
  if (i == 0) {
    stats[0] = (float)(fv / n);
    stats[1] = (float)(pv / n);
    stats[2] = (float)en;
    stats[3] = (float)(z / (double)T);
  }
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <typename E, int TG, int NT, int G, bool PRE>
hipError_t launch_g(const RouteArgs& a, int blocks, hipStream_t s) {
  constexpr bool DIRECT = !PRE && TG == 1 && NT <= 2;
  constexpr int TOK = 16 * TG, NP = 16 * NT;
  constexpr int kLd = chunk_k<TG, NT>() + 4;
  constexpr size_t stage = (size_t)(TOK + NP) * kLd * sizeof(float);
  constexpr size_t logits = (size_t)TOK * kLd * sizeof(float) + (size_t)TOK * (NP + 1) * sizeof(float);
  constexpr size_t direct = (size_t)(TOK * (NP + 1) > 4 * NP ? TOK * (NP + 1) : 4 * NP) * sizeof(float);
  constexpr size_t lds = (DIRECT || PRE) ? direct : (stage > logits ? stage : logits);
  static_assert(lds <= 160 * 1024, "router tile exceeds the LDS of a CU");
  if constexpr (lds > 64 * 1024) {
    static bool attr_set = false;   // once per instantiation (idempotent)
    if (!attr_set) {
      const hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&route_kernel<E, TG, NT, G, DIRECT, PRE>),
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  hipLaunchKernelGGL((route_kernel<E, TG, NT, G, DIRECT, PRE>), dim3(blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename E, int TG, int NT, int G>
hipError_t launch_gp(const RouteArgs& a, int blocks, hipStream_t s) {
  if (a.pre != nullptr) {
    if constexpr (TG == 1) return launch_g<E, TG, NT, G, true>(a, blocks, s);
    else return hipErrorInvalidValue;
  }
  return launch_g<E, TG, NT, G, false>(a, blocks, s);
}

// Lanes per token G: up to 16 experts, the smallest power of two >= N (at
// least 4), one expert per lane; wider routers use 16 lanes per token, each
// holding NT experts, so a wave selects for four tokens at once with
// four-step butterflies.
template <typename E, int TG, int NT>
hipError_t launch_gsel(const moe_problem_t& p, const RouteArgs& a, int blocks, hipStream_t s) {
  if constexpr (NT == 1) {
    if (p.N <= 4) return launch_gp<E, TG, 1, 4>(a, blocks, s);
    if (p.N <= 8) return launch_gp<E, TG, 1, 8>(a, blocks, s);
    return launch_gp<E, TG, 1, 16>(a, blocks, s);
  } else {
    return launch_gp<E, TG, NT, 16>(a, blocks, s);
  }
}

template <typename E, int TG>
hipError_t launch_nt(const moe_problem_t& p, const RouteArgs& a, int blocks, hipStream_t s) {
  const int nt = pow2_at_least((p.N + 15) / 16);
  switch (nt) {
    case 1: return launch_gsel<E, TG, 1>(p, a, blocks, s);
    case 2: return launch_gsel<E, TG, 2>(p, a, blocks, s);
    case 4: return launch_gsel<E, TG, 4>(p, a, blocks, s);
    case 8: return launch_gsel<E, TG, 8>(p, a, blocks, s);
    case 16: return launch_gsel<E, TG, 16>(p, a, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
hipError_t launch_tg(const moe_problem_t& p, const RouteArgs& a, int blocks, hipStream_t s) {
  switch (route_tokens_per_block(p)) {
    case 16: return launch_nt<E, 1>(p, a, blocks, s);
    case 32: return launch_nt<E, 2>(p, a, blocks, s);
    case 64: return launch_nt<E, 4>(p, a, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// bf16 token batches with more than 32 experts (where the fp32 router
// products, not the token stream, bound the router): the logits come from
// route_logits_kernel over S slices of d, chosen so that the grid has at
// least ~256 blocks (one per CU, whose LDS the ring fills) with S dividing
// d/64; the selection kernel then reads them.  Narrower routers keep the
// fused fp32 kernel, which streams the tokens in one launch.
// Up to 32 experts: 4 waves of 32 tokens and a 5-stage ring (the token
// stream is the traffic; four chunks in flight).  Wider: 8 waves of 32
// tokens x 2 expert tiles of 32, 128 tokens per block, a 3-stage ring: the
// weight parts, re-read by every block, are shared by twice as many tokens.
struct Bf3Plan {
  int exp_t, ne, np, tokb, gx, gy, S;
};
Bf3Plan bf3_plan(const moe_problem_t& p) {
  Bf3Plan q;
  q.exp_t = p.N > 32 ? 2 : 1;
  q.ne = 32 * q.exp_t;
  q.np = (p.N + q.ne - 1) / q.ne * q.ne;
  q.tokb = 128;
  q.gx = (p.T + q.tokb - 1) / q.tokb;
  q.gy = q.np / q.ne;
  const int want = (256 + q.gx * q.gy - 1) / (q.gx * q.gy);
  const int kc = p.d / 64;
  q.S = kc;
  for (int c = 1; c <= kc; ++c)
    if (kc % c == 0 && c >= want) {
      q.S = c;
      break;
    }
  return q;
}
// slices the selection kernel sums itself; more are summed by
// route_pre_reduce_kernel first
constexpr int kSelectSlices = 8;

// fp32 token batches with fewer than 256 tiles of 16 tokens would leave most
// of the chip idle with one block per 16 tokens: their logits are computed
// in pre_splits slices of d by route_partial_kernel first (at least ~512
// blocks), then summed by the routing blocks.  0: the fused path.
bool use_bf3(const moe_problem_t& p) { return p.dtype == MOE_BF16 && p.N > 32; }

int route_pre_splits(const moe_problem_t& p) {
  if (p.T == 0) return 0;
  if (use_bf3(p)) return bf3_plan(p).S;
  const int tiles = (p.T + 15) / 16;
  if (tiles >= 256) return 0;
  const int groups = (p.N + 63) / 64;
  int S = 1;
  while (S < 32 && S * 2 * 32 <= p.d / 4 && p.d % (S * 2 * 32) == 0 && tiles * groups * S < 512)
    S *= 2;
  return S;
}

// [S][T][N] partial logits, their sum when S > kSelectSlices (bf16) or S > 0
// (fp32), and for bf16 the three weight parts [3][Np][d]
size_t route_pre_bytes(const moe_problem_t& p) {
  const int S = route_pre_splits(p);
  if (S == 0) return 0;
  const size_t TN = (size_t)p.T * p.N * sizeof(float);
  if (!use_bf3(p)) return (size_t)(S + 1) * TN;
  const Bf3Plan q = bf3_plan(p);
  const size_t logits = align_up((size_t)(S + (S > kSelectSlices ? 1 : 0)) * TN, kAlign);
  return logits + (size_t)3 * q.np * p.d * sizeof(uint16_t);
}

// Small expert counts keep the router HBM-bound: few tokens per block, many
// blocks.  Wide routers reuse the staged router weights over more tokens.
int route_tokens_per_block(const moe_problem_t& p) {
  if (route_pre_splits(p) > 0) return 16;
  if (p.N <= 32) return 16;
  if ((long long)p.T >= 64LL * 256) return 64;
  if ((long long)p.T >= 32LL * 256) return 32;
  return 16;
}

hipError_t launch_route(const moe_problem_t& p, const void* u, const float* w_router,
                        const float* b_router, const float* noise, float* scores,
                        int32_t* topk_idx, float* topk_gate, float* mean_prob,
                        float* lse_sq, float* part, int route_blocks, float* pre,
                        hipStream_t s) {
  RouteArgs a;
  a.u = u;
  a.w = w_router;
  a.b = b_router;
  a.noise = noise;
  a.w_noise = p.noise_weight;
  a.scores = scores;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.lse_sq = lse_sq;
  a.part = part;
  a.T = p.T;
  a.d = p.d;
  a.N = p.N;
  a.K = p.K;
  a.gating = p.gating;
  a.pre = nullptr;
  a.pre_splits = route_pre_splits(p);
  const long long TN = (long long)p.T * p.N;
  if (use_bf3(p)) {
    const Bf3Plan q = bf3_plan(p);
    const int S = q.S, dk = p.d / S;
    uint16_t* wp = reinterpret_cast<uint16_t*>(
        reinterpret_cast<char*>(pre) +
        align_up((size_t)(S + (S > kSelectSlices ? 1 : 0)) * (size_t)TN * sizeof(float), kAlign));
    const long long pieces = (long long)q.np * p.d / 4;
    hipLaunchKernelGGL(route_split_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                       w_router, p.N, q.np, p.d, wp);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    const dim3 grid(q.gx, q.gy, S);
    if (q.exp_t == 1)
      hipLaunchKernelGGL((route_logits_kernel<1, 4, 5>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(u),
                         (const uint16_t*)wp, p.T, p.d, p.N, q.np, dk, pre);
    else
      hipLaunchKernelGGL((route_logits_kernel<2, 8, 3>), grid, dim3(512), 0, s, static_cast<const uint16_t*>(u),
                         (const uint16_t*)wp, p.T, p.d, p.N, q.np, dk, pre);
    e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    a.pre = pre;
    if (S > kSelectSlices) {
      float* summed = pre + (size_t)S * TN;
      hipLaunchKernelGGL(route_pre_reduce_kernel, dim3((unsigned)((TN + 255) / 256)), dim3(256), 0, s,
                         (const float*)pre, S, TN, summed);
      e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      a.pre = summed;
      a.pre_splits = 1;
    }
  } else if (a.pre_splits > 0) {
    const int S = a.pre_splits, dk = p.d / S;
    const int nt = pow2_at_least((p.N + 15) / 16);
    const dim3 grid((p.T + 15) / 16, S, (p.N + 63) / 64);
    if (p.dtype == MOE_BF16) {
      if (nt == 1) hipLaunchKernelGGL((route_partial_kernel<uint16_t, 1>), grid, dim3(kThreads), 0, s, u, w_router, p.T, p.d, p.N, dk, pre);
      else hipLaunchKernelGGL((route_partial_kernel<uint16_t, 2>), grid, dim3(kThreads), 0, s, u, w_router, p.T, p.d, p.N, dk, pre);
    } else {
      if (nt == 1) hipLaunchKernelGGL((route_partial_kernel<float, 1>), grid, dim3(kThreads), 0, s, u, w_router, p.T, p.d, p.N, dk, pre);
      else if (nt == 2) hipLaunchKernelGGL((route_partial_kernel<float, 2>), grid, dim3(kThreads), 0, s, u, w_router, p.T, p.d, p.N, dk, pre);
      else hipLaunchKernelGGL((route_partial_kernel<float, 4>), grid, dim3(kThreads), 0, s, u, w_router, p.T, p.d, p.N, dk, pre);
    }
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    // the slices summed into slice S, which the routing blocks then read
    float* summed = pre + (size_t)S * TN;
    hipLaunchKernelGGL(route_pre_reduce_kernel, dim3((unsigned)((TN + 255) / 256)), dim3(256), 0, s,
                       (const float*)pre, S, TN, summed);
    e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    a.pre = summed;
    a.pre_splits = 1;
  }
  hipError_t e = p.dtype == MOE_BF16 ? launch_tg<uint16_t>(p, a, route_blocks, s)
                                     : launch_tg<float>(p, a, route_blocks, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_finalize_kernel, dim3(p.N), dim3(256), 0, s, (const float*)part,
                     route_blocks, p.N, p.T, mean_prob);
  return hipGetLastError();
}

hipError_t launch_router_stats(const moe_problem_t& p, const int32_t* expert_counts,
                               const float* mean_prob, const float* lse_sq, float* stats,
                               hipStream_t s) {
  hipLaunchKernelGGL(router_stats_kernel, dim3(1), dim3(256), 0, s, expert_counts, mean_prob,
                     lse_sq, p.T, p.N, p.K, stats);
  return hipGetLastError();
}

}  // namespace moe
