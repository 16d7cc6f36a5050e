// Stage 3 -- expert FFNs as grouped GEMMs over ragged per-expert row groups.
//
// "MoE: Choosing Which MLPs to Use for Each Token": each expert is a gated
// MLP with Gate, Up and Down weights (Figure 1) applied to the tokens of its
// group, row by row with no mixing between tokens ("From Router to
// Combine"); shared experts process every token (Figure 4).  "Mixture-of-
// Experts (MoE)" ML notes: every expert is structurally a standard FFN.
//
// Both GEMMs read their operands K-contiguous ([row][k] activations,
// [out][in] weights), which is the operand layout of the 32x32x16 bf16
// matrix-core instruction: lane l holds 8 consecutive k of row l%32.
//   GEMM-1: act[r][f] = SiLU(x_r . Wg_e[f]) * (x_r . Wu_e[f])   (SwiGLU)
//           act[r][f] = ReLU(x_r . W1_e[f])                    (ReLU FFN)
//   GEMM-2: y[r][j]   = act_r . Wd_e[j]
// The group of a row block is looked up on the device from the expert
// offsets, so the host never learns the ragged sizes.
#include "moe_internal.h"

namespace moe {
namespace {

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };

struct GemmArgs {
  const void* A;            // activations [rows_alloc][lda]
  const void* B0;           // weights of group 0: [Ndim][ldb] per K-segment
  const void* B1;           // up-projection weights (SwiGLU), same layout
  void* C;                  // [rows][ldc]
  const int32_t* offsets;   // [G+1] group row offsets, or null: one group [0, M)
  const int32_t* tiles;     // [G+1] prefix of row tiles per group (with offsets)
  int G;
  int M;                    // rows of the single group when offsets == null
  int rows_alloc;           // rows addressable through A (loads are clamped)
  int Ndim;                 // output columns
  int Kdim;                 // reduction length
  int lda, ldb, ldc;
  int kseg;                 // K-segment length of B (Kdim when unsegmented)
  size_t kseg_stride;       // elements between K-segments of B
  size_t b_group_stride;    // elements between consecutive groups' B
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

template <int EPI>
__device__ __forceinline__ float epilogue(float g, float up) {
  if constexpr (EPI == EPI_SWIGLU) return silu(g) * up;
  else if constexpr (EPI == EPI_RELU) return g > 0.0f ? g : 0.0f;
  else return g;
}

// Locate the row block: returns false when the block has no work.
__device__ __forceinline__ bool find_tile(const GemmArgs& a, int bx, int BM, int& g, int& row0,
                                          int& rows) {
  if (a.offsets == nullptr) {
    g = 0;
    row0 = bx * BM;
    rows = a.M - row0;
    if (rows > BM) rows = BM;
    return rows > 0;
  }
  if (bx >= a.tiles[a.G]) return false;
  int lo = 0, hi = a.G;            // tiles[lo] <= bx < tiles[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tiles[mid] <= bx) lo = mid;
    else hi = mid;
  }
  g = lo;
  const int mt = bx - a.tiles[g];
  row0 = a.offsets[g] + mt * BM;
  rows = a.offsets[g + 1] - row0;
  if (rows > BM) rows = BM;
  return rows > 0;
}

// Consecutive logical blocks are spread by the hardware over the 8 XCDs
// round-robin; remap so that each XCD gets a contiguous run of logical
// blocks (row blocks sharing one weight tile then meet in one L2).
__device__ __forceinline__ void xcd_remap(int& bx, int& by) {
  const int nx = gridDim.x, total = gridDim.x * gridDim.y;
  int lin = blockIdx.x + blockIdx.y * nx;
  const int full = total - total % 8;
  if (lin < full) lin = (lin % 8) * (full / 8) + lin / 8;
  bx = lin % nx;
  by = lin / nx;
}

// ------------------------------------------------------------ bf16 MFMA
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;

// LDS tiles are [rows][64 bf16] = 8 chunks of 16 bytes per row; chunk c of
// row r lives at slot c ^ (r & 7) so that the 32 rows read by one MFMA
// operand load spread over all banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

template <int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][BM * 8];
  __shared__ u32x4 sB[2][BN * 8];
  int bx, by;
  xcd_remap(bx, by);
  int g, row0, rows;
  if (!find_tile(a, bx, BM, g, row0, rows)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bg = static_cast<const uint16_t*>(a.B0) + (size_t)g * a.b_group_stride;
  const uint16_t* Bu = EPI == EPI_SWIGLU
                           ? static_cast<const uint16_t*>(a.B1) + (size_t)g * a.b_group_stride
                           : Bg;
  // SwiGLU tiles hold 64 act columns: B rows 0..63 gate, 64..127 up
  const int n0 = EPI == EPI_SWIGLU ? by * (BN / 2) : by * BN;

  // global -> LDS: thread loads chunk lc of rows lr + 32 j (row offsets in
  // elements; B rows of SwiGLU tiles alternate gate (0..63) and up (64..127))
  const int lc = tid & 7, lr = tid >> 3;
  size_t oa[4], ob[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = row0 + lr + 32 * j;
    r = r < a.rows_alloc ? r : a.rows_alloc - 1;
    oa[j] = (size_t)r * a.lda + lc * 8;
    const int tr = lr + 32 * j;
    int n = EPI == EPI_SWIGLU ? n0 + (tr & 63) : n0 + tr;
    n = n < a.Ndim ? n : a.Ndim - 1;
    ob[j] = (size_t)n * a.ldb + lc * 8;
  }
  const uint16_t* pb_lo = Bg;                                  // B rows 0..63 of the tile
  const uint16_t* pb_hi = EPI == EPI_SWIGLU ? Bu : Bg;         // B rows 64..127
  u32x4 ra[4], rb[4];
  // (explicitly unrolled: the staging registers must never be indexed
  // dynamically, or they would be demoted to scratch)
#define MOE_GLOAD1(j_, kb_, boff_)                                                  \
  ra[j_] = *reinterpret_cast<const u32x4*>(A + oa[j_] + (kb_));                     \
  rb[j_] = *reinterpret_cast<const u32x4*>(((j_) < 2 ? pb_lo : pb_hi) + ob[j_] + (boff_));
#define MOE_GLOAD(kt_)                                                              \
  do {                                                                              \
    const int kb_ = (kt_) * BK;                                                     \
    const int seg_ = kb_ / a.kseg;                                                  \
    const size_t boff_ = (size_t)seg_ * a.kseg_stride + (kb_ - seg_ * a.kseg);      \
    MOE_GLOAD1(0, kb_, boff_) MOE_GLOAD1(1, kb_, boff_)                             \
    MOE_GLOAD1(2, kb_, boff_) MOE_GLOAD1(3, kb_, boff_)                             \
  } while (0)
#define MOE_SSTORE1(j_, buf_)                                                       \
  sA[(buf_)][swz(lr + 32 * (j_), lc)] = ra[j_];                                     \
  sB[(buf_)][swz(lr + 32 * (j_), lc)] = rb[j_];
#define MOE_SSTORE(buf_)                                                            \
  do {                                                                              \
    MOE_SSTORE1(0, buf_) MOE_SSTORE1(1, buf_) MOE_SSTORE1(2, buf_) MOE_SSTORE1(3, buf_) \
  } while (0)

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // B rows used by this wave for its two n-tiles
  int brow[2];
  if (EPI == EPI_SWIGLU) {
    brow[0] = wn * 32;          // gate rows
    brow[1] = 64 + wn * 32;     // up rows, same act columns
  } else {
    brow[0] = wn * 64;
    brow[1] = wn * 64 + 32;
  }

  const int nk = a.Kdim / BK;
  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 q = sA[buf][swz(wm * 64 + i * 32 + (lane & 31), c)];
        fa[i] = __builtin_bit_cast(bf16x8, q);
        const u32x4 w = sB[buf][swz(brow[i] + (lane & 31), c)];
        fb[i] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_SSTORE(buf ^ 1);
    __syncthreads();
  }

#undef MOE_GLOAD1
#undef MOE_GLOAD
#undef MOE_SSTORE1
#undef MOE_SSTORE
  // epilogue: lane holds column lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4
  uint16_t* C = static_cast<uint16_t*>(a.C);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= rows) continue;
      if (EPI == EPI_SWIGLU) {
        const int col = n0 + wn * 32 + (lane & 31);
        if (col < a.Ndim)
          C[(size_t)(row0 + r) * a.ldc + col] = f32_to_bf16(epilogue<EPI>(acc[i][0][v], acc[i][1][v]));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + brow[j] + (lane & 31);
          if (col < a.Ndim)
            C[(size_t)(row0 + r) * a.ldc + col] = f32_to_bf16(epilogue<EPI>(acc[i][j][v], 0.0f));
        }
      }
    }
  }
}

// --------------------------------------------------------------- fp32
// Plain fp32 path (one thread per output element), for fp32 problems.
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmArgs a, int BMr) {
  int g, row0, rows;
  if (!find_tile(a, blockIdx.x, BMr, g, row0, rows)) return;
  const int col = blockIdx.y * 256 + threadIdx.x;
  if (col >= a.Ndim) return;
  const float* A = static_cast<const float*>(a.A);
  const float* Bg = static_cast<const float*>(a.B0) + (size_t)g * a.b_group_stride;
  const float* Bu = EPI == EPI_SWIGLU ? static_cast<const float*>(a.B1) + (size_t)g * a.b_group_stride
                                      : nullptr;
  float* C = static_cast<float*>(a.C);
  for (int r = 0; r < rows; ++r) {
    const float* x = A + (size_t)(row0 + r) * a.lda;
    float s0 = 0.0f, s1 = 0.0f;
    for (int k = 0; k < a.Kdim; ++k) {
      const int seg = k / a.kseg;
      const size_t off = (size_t)seg * a.kseg_stride + (size_t)col * a.ldb + (k - seg * a.kseg);
      s0 = fmaf(x[k], Bg[off], s0);
      if (EPI == EPI_SWIGLU) s1 = fmaf(x[k], Bu[off], s1);
    }
    C[(size_t)(row0 + r) * a.ldc + col] = epilogue<EPI>(s0, s1);
  }
}

// tiles[g+1] = tiles[g] + ceil((offsets[g+1]-offsets[g]) / BM), one block
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t* offsets, int G, int BMr,
                                                        int32_t* tiles) {
  __shared__ int32_t s[256];
  const int g = threadIdx.x;
  s[g] = g < G ? (offsets[g + 1] - offsets[g] + BMr - 1) / BMr : 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = g >= o ? s[g - o] : 0;
    __syncthreads();
    s[g] += v;
    __syncthreads();
  }
  if (g < G) tiles[g + 1] = s[g];
  if (g == 0) tiles[0] = 0;
}

hipError_t run_gemm(const GemmArgs& a, int epi, bool bf16, int mtiles_max, hipStream_t s) {
  if (bf16) {
    const int bn = epi == EPI_SWIGLU ? BN / 2 : BN;
    dim3 grid(mtiles_max, (a.Ndim + bn - 1) / bn);
    switch (epi) {
      case EPI_SWIGLU:
        hipLaunchKernelGGL(grouped_gemm_bf16_kernel<EPI_SWIGLU>, grid, dim3(kThreads), 0, s, a);
        break;
      case EPI_RELU:
        hipLaunchKernelGGL(grouped_gemm_bf16_kernel<EPI_RELU>, grid, dim3(kThreads), 0, s, a);
        break;
      default:
        hipLaunchKernelGGL(grouped_gemm_bf16_kernel<EPI_NONE>, grid, dim3(kThreads), 0, s, a);
        break;
    }
  } else {
    dim3 grid(mtiles_max, (a.Ndim + 255) / 256);
    switch (epi) {
      case EPI_SWIGLU:
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, a, BM);
        break;
      case EPI_RELU:
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_RELU>, grid, dim3(256), 0, s, a, BM);
        break;
      default:
        hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_NONE>, grid, dim3(256), 0, s, a, BM);
        break;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_ffn(const moe_problem_t& p, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, const void* u, const void* ws_gate,
                              const void* ws_up, const void* ws_down, void* y_perm,
                              void* y_shared, int32_t* tiles, void* act, void* act_shared,
                              hipStream_t s) {
  const bool bf16 = p.dtype == MOE_BF16;
  const int epi1 = p.act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_RELU;
  const int rows_alloc = p.T * p.K;
  const int mtiles_max = (rows_alloc + BM - 1) / BM + p.N;

  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, offsets, p.N, BM, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // routed experts
  GemmArgs g1{};
  g1.A = x_perm;
  g1.B0 = w_gate;
  g1.B1 = w_up;
  g1.C = act;
  g1.offsets = offsets;
  g1.tiles = tiles;
  g1.G = p.N;
  g1.rows_alloc = rows_alloc;
  g1.Ndim = p.d_ff;
  g1.Kdim = p.d;
  g1.lda = p.d;
  g1.ldb = p.d;
  g1.ldc = p.d_ff;
  g1.kseg = p.d;
  g1.kseg_stride = 0;
  g1.b_group_stride = (size_t)p.d_ff * p.d;
  if ((e = run_gemm(g1, epi1, bf16, mtiles_max, s)) != hipSuccess) return e;

  GemmArgs g2 = g1;
  g2.A = act;
  g2.B0 = w_down;
  g2.B1 = nullptr;
  g2.C = y_perm;
  g2.Ndim = p.d;
  g2.Kdim = p.d_ff;
  g2.lda = p.d_ff;
  g2.ldb = p.d_ff;
  g2.ldc = p.d;
  g2.kseg = p.d_ff;
  g2.b_group_stride = (size_t)p.d * p.d_ff;
  if ((e = run_gemm(g2, EPI_NONE, bf16, mtiles_max, s)) != hipSuccess) return e;

  if (p.n_shared > 0) {
    // all shared experts as one expert of width n_shared*d_ff_shared: the
    // gate/up rows of consecutive experts are contiguous; the down
    // projection is K-segmented, one segment per shared expert
    const int ws_w = p.n_shared * p.d_ff_shared;
    const int mt = (p.T + BM - 1) / BM;
    GemmArgs s1{};
    s1.A = u;
    s1.B0 = ws_gate;
    s1.B1 = ws_up;
    s1.C = act_shared;
    s1.offsets = nullptr;
    s1.tiles = nullptr;
    s1.G = 1;
    s1.M = p.T;
    s1.rows_alloc = p.T;
    s1.Ndim = ws_w;
    s1.Kdim = p.d;
    s1.lda = p.d;
    s1.ldb = p.d;
    s1.ldc = ws_w;
    s1.kseg = p.d;
    s1.kseg_stride = 0;
    s1.b_group_stride = 0;
    if ((e = run_gemm(s1, epi1, bf16, mt, s)) != hipSuccess) return e;
    GemmArgs s2 = s1;
    s2.A = act_shared;
    s2.B0 = ws_down;
    s2.B1 = nullptr;
    s2.C = y_shared;
    s2.Ndim = p.d;
    s2.Kdim = ws_w;
    s2.lda = ws_w;
    s2.ldb = p.d_ff_shared;
    s2.ldc = p.d;
    s2.kseg = p.d_ff_shared;
    s2.kseg_stride = (size_t)p.d * p.d_ff_shared;
    if ((e = run_gemm(s2, EPI_NONE, bf16, mt, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
