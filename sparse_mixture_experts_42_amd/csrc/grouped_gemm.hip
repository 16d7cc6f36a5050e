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
  const int32_t* tiles;     // [G+1] prefix of full-height row tiles per group
  const int32_t* tails;     // [G+1] prefix of short tail tiles per group
  int tail_rows;            // tallest tail tile (0: no tail tiles)
  int ext_rows;             // rows a group's last full tile may run past its height
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

// Row tiles of a group of n rows: full-height tiles (the last may be partly
// filled).  A group a few rows past a multiple of the tile height does not
// pay for a whole extra tile: when it has a full tile and the remainder is at
// most ext_rows rows, its last full tile is extended by the remainder (one
// taller tile that reuses the same weight panels); a group shorter than one
// tile with at most tail_rows rows gets one short tail tile instead.
__host__ __device__ inline void split_rows(int n, int BM, int tail_rows, int ext_rows, int& full,
                                           int& tail) {
  const int q = n / BM, rem = n % BM;
  full = q;
  tail = 0;
  if (rem == 0 || (q > 0 && rem <= ext_rows)) return;
  if (tail_rows > 0 && rem <= tail_rows) tail = 1;
  else full = q + 1;
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

constexpr int kPatchN = 4;   // n-tiles per patch: an XCD works on m-tiles x 4 n-tiles of one group

// Full-height tiles of all groups (single-group form: from M).
__host__ __device__ inline int full_tiles_total(const GemmArgs& a, int BM) {
  if (a.offsets != nullptr) return a.tiles[a.G];
  int f, t;
  split_rows(a.M, BM, a.tail_rows, a.ext_rows, f, t);
  return f;
}

// 1-D grid: blocks [0, full tiles x n-tiles) are the full-height tiles, the
// blocks after them the tail tiles.  The hardware hands consecutive blocks
// to the 8 XCDs round-robin, each XCD with its own L2; full-tile block h is
// remapped so that each XCD owns a contiguous run of logical tiles, and
// logical tiles walk each group in patches of (all its row tiles) x kPatchN
// n-tiles, so the activation and weight panels of a patch are fetched into
// one L2 once and shared by the blocks of the patch.  rows is at most BM,
// except for a group's last tile, which may run up to ext_rows further.
__host__ __device__ inline void find_tile_2d(const GemmArgs& a, int BM, int ntiles, int h, int real,
                                             int& g, int& row0, int& rows, int& nt) {
  int mt_g, base;
  const int full = real - real % 8;
  const int L = h < full ? (h % 8) * (full / 8) + h / 8 : h;
  if (a.offsets == nullptr) {
    g = 0;
    mt_g = real / ntiles;
    base = 0;
  } else {
    int lo = 0, hi = a.G;          // tiles[lo]*ntiles <= L < tiles[hi]*ntiles
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tiles[mid] * ntiles <= L) lo = mid;
      else hi = mid;
    }
    g = lo;
    mt_g = a.tiles[g + 1] - a.tiles[g];
    base = a.tiles[g] * ntiles;
  }
  const int l = L - base;
  const int nb = l / (mt_g * kPatchN);
  const int rem = l - nb * mt_g * kPatchN;
  const int nbe = ntiles - nb * kPatchN < kPatchN ? ntiles - nb * kPatchN : kPatchN;
  const int mt = rem / nbe;
  nt = nb * kPatchN + rem % nbe;
  row0 = (a.offsets == nullptr ? 0 : a.offsets[g]) + mt * BM;
  const int end = a.offsets == nullptr ? a.M : a.offsets[g + 1];
  rows = end - row0;
  if (mt < mt_g - 1 && rows > BM) rows = BM;
}

// Tail tile h (counted from the first tail block): n-tile fastest.  Returns
// false past the last tail tile.
__host__ __device__ inline bool find_tail(const GemmArgs& a, int BM, int ntiles, int h, int& g,
                                          int& row0, int& rows, int& nt) {
  if (a.tail_rows == 0) return false;
  const int ti = h / ntiles;
  nt = h - ti * ntiles;
  int full, end;
  if (a.offsets == nullptr) {
    int t;
    split_rows(a.M, BM, a.tail_rows, a.ext_rows, full, t);
    if (ti >= t) return false;
    g = 0;
    row0 = full * BM;
    end = a.M;
  } else {
    if (ti >= a.tails[a.G]) return false;
    int lo = 0, hi = a.G;          // tails[lo] <= ti < tails[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tails[mid] <= ti) lo = mid;
      else hi = mid;
    }
    g = lo;
    row0 = a.offsets[g] + (a.tiles[g + 1] - a.tiles[g]) * BM;
    end = a.offsets[g + 1];
  }
  rows = end - row0;
  return rows > 0;
}

// ------------------------------------------------------------ bf16 MFMA
// Block tile BM x BN (BN counts weight rows: for SwiGLU the first half are
// gate rows and the second half the up rows of the same BN/2 act columns),
// WGM x WGN waves (4 or 8), each wave a (BM/WGM) x (BN/WGN) grid of 32x32
// accumulators.  K advances 64 at a time through two LDS stages that are
// filled straight from global memory (buffer loads to LDS, no register
// staging) while the matrix cores work on the other stage.  Eight waves put
// two on every SIMD, so one wave's matrix instructions run while the other
// waits on LDS reads or on the stage barrier.
constexpr int BK = 64;               // k per stage: 128 bytes per tile row

typedef __attribute__((address_space(3))) void lds_t;

// LDS tiles are [rows][64 bf16] = 8 chunks of 16 bytes per row.  The LDS
// has 64 banks (256 bytes) and serves a 16-byte read for 16 lanes at once,
// i.e. 16 consecutive tile rows at one logical chunk; chunk c of row r is
// stored at slot c ^ ((r >> 1) & 7), which puts those 16 rows on 16
// different 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float silu_fast(float g) {
  // g * sigmoid(g) with the hardware exp2 and reciprocal
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// One BM x BN output tile of group g (rows [row0, row0+rows), n-tile by),
// staged through the caller's LDS arrays (at least BM and BN rows a stage).
template <int EPI, int BM, int BN, int WGM, int WGN, int SAN, int SBN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int g, int row0, int rows, int by,
                                          u32x4 (&sA)[2][SAN], u32x4 (&sB)[2][SBN]) {
  constexpr int NW = WGM * WGN;                   // waves
  constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;     // 32x32 accumulators per wave
  constexpr int AI = BM / 8 / NW, BI = BN / 8 / NW;   // 1-KB direct loads per wave per stage
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(AI >= 1 && BI >= 1, "every wave loads A and B rows");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  static_assert(SAN >= BM * 8 && SBN >= BN * 8, "LDS stages hold the tile");
  constexpr int BNH = EPI == EPI_SWIGLU ? BN / 2 : BN;   // output columns per tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  // the tile coordinates are block-uniform; saying so keeps the buffer
  // descriptors built from them in scalar registers
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  by = __builtin_amdgcn_readfirstlane(by);
  const int wm = wave / WGN, wn = wave % WGN;
  const int n0 = by * BNH;

  // Direct loads: load i of this wave fills tile rows R0 .. R0+8 with
  // R0 = 8q, q = wave*AI + i (1 KB of LDS); lane l writes slot l%8 of row
  // R0 + l/8, which holds logical chunk (l%8) ^ ((R0 + l/8) >> 1 & 7)
  // = (l%8) ^ (4*(q&1) + l/16): one lane mapping for even q, one for odd.
  const int lrow = lane >> 3;
  const int lchunk_even = (lane & 7) ^ (lrow >> 1);
  const int lchunk_odd = (lane & 7) ^ (4 + (lrow >> 1));
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(static_cast<const uint16_t*>(a.A) + (size_t)row0 * a.lda, (uint32_t)rows * a.lda * 2);
  // instruction i of this wave covers q = wave*AI + i
  const uint32_t a_voff_e = (uint32_t)((wave * AI * 8 + lrow) * a.lda + lchunk_even * 8) * 2;
  const uint32_t a_voff_o = (uint32_t)((wave * AI * 8 + lrow) * a.lda + lchunk_odd * 8) * 2;
  const uint32_t a_step = 8u * a.lda * 2;

  // B rows of this wave: [wave*BN/NW, +BN/NW) of the tile.  SwiGLU: the
  // first half of the waves load gate rows, the second half the up rows of
  // the same columns.
  const uint16_t* Bsrc = static_cast<const uint16_t*>(a.B0) + (size_t)g * a.b_group_stride;
  int b_local0 = wave * (BN / NW);
  if constexpr (EPI == EPI_SWIGLU) {
    if (wave >= NW / 2) {
      Bsrc = static_cast<const uint16_t*>(a.B1) + (size_t)g * a.b_group_stride;
      b_local0 -= BN / 2;
    }
  }
  Bsrc += (size_t)n0 * a.ldb;
  const int b_valid = a.Ndim - n0 < BNH ? a.Ndim - n0 : BNH;
  const uint32_t b_bytes = (uint32_t)b_valid * a.ldb * 2;
  const uint32_t b_voff_e = (uint32_t)((b_local0 + lrow) * a.ldb + lchunk_even * 8) * 2;
  const uint32_t b_voff_o = (uint32_t)((b_local0 + lrow) * a.ldb + lchunk_odd * 8) * 2;
  const uint32_t b_step = 8u * a.ldb * 2;

  lds_t* ldsA[2] = {(lds_t*)&sA[0][wave * AI * 64], (lds_t*)&sA[1][wave * AI * 64]};
  lds_t* ldsB[2] = {(lds_t*)&sB[0][wave * BI * 64], (lds_t*)&sB[1][wave * BI * 64]};

  auto issue = [&](int kt, int buf) {
    const int kb = kt * BK;
    const int seg = kb / a.kseg;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bsrc + (size_t)seg * a.kseg_stride, b_bytes);
    const uint32_t ka = (uint32_t)kb * 2, kbb = (uint32_t)(kb - seg * a.kseg) * 2;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const bool odd = ((wave * AI + i) & 1) != 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_t*)((char*)ldsA[buf] + i * 1024), 16,
                                               (odd ? a_voff_o : a_voff_e) + i * a_step + ka, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const bool odd = ((wave * BI + i) & 1) != 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_t*)((char*)ldsB[buf] + i * 1024), 16,
                                               (odd ? b_voff_o : b_voff_e) + i * b_step + kbb, 0, 0, 0);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // first row of each n-tile of this wave inside the B tile
  auto brow = [&](int j) {
    if constexpr (EPI == EPI_SWIGLU)
      return j < TN / 2 ? wn * (WTN / 2) + 32 * j : BN / 2 + wn * (WTN / 2) + 32 * (j - TN / 2);
    else
      return wn * WTN + 32 * j;
  };

  const int nk = a.Kdim / BK;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
    // operand fragments of k-step kk+1 are read while k-step kk multiplies
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[0][i] = __builtin_bit_cast(bf16x8, sA[buf][swz(wm * WTM + i * 32 + (lane & 31), (lane >> 5))]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[0][j] = __builtin_bit_cast(bf16x8, sB[buf][swz(brow(j) + (lane & 31), (lane >> 5))]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
        const int c = (kk + 1) * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[cur ^ 1][i] = __builtin_bit_cast(bf16x8, sA[buf][swz(wm * WTM + i * 32 + (lane & 31), c)]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[cur ^ 1][j] = __builtin_bit_cast(bf16x8, sB[buf][swz(brow(j) + (lane & 31), c)]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // epilogue: lane holds column lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4
  uint16_t* C = static_cast<uint16_t*>(a.C);
  constexpr int OUT_TN = EPI == EPI_SWIGLU ? TN / 2 : TN;
  const int col_base = n0 + (EPI == EPI_SWIGLU ? wn * (WTN / 2) : wn * WTN) + (lane & 31);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < OUT_TN; ++j) {
      const int col = col_base + 32 * j;
      if (col >= a.Ndim) continue;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        f32x2 pr;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float x = acc[i][j][v + q];
          if constexpr (EPI == EPI_SWIGLU) pr[q] = silu_fast(x) * acc[i][j + TN / 2][v + q];
          else if constexpr (EPI == EPI_RELU) pr[q] = x > 0.0f ? x : 0.0f;
          else pr[q] = x;
        }
        const uint32_t packed = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = wm * WTM + i * 32 + 8 * ((v + q) >> 2) + 4 * (lane >> 5) + ((v + q) & 3);
          if (r < rows)
            C[(size_t)(row0 + r) * a.ldc + col] = (uint16_t)(q ? packed >> 16 : packed & 0xffffu);
        }
      }
    }
  }
}

// Groups of many rows: 256x256 tiles on 8 waves (128x64 each).  A group's
// last tile grows to 320 rows (160x64 per wave) when the group ends at most
// 64 rows past a multiple of 256, and groups of at most 64 rows get a 64-row
// tail tile (32x64 per wave).
constexpr int kTailRows = 64;
constexpr int kExtRows = 64;

template <int EPI>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][(256 + kExtRows) * 8];
  __shared__ u32x4 sB[2][256 * 8];
  constexpr int BNH = EPI == EPI_SWIGLU ? 128 : 256;
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, 256) * ntiles;
  const int h = blockIdx.x;
  int g, row0, rows, by;
  if (h < real) {
    find_tile_2d(a, 256, ntiles, h, real, g, row0, rows, by);
    if (rows > 256) gemm_tile<EPI, 256 + kExtRows, 256, 2, 4>(a, g, row0, rows, by, sA, sB);
    else gemm_tile<EPI, 256, 256, 2, 4>(a, g, row0, rows, by, sA, sB);
  } else if (find_tail(a, 256, ntiles, h - real, g, row0, rows, by)) {
    gemm_tile<EPI, kTailRows, 256, 2, 4>(a, g, row0, rows, by, sA, sB);
  }
}

// Groups of a few rows (decode-sized batches): 32x256 tiles on 4 waves.
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_small_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][32 * 8];
  __shared__ u32x4 sB[2][256 * 8];
  constexpr int BNH = EPI == EPI_SWIGLU ? 128 : 256;
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, 32) * ntiles;
  const int h = blockIdx.x;
  if (h >= real) return;
  int g, row0, rows, by;
  find_tile_2d(a, 32, ntiles, h, real, g, row0, rows, by);
  gemm_tile<EPI, 32, 256, 1, 4>(a, g, row0, rows, by, sA, sB);
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

// Prefix sums over the groups of their full-height and tail row tiles
// (split_rows), one block: tiles[g], tails[g] for g = 0..G.
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t* offsets, int G, int BMr,
                                                        int tail_rows, int ext_rows,
                                                        int32_t* tiles, int32_t* tails) {
  __shared__ int32_t s[256], t[256];
  const int g = threadIdx.x;
  int f = 0, tl = 0;
  if (g < G) split_rows(offsets[g + 1] - offsets[g], BMr, tail_rows, ext_rows, f, tl);
  s[g] = f;
  t[g] = tl;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = g >= o ? s[g - o] : 0;
    const int w = g >= o ? t[g - o] : 0;
    __syncthreads();
    s[g] += v;
    t[g] += w;
    __syncthreads();
  }
  if (g < G) {
    tiles[g + 1] = s[g];
    tails[g + 1] = t[g];
  }
  if (g == 0) {
    tiles[0] = 0;
    tails[0] = 0;
  }
}

// Tile shape per problem: large groups use 256x256 tiles (8 waves of
// 128x64); groups of a few rows (decode-sized batches) use 32-row tiles so the
// matrix cores do not multiply mostly-empty rows.
struct TileShape { int bm; };

TileShape pick_tiles(int rows_per_group) { return TileShape{rows_per_group >= 128 ? 256 : 32}; }

template <int EPI>
hipError_t launch_bf16(const GemmArgs& a, int bm, int mtiles, hipStream_t s) {
  constexpr int BNH = EPI == EPI_SWIGLU ? 128 : 256;
  dim3 grid(mtiles * ((a.Ndim + BNH - 1) / BNH));
  if (bm == 256)
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<EPI>, grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16_small_kernel<EPI>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t run_gemm(const GemmArgs& a, int epi, bool bf16, int bm, int mtiles, hipStream_t s) {
  if (bf16) {
    switch (epi) {
      case EPI_SWIGLU: return launch_bf16<EPI_SWIGLU>(a, bm, mtiles, s);
      case EPI_RELU: return launch_bf16<EPI_RELU>(a, bm, mtiles, s);
      default: return launch_bf16<EPI_NONE>(a, bm, mtiles, s);
    }
  }
  dim3 grid(mtiles, (a.Ndim + 255) / 256);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, a, bm);
      break;
    case EPI_RELU:
      hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_RELU>, grid, dim3(256), 0, s, a, bm);
      break;
    default:
      hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI_NONE>, grid, dim3(256), 0, s, a, bm);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_ffn(const moe_problem_t& p, int rows_alloc, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, const void* u, const void* ws_gate,
                              const void* ws_up, const void* ws_down, void* y_perm,
                              void* y_shared, int32_t* tiles, void* act, void* act_shared,
                              hipStream_t s) {
  const bool bf16 = p.dtype == MOE_BF16;
  const int epi1 = p.act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_RELU;
  // fp32 problems: one block per 128 rows; bf16: tiles sized to the mean
  // group (all groups share one tile height so the plan is one prefix sum)
  const int bm = bf16 ? pick_tiles(rows_alloc / p.N).bm : 128;
  const int tail_rows = bf16 && bm == 256 ? kTailRows : 0;
  const int ext_rows = bf16 && bm == 256 ? kExtRows : 0;
  // grid bound: at most rows/bm + 1 full tiles and one tail tile per group
  const int mtiles_max = (rows_alloc + bm - 1) / bm + p.N + (tail_rows > 0 ? p.N : 0);
  int32_t* tails = tiles + (p.N + 2);

  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, offsets, p.N, bm, tail_rows,
                     ext_rows, tiles, tails);
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
  g1.tails = tails;
  g1.tail_rows = tail_rows;
  g1.ext_rows = ext_rows;
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
  if ((e = run_gemm(g1, epi1, bf16, bm, mtiles_max, s)) != hipSuccess) return e;

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
  if ((e = run_gemm(g2, EPI_NONE, bf16, bm, mtiles_max, s)) != hipSuccess) return e;

  if (p.n_shared > 0) {
    // all shared experts as one expert of width n_shared*d_ff_shared: the
    // gate/up rows of consecutive experts are contiguous; the down
    // projection is K-segmented, one segment per shared expert
    const int ws_w = p.n_shared * p.d_ff_shared;
    const int sbm = bf16 ? pick_tiles(p.T).bm : 128;
    const int s_tail = bf16 && sbm == 256 ? kTailRows : 0;
    const int s_ext = bf16 && sbm == 256 ? kExtRows : 0;
    int mt = (p.T + sbm - 1) / sbm;
    if (s_tail > 0) {
      int f, t;
      split_rows(p.T, sbm, s_tail, s_ext, f, t);
      mt = f + t;
    }
    GemmArgs s1{};
    s1.A = u;
    s1.B0 = ws_gate;
    s1.B1 = ws_up;
    s1.C = act_shared;
    s1.offsets = nullptr;
    s1.tiles = nullptr;
    s1.tails = nullptr;
    s1.tail_rows = s_tail;
    s1.ext_rows = s_ext;
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
    if ((e = run_gemm(s1, epi1, bf16, sbm, mt, s)) != hipSuccess) return e;
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
    if ((e = run_gemm(s2, EPI_NONE, bf16, sbm, mt, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
