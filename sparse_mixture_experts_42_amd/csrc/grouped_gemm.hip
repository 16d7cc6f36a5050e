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

// Epilogues.  The two backward ones run on the recomputed gate (and up)
// accumulators of GEMM-1 with the activation gradient dA = dY W_down as the
// extra input D: they write the activation a (to C, for dW_down) and the
// pre-activation gradients (to C2, [rows][2*Ndim]: dG then dU; ReLU: dG).
enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3, EPI_RELU_BWD = 4 };

template <int EPI>
constexpr bool gated() { return EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD; }

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
  // backward epilogues: D = dA [rows][ldd]; C2 = pre-activation gradients
  const void* D;
  int ldd;
  void* C2;
  int ldc2;
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
// The row tiles of patch nb are taken in an order rotated by nb: a block at
// a given position of successive patches tends to land on the same CU (the
// CUs finish their tiles in the same order), and without the rotation the
// same few CUs would draw every group's taller last tile.
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
  const int mt = (rem / nbe + nb) % mt_g;
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

__device__ __forceinline__ float sigmoid_fast(float g) {
  // 1 / (1 + e^-g) with the hardware exp2 and reciprocal
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

__device__ __forceinline__ float silu_fast(float g) { return g * sigmoid_fast(g); }

// ---------------------------------------------------- k-major operands
// The backward GEMMs read operands whose reduction index k is the row index
// of a row-major array (W_down as [d][d_ff] for dY W_down, the stacked
// [W_gate; W_up] for dGU W, and every operand of the weight gradients,
// which reduce over the rows of a group).  Such a tile, 64 k-rows x 256
// columns (512 bytes a row), is loaded row by row into LDS and transposed
// on the way to the matrix cores by ds_read_b64_tr_b16.
//
// LDS layout: 16-byte chunk c of tile row r sits at slot c ^ 4*(r%4).  A
// transposing read fetches, per 16 lanes, 8 bytes from 4 consecutive rows
// at 4 consecutive 8-byte positions; with the XOR the 32 lanes of each half
// wave hit 16 different 16-byte bank groups.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// voffset (bytes, from the tile's first row and column) of direct load q of
// a k-major tile: the instruction fills LDS rows 2q and 2q+1; lane l writes
// slot l%32 of row 2q + l/32, which holds chunk (l%32) ^ 4*(row%4).
__host__ __device__ inline uint32_t kmajor_voff(int q, int lane, int ld) {
  const int r = 2 * q + (lane >> 5);
  const int c = (lane & 31) ^ (4 * (r & 3));
  return (uint32_t)(r * ld + c * 8) * 2u;
}

// MFMA operand of a k-major LDS tile: lane l gets column col0 + l%32 at the
// eight k = 16*kk + 8*(l/32) .. +7.  Each 16-lane group of a transposing
// read hands lane i element i%4 of the 8 bytes that lane 4j + i/4 of the
// group addressed (as its j-th element), so lane s of a group addresses row
// k0 + s/4, columns 4*(s%4) .. +3 past the group's first column.
__host__ __device__ inline int kmajor_read_off(int kk, int col0, int lane) {
  const int s = lane & 15;
  const int row = 16 * kk + 8 * (lane >> 5) + (s >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  return row * 512 + (((col >> 3) ^ (4 * (row & 3))) << 4) + ((col >> 2) & 1) * 8;
}

__device__ __forceinline__ bf16x8 read_kmajor(const char* tile, int kk, int col0, int lane) {
  const int off = kmajor_read_off(kk, col0, lane);
  // the second read is 4 rows further: same row%4, hence the same slot
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + off + 4 * 512));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}


// One BM x BN output tile of group g (rows [row0, row0+rows), n-tile by),
// staged through the caller's LDS arrays (at least BM and BN rows a stage).
//
// BT: B is k-major (B[k][n] row-major, n contiguous; see above) instead of
// [n][k]; only with EPI_NONE and BN = 256.  PIPE: the software-pipelined
// main loop (256-column tiles); otherwise a plain double-buffered loop.
template <int EPI, int BM, int BN, int WGM, int WGN, int SAN, int SBN, bool BT = false, bool PIPE = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int g, int row0, int rows, int by,
                                          u32x4 (&sA)[2][SAN], u32x4 (&sB)[2][SBN]) {
  constexpr int NW = WGM * WGN;                   // waves
  constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;     // 32x32 accumulators per wave
  constexpr bool GATED = gated<EPI>();
  // 1-KB direct loads per wave per stage
  constexpr int AI = BM / 8 / NW, BI = BT ? 32 / NW : BN / 8 / NW;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(AI >= 1 && BI >= 1, "every wave loads A and B rows");
  static_assert(!GATED || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  static_assert(SAN >= BM * 8 && SBN >= BN * 8, "LDS stages hold the tile");
  static_assert(!BT || (EPI == EPI_NONE && BN == 256), "k-major B: plain epilogue, 256 columns");
  constexpr int BNH = GATED ? BN / 2 : BN;        // output columns per tile

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
  if constexpr (GATED) {
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
    const uint32_t ka = (uint32_t)kb * 2, kbb = (uint32_t)(kb - seg * a.kseg) * 2;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const bool odd = ((wave * AI + i) & 1) != 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_t*)((char*)ldsA[buf] + i * 1024), 16,
                                               (odd ? a_voff_o : a_voff_e) + i * a_step + ka, 0, 0, 0);
    }
    if constexpr (BT) {
      // k-major B: segment 0 from B0, segment 1 from B1; rows of the
      // segment, columns n0 .. n0+255
      const uint16_t* base = static_cast<const uint16_t*>(seg == 0 ? a.B0 : a.B1) +
                             (size_t)g * a.b_group_stride + n0;
      const __amdgpu_buffer_rsrc_t rBT =
          make_rsrc(base, (uint32_t)((size_t)a.kseg * a.ldb - n0) * 2u);
      const uint32_t krow = (uint32_t)(kb - seg * a.kseg) * (uint32_t)a.ldb * 2u;
#pragma unroll
      for (int i = 0; i < BI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rBT, (lds_t*)((char*)ldsB[buf] + i * 1024), 16,
                                                 kmajor_voff(wave * BI + i, lane, a.ldb) + krow,
                                                 0, 0, 0);
      return;
    }
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bsrc + (size_t)seg * a.kseg_stride, b_bytes);
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
    if constexpr (GATED)
      return j < TN / 2 ? wn * (WTN / 2) + 32 * j : BN / 2 + wn * (WTN / 2) + 32 * (j - TN / 2);
    else
      return wn * WTN + 32 * j;
  };

  const int nk = a.Kdim / BK;
  if constexpr (PIPE) {
    static_assert(BN == 256, "pipelined tile: 256 columns");
    // Software pipeline with a fixed instruction order.  Fragments of
    // k-step kk+1 are read between the matrix instructions of k-step kk, in
    // the order the matrix instructions consume them.  The stage barrier
    // sits in the middle of k-step 3: the first half of its matrix
    // instructions runs before it, the second half after it, while the next
    // stage's first fragments are read.  From that barrier on, the buffer of
    // the stage just finished is free, so the loads of the stage after next
    // start at once and continue through k-steps 0 and 1, one per two matrix
    // instructions per wave: a burst of them would stall the wave's issue
    // (the load path takes about one 1-KB load per 16 cycles per CU).
    // Every K-segment length is a multiple of BK, so the segment of a stage
    // advances without a division.  The loads issued during the last stage
    // get an empty buffer range: they read nothing, and their LDS buffer is
    // never read.
    constexpr int NL = AI + BI;                       // loads per wave per stage
    const uint32_t a_bytes = (uint32_t)rows * a.lda * 2;
    const void* a_base = static_cast<const uint16_t*>(a.A) + (size_t)row0 * a.lda;
    int seg_n = 0, koff_n = 0;                        // segment and offset of the stage to load
    auto issue_part = [&](int kt_n, bool live, int buf, int lo, int hi) {
      const __amdgpu_buffer_rsrc_t rAx = make_rsrc(a_base, live ? a_bytes : 0u);
      const uint32_t ka = (uint32_t)kt_n * BK * 2;
#pragma unroll
      for (int i = 0; i < AI; ++i) {
        if (i < lo || i >= hi) continue;
        const bool odd = ((wave * AI + i) & 1) != 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rAx, (lds_t*)((char*)ldsA[buf] + i * 1024), 16,
                                                 (odd ? a_voff_o : a_voff_e) + i * a_step + ka, 0, 0, 0);
      }
      if constexpr (BT) {
        const uint16_t* base = static_cast<const uint16_t*>(seg_n == 0 ? a.B0 : a.B1) +
                               (size_t)g * a.b_group_stride + n0;
        const __amdgpu_buffer_rsrc_t rBT =
            make_rsrc(base, live ? (uint32_t)((size_t)a.kseg * a.ldb - n0) * 2u : 0u);
        const uint32_t krow = (uint32_t)koff_n * (uint32_t)a.ldb * 2u;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          if (AI + i < lo || AI + i >= hi) continue;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rBT, (lds_t*)((char*)ldsB[buf] + i * 1024), 16,
                                                   kmajor_voff(wave * BI + i, lane, a.ldb) + krow,
                                                   0, 0, 0);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rBx =
            make_rsrc(Bsrc + (size_t)seg_n * a.kseg_stride, live ? b_bytes : 0u);
        const uint32_t kbb = (uint32_t)koff_n * 2;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          if (AI + i < lo || AI + i >= hi) continue;
          const bool odd = ((wave * BI + i) & 1) != 0;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rBx, (lds_t*)((char*)ldsB[buf] + i * 1024), 16,
                                                   (odd ? b_voff_o : b_voff_e) + i * b_step + kbb, 0, 0, 0);
        }
      }
    };
    auto advance = [&]() {
      koff_n += BK;
      if (koff_n == a.kseg) { koff_n = 0; ++seg_n; }
    };
    auto read_frags = [&](bf16x8 (&fa_)[TM], bf16x8 (&fb_)[TN], int buf, int kk) {
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa_[i] = __builtin_bit_cast(bf16x8, sA[buf][swz(wm * WTM + i * 32 + (lane & 31), c)]);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BT) fb_[j] = read_kmajor((const char*)&sB[buf][0], kk, brow(j), lane);
        else fb_[j] = __builtin_bit_cast(bf16x8, sB[buf][swz(brow(j) + (lane & 31), c)]);
      }
    };
    // Fragment r of a k-step, in the order the matrix instructions of row
    // 0 need them first: A row 0, the B columns, then A rows 1.. .
    auto read_one = [&](bf16x8 (&ra)[TM], bf16x8 (&rb)[TN], int rbuf, int rkk, int r) {
      const int c = rkk * 2 + (lane >> 5);
      const int ia = r == 0 ? 0 : (r <= TN ? -1 : r - TN);
      if (ia >= 0) {
        ra[ia] = __builtin_bit_cast(bf16x8, sA[rbuf][swz(wm * WTM + ia * 32 + (lane & 31), c)]);
      } else {
        const int jj = r - 1;
        if constexpr (BT) rb[jj] = read_kmajor((const char*)&sB[rbuf][0], rkk, brow(jj), lane);
        else rb[jj] = __builtin_bit_cast(bf16x8, sB[rbuf][swz(brow(jj) + (lane & 31), c)]);
      }
    };
    // One k-step in a fixed order: matrix instruction s is followed by
    // fragment read s / RS of the next k-step when s % RS == 0, and by load
    // l0 + s / 2 of the next stage when s is odd; each step is fenced so the
    // compiler keeps the order.
    auto kstep = [&](const bf16x8 (&fa_)[TM], const bf16x8 (&fb_)[TN], int i0, int i1,
                     bf16x8 (&ra)[TM], bf16x8 (&rb)[TN], int rbuf, int rkk, bool rd, int RS,
                     int kt_n, bool live, int lbuf, int l0, int l1) {
      int s = 0;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i < i0 || i >= i1) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_[i], fb_[j], acc[i][j], 0, 0, 0);
          if (rd && s % RS == 0 && s / RS < TM + TN) read_one(ra, rb, rbuf, rkk, s / RS);
          if ((s & 1) && l0 + s / 2 < l1) issue_part(kt_n, live, lbuf, l0 + s / 2, l0 + s / 2 + 1);
          __builtin_amdgcn_sched_barrier(0);
          ++s;
        }
      }
      // reads or loads left over when the k-step has fewer instructions
#pragma unroll
      for (int t = 0; t < TM + TN; ++t)
        if (rd && t * RS >= s) read_one(ra, rb, rbuf, rkk, t);
#pragma unroll
      for (int t = 0; t < NL; ++t)
        if (l0 + t < l1 && 2 * t + 1 >= s) issue_part(kt_n, live, lbuf, l0 + t, l0 + t + 1);
    };
    constexpr int H = TM / 2;
    bf16x8 fa[2][TM], fb[2][TN];
    issue_part(0, true, 0, 0, NL);
    advance();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    read_frags(fa[0], fb[0], 0, 0);
    // k-steps 0, 1, 2 and the first half of 3 of stage kt; loads l0.. of
    // stage kt+1 are issued during k-steps 0 and 1 (the first ones already
    // went out after the previous barrier)
    auto body = [&](int kt, int l0) {
      const int buf = kt & 1;
      const bool live = kt + 1 < nk;
      const int lm = l0 + TM * TN / 2 < NL ? l0 + TM * TN / 2 : NL;
      kstep(fa[0], fb[0], 0, TM, fa[1], fb[1], buf, 1, true, 2, kt + 1, live, buf ^ 1, l0, lm);
      kstep(fa[1], fb[1], 0, TM, fa[0], fb[0], buf, 2, true, 2, kt + 1, live, buf ^ 1, lm, NL);
      kstep(fa[0], fb[0], 0, TM, fa[1], fb[1], buf, 3, true, 2, 0, false, 0, 0, 0);
      kstep(fa[1], fb[1], 0, H, fa[0], fb[0], 0, 0, false, 1, 0, false, 0, 0, 0);
      advance();
    };
    // loads issued during the second half of k-step 3 (one per two matrix
    // instructions)
    constexpr int LB = (TM - H) * TN / 2 < NL ? (TM - H) * TN / 2 : NL;
    body(0, 0);
    // The loop starts at the stage barrier, where every wait has drained,
    // so the waits on the fragment reads after it stay exact.  The buffer
    // of stage kt-1 is free from here on, so the loads of stage kt+1 start
    // at once.
    for (int kt = 1; kt < nk; ++kt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // second half of k-step 3 of stage kt-1, reading the first
      // fragments of stage kt
      kstep(fa[1], fb[1], H, TM, fa[0], fb[0], kt & 1, 0, true, 1, kt + 1, kt + 1 < nk, (kt + 1) & 1, 0, LB);
      body(kt, LB);
    }
    kstep(fa[1], fb[1], H, TM, fa[0], fb[0], 0, 0, false, 1, 0, false, 0, 0, 0);
    // the empty loads of the last stage still write the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  } else {
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
    for (int j = 0; j < TN; ++j) {
      if constexpr (BT) fb[0][j] = read_kmajor((const char*)&sB[buf][0], 0, brow(j), lane);
      else fb[0][j] = __builtin_bit_cast(bf16x8, sB[buf][swz(brow(j) + (lane & 31), (lane >> 5))]);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
        const int c = (kk + 1) * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[cur ^ 1][i] = __builtin_bit_cast(bf16x8, sA[buf][swz(wm * WTM + i * 32 + (lane & 31), c)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (BT) fb[cur ^ 1][j] = read_kmajor((const char*)&sB[buf][0], kk + 1, brow(j), lane);
          else fb[cur ^ 1][j] = __builtin_bit_cast(bf16x8, sB[buf][swz(brow(j) + (lane & 31), c)]);
        }
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

  }

  // epilogue: lane holds column lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4
  uint16_t* C = static_cast<uint16_t*>(a.C);
  constexpr int OUT_TN = GATED ? TN / 2 : TN;
  const int col_base = n0 + (GATED ? wn * (WTN / 2) : wn * WTN) + (lane & 31);
  if constexpr (PIPE && EPI == EPI_SWIGLU_BWD) {
    // Backward epilogue.  The dA tile is staged in LDS as bf16 [BM][128] by
    // direct loads.  Neighbouring lanes swap one value of each accumulator
    // pair in place, so that each lane holds two adjacent columns of one
    // row (the even lane row r, the odd lane row r+1), and read the matching
    // dA pair as one 4-byte word.  a, dG and dU then go out as bf16 pairs.
    // 16-byte chunk c of staged row r sits at slot c ^ 4*(r%2 + 2*(r/4 %2)),
    // which keeps the pair reads of one instruction (rows r, r+1, r+4, r+5)
    // on disjoint banks.
    static_assert(BM * 256 <= 2 * SAN * 16, "staged tile fits the A stages");
    static_assert(OUT_TN == 1, "one 32-column output block per wave");
    uint32_t* st = reinterpret_cast<uint32_t*>(&sA[0][0]);
    u32x4* stv = &sA[0][0];
    auto slot = [](int r, int c) { return c ^ (((r & 1) | ((r >> 1) & 2)) << 2); };
    const uint16_t* D = static_cast<const uint16_t*>(a.D);
    uint16_t* C2 = static_cast<uint16_t*>(a.C2);
    const int wcol = wn * (WTN / 2);                    // first output column of the wave
    const bool odd = (lane & 1) != 0;
    auto pair_row = [&](int i, int v) { return wm * WTM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3) + (odd ? 1 : 0); };
    const int pc = wcol + (lane & 31) - (odd ? 1 : 0);  // the lane's (even) first column
    __syncthreads();               // the loop's LDS reads are done
    {
      // direct loads of the dA tile: load q of the wave fills staged rows
      // 4q' .. 4q'+3 (q' = wave*DQ + q), lane l row 4q' + l/16 at slot l%16,
      // which holds chunk (l%16) ^ slot-XOR of that row; rows past the
      // group read 0 through the descriptor's size
      constexpr int DQ = BM / 4 / NW;
      static_assert(DQ * 4 * NW == BM, "whole rows per wave");
      const __amdgpu_buffer_rsrc_t rD = make_rsrc(D + (size_t)row0 * a.ldd, (uint32_t)rows * a.ldd * 2u);
#pragma unroll
      for (int q = 0; q < DQ; ++q) {
        const int r = (wave * DQ + q) * 4 + (lane >> 4);
        const int ch = slot(r, lane & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (lds_t*)&stv[(wave * DQ + q) * 64], 16,
                                                 (uint32_t)(r * a.ldd + n0 + 8 * ch) * 2u, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int j = jj * (TN / 2);                   // gate block, then up block
          const float got = __shfl_xor(odd ? acc[i][j][v] : acc[i][j][v + 1], 1);
          const float x0 = acc[i][j][v], x1 = acc[i][j][v + 1];
          acc[i][j][v] = odd ? got : x0;
          acc[i][j][v + 1] = odd ? x1 : got;
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t dap[TM * 8];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int r = pair_row(i, v);
        dap[i * 8 + v / 2] = st[r * 64 + slot(r, pc >> 3) * 4 + ((pc >> 1) & 3)];
      }
    // a, dG and dU straight to global memory as bf16 pairs (4 bytes a lane),
    // through buffer descriptors over the tile's rows: stores to rows past
    // the group fall outside them and are dropped
    const uint32_t lane_row = (uint32_t)(wm * WTM + 4 * (lane >> 5) + (odd ? 1 : 0));
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(C + (size_t)row0 * a.ldc + n0, (uint32_t)((size_t)rows * a.ldc * 2 - (size_t)n0 * 2));
    const __amdgpu_buffer_rsrc_t rG =
        make_rsrc(C2 + (size_t)row0 * a.ldc2 + n0, (uint32_t)((size_t)rows * a.ldc2 * 2 - (size_t)n0 * 2));
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(C2 + (size_t)row0 * a.ldc2 + a.Ndim + n0,
                                                (uint32_t)((size_t)rows * a.ldc2 * 2 - (size_t)(a.Ndim + n0) * 2));
    const bool col_ok = n0 + pc < a.Ndim;
    const uint32_t vC = (lane_row * a.ldc + pc) * 2u, vG = (lane_row * a.ldc2 + pc) * 2u;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const uint32_t dp = dap[i * 8 + v / 2];
        f32x2 pa, pg, pu;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float gv = acc[i][0][v + q], uv = acc[i][TN / 2][v + q];
          const float sg = sigmoid_fast(gv);
          const float sl = gv * sg;
          const float da = __builtin_bit_cast(float, q ? (dp & 0xffff0000u) : (dp << 16));
          pa[q] = sl * uv;
          pg[q] = da * uv * sg * (1.0f + gv * (1.0f - sg));
          pu[q] = da * sl;
        }
        if (!col_ok) continue;
        const int rr = 32 * i + 8 * (v >> 2) + (v & 3);   // uniform part of the row
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, __builtin_convertvector(pa, bf16x2)),
                                              rC, vC, rr * a.ldc * 2, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, __builtin_convertvector(pg, bf16x2)),
                                              rG, vG, rr * a.ldc2 * 2, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, __builtin_convertvector(pu, bf16x2)),
                                              rU, vG, rr * a.ldc2 * 2, 0);
      }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU_BWD || EPI == EPI_RELU_BWD) {
    // a = act(g[, v]) to C; dG (and dU) from dA to C2
    const uint16_t* D = static_cast<const uint16_t*>(a.D);
    uint16_t* C2 = static_cast<uint16_t*>(a.C2);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < OUT_TN; ++j) {
        const int col = col_base + 32 * j;
        if (col >= a.Ndim) continue;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          f32x2 pa, pg, pu;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int r = wm * WTM + i * 32 + 8 * ((v + q) >> 2) + 4 * (lane >> 5) + ((v + q) & 3);
            const float da = r < rows ? bf16_to_f32(D[(size_t)(row0 + r) * a.ldd + col]) : 0.0f;
            const float gv = acc[i][j][v + q];
            if constexpr (EPI == EPI_SWIGLU_BWD) {
              const float up = acc[i][j + TN / 2][v + q];
              const float sg = sigmoid_fast(gv);
              const float sl = gv * sg;
              pa[q] = sl * up;
              pg[q] = da * up * sg * (1.0f + gv * (1.0f - sg));
              pu[q] = da * sl;
            } else {
              pa[q] = gv > 0.0f ? gv : 0.0f;
              pg[q] = gv > 0.0f ? da : 0.0f;
              pu[q] = 0.0f;
            }
          }
          const uint32_t qa = __builtin_bit_cast(uint32_t, __builtin_convertvector(pa, bf16x2));
          const uint32_t qg = __builtin_bit_cast(uint32_t, __builtin_convertvector(pg, bf16x2));
          const uint32_t qu = __builtin_bit_cast(uint32_t, __builtin_convertvector(pu, bf16x2));
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int r = wm * WTM + i * 32 + 8 * ((v + q) >> 2) + 4 * (lane >> 5) + ((v + q) & 3);
            if (r >= rows) continue;
            const size_t row = (size_t)(row0 + r);
            C[row * a.ldc + col] = (uint16_t)(q ? qa >> 16 : qa & 0xffffu);
            C2[row * a.ldc2 + col] = (uint16_t)(q ? qg >> 16 : qg & 0xffffu);
            if constexpr (EPI == EPI_SWIGLU_BWD)
              C2[row * a.ldc2 + a.Ndim + col] = (uint16_t)(q ? qu >> 16 : qu & 0xffffu);
          }
        }
      }
    }
    return;
  }
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

template <int EPI, bool BT = false>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][(256 + kExtRows) * 8];
  __shared__ u32x4 sB[2][256 * 8];
  constexpr int BNH = gated<EPI>() ? 128 : 256;
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, 256) * ntiles;
  const int h = blockIdx.x;
  int g, row0, rows, by;
  if (h < real) {
    find_tile_2d(a, 256, ntiles, h, real, g, row0, rows, by);
    if (rows > 256) gemm_tile<EPI, 256 + kExtRows, 256, 2, 4, (256 + kExtRows) * 8, 256 * 8, BT, true>(a, g, row0, rows, by, sA, sB);
    else gemm_tile<EPI, 256, 256, 2, 4, (256 + kExtRows) * 8, 256 * 8, BT, true>(a, g, row0, rows, by, sA, sB);
  } else if (find_tail(a, 256, ntiles, h - real, g, row0, rows, by)) {
    gemm_tile<EPI, kTailRows, 256, 2, 4, (256 + kExtRows) * 8, 256 * 8, BT, true>(a, g, row0, rows, by, sA, sB);
  }
}

// Groups of a few rows (decode-sized batches): 32x256 tiles on 4 waves.
template <int EPI, bool BT = false>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_small_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][32 * 8];
  __shared__ u32x4 sB[2][256 * 8];
  constexpr int BNH = gated<EPI>() ? 128 : 256;
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, 32) * ntiles;
  const int h = blockIdx.x;
  if (h >= real) return;
  int g, row0, rows, by;
  find_tile_2d(a, 32, ntiles, h, real, g, row0, rows, by);
  gemm_tile<EPI, 32, 256, 1, 4, 32 * 8, 256 * 8, BT>(a, g, row0, rows, by, sA, sB);
}

// Groups of a few hundred rows (e.g. a Switch-shaped layer with capacity
// 640): 128x256 tiles on 8 waves of 64x64, so a narrow output (few column
// tiles) still spreads over more CUs than 256-row tiles would.
template <int EPI, bool BT = false>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_mid_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][128 * 8];
  __shared__ u32x4 sB[2][256 * 8];
  constexpr int BNH = gated<EPI>() ? 128 : 256;
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, 128) * ntiles;
  const int h = blockIdx.x;
  if (h >= real) return;
  int g, row0, rows, by;
  find_tile_2d(a, 128, ntiles, h, real, g, row0, rows, by);
  gemm_tile<EPI, 128, 256, 2, 4, 128 * 8, 256 * 8, BT, true>(a, g, row0, rows, by, sA, sB);
}

// The plain down projection of mid-sized groups: the 128-row tiles of the
// plan, 128 columns wide, each split into two 64-row blocks on 8 waves of
// 32x32 (the unpipelined tile body).  An output with few column tiles
// (d = 768 has three of 256) then still spreads over every CU, and the
// 48 KB of LDS per block lets three blocks share a CU.
template <int EPI>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_mid_narrow_kernel(GemmArgs a) {
  __shared__ u32x4 sA[2][64 * 8];
  __shared__ u32x4 sB[2][128 * 8];
  const int ntiles = (a.Ndim + 127) / 128;
  const int real = full_tiles_total(a, 128) * ntiles;
  // blocks [0, real) take the upper 64 rows of each 128-row tile, blocks
  // [real, 2 real) the lower 64
  int h = blockIdx.x, half = 0;
  if (h >= real) {
    h -= real;
    half = 1;
  }
  if (h >= real) return;
  int g, row0, rows, by;
  find_tile_2d(a, 128, ntiles, h, real, g, row0, rows, by);
  row0 += 64 * half;
  rows -= 64 * half;
  if (rows <= 0) return;
  if (rows > 64) rows = 64;
  gemm_tile<EPI, 64, 128, 2, 4, 64 * 8, 128 * 8>(a, g, row0, rows, by, sA, sB);
}

// ------------------------------------------------------ weight gradients
// dW = A^T B per group, reducing over the group's rows: A [rows][lda]
// supplies the output rows m (its columns), B [rows][ldb] the output
// columns n.  Both operands are k-major (the rows are the reduction), so
// both go through the transposing LDS reads.  256x256 output tiles on 8
// waves of 128x64; one block per (group, m-tile, n-tile), looping over the
// group's rows 64 at a time (rows past the group read as zero through the
// buffer descriptors' sizes).  An empty group writes zeros.
struct WgradArgs {
  const void* A;
  int lda;
  const void* B;
  int ldb;
  const int32_t* offsets;   // [G+1] row groups, or null: one group of Krows rows
  int G, Krows;
  int M, N;                 // output rows (A columns) and columns (B columns)
  void* C;                  // output rows m < msplit
  void* C2;                 // output rows m >= msplit (as row m - msplit)
  int msplit;
  size_t c_group_stride;    // elements between consecutive groups' outputs
  int ldc;
  int nseg;                 // column n goes to segment n / nseg ...
  size_t nseg_stride;       // ... at nseg_stride elements per segment, column n % nseg
};

__global__ __launch_bounds__(512) void grouped_wgrad_kernel(WgradArgs a) {
  // operand stages, then the output tile: 128 KB in one array
  __shared__ u32x4 smem[4][256 * 8];
  u32x4 (&sA)[2][256 * 8] = *reinterpret_cast<u32x4 (*)[2][256 * 8]>(&smem[0]);
  u32x4 (&sB)[2][256 * 8] = *reinterpret_cast<u32x4 (*)[2][256 * 8]>(&smem[2]);
  constexpr int NW = 8, WGN = 4, WTM = 128, WTN = 64, TM = 4, TN = 2, PER = 32 / NW;
  const int mtn = (a.M + 255) / 256, ntn = (a.N + 255) / 256;
  const int per_g = mtn * ntn, total = a.G * per_g;
  // XCD-contiguous runs of tiles (consecutive blocks go to different XCDs;
  // gridDim is a multiple of 8, so a block stays on one).
  const int full = total - total % 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  lds_t* ldsA[2] = {(lds_t*)&sA[0][wave * PER * 64], (lds_t*)&sA[1][wave * PER * 64]};
  lds_t* ldsB[2] = {(lds_t*)&sB[0][wave * PER * 64], (lds_t*)&sB[1][wave * PER * 64]};

  // tile h: group, output tile origin, the group's rows and operand descriptors
  struct Tile {
    int g, m0, n0, rows;
    __amdgpu_buffer_rsrc_t rA, rB;
  };
  auto setup = [&](int h) __attribute__((always_inline)) {
    Tile t;
    const int L = h < full ? (h % 8) * (full / 8) + h / 8 : h;
    t.g = __builtin_amdgcn_readfirstlane(L / per_g);
    const int rem = L - t.g * per_g;
    const int mt = __builtin_amdgcn_readfirstlane(rem / ntn);
    const int nt = __builtin_amdgcn_readfirstlane(rem - mt * ntn);
    const int r0 = __builtin_amdgcn_readfirstlane(a.offsets ? a.offsets[t.g] : 0);
    t.rows = __builtin_amdgcn_readfirstlane(a.offsets ? a.offsets[t.g + 1] - r0 : a.Krows);
    t.m0 = mt * 256;
    t.n0 = nt * 256;
    const long long abytes = ((long long)t.rows * a.lda - t.m0) * 2;
    const long long bbytes = ((long long)t.rows * a.ldb - t.n0) * 2;
    t.rA = make_rsrc(static_cast<const uint16_t*>(a.A) + (size_t)r0 * a.lda + t.m0,
                     (uint32_t)(abytes > 0 ? abytes : 0));
    t.rB = make_rsrc(static_cast<const uint16_t*>(a.B) + (size_t)r0 * a.ldb + t.n0,
                     (uint32_t)(bbytes > 0 ? bbytes : 0));
    return t;
  };
  auto issue = [&](const Tile& t, int kt, int buf) __attribute__((always_inline)) {
    const uint32_t ka = (uint32_t)kt * BK * (uint32_t)a.lda * 2u;
    const uint32_t kb = (uint32_t)kt * BK * (uint32_t)a.ldb * 2u;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rA, (lds_t*)((char*)ldsA[buf] + i * 1024), 16,
                                               kmajor_voff(wave * PER + i, lane, a.lda) + ka, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rB, (lds_t*)((char*)ldsB[buf] + i * 1024), 16,
                                               kmajor_voff(wave * PER + i, lane, a.ldb) + kb, 0, 0, 0);
  };

  // Persistent: block b takes tiles b, b + gridDim, ...  A tile's first
  // operand stage is issued during the previous tile's epilogue, before
  // that tile's output stores, so the load latency and the store drain
  // overlap (one counter covers both on this target).
  int h = blockIdx.x;
  if (h >= total) return;
  Tile t = setup(h);
  if (t.rows > 0) issue(t, 0, 0);
  for (; h < total; h += gridDim.x) {
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (t.rows + BK - 1) / BK;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(t, kt + 1, buf ^ 1);
    const char* tA = (const char*)&sA[buf][0];
    const char* tB = (const char*)&sB[buf][0];
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = read_kmajor(tA, 0, wm * WTM + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = read_kmajor(tB, 0, wn * WTN + 32 * j, lane);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[cur ^ 1][i] = read_kmajor(tA, kk + 1, wm * WTM + 32 * i, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[cur ^ 1][j] = read_kmajor(tB, kk + 1, wn * WTN + 32 * j, lane);
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

  // epilogue: the tile goes through LDS as bf16 [256][256] (the operand
  // stages are free after the loop's last barrier) and out in 16-byte
  // stores.  Lane holds column lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4;
  // neighbouring lanes swap one value so that each writes a 4-byte pair of
  // columns: the even lane row r, the odd lane row r+1.
  uint32_t* stile = reinterpret_cast<uint32_t*>(&smem[0][0]);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const bool odd = (lane & 1) != 0;
        const float give = odd ? acc[i][j][v] : acc[i][j][v + 1];
        const float got = __shfl_xor(give, 1);
        f32x2 pr;
        pr[0] = odd ? got : acc[i][j][v];
        pr[1] = odd ? acc[i][j][v + 1] : got;
        const int r = wm * WTM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3) + (odd ? 1 : 0);
        const int c = wn * WTN + 32 * j + (lane & 31) - (odd ? 1 : 0);
        stile[r * 128 + (c >> 1)] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
      }
  __syncthreads();
  constexpr int kOut = 256 * 32 / 512;        // 16-byte pieces per thread
  u32x4 outv[kOut];
  const u32x4* vt = &smem[0][0];
#pragma unroll
  for (int it = 0; it < kOut; ++it) outv[it] = vt[tid + 512 * it];
  __syncthreads();                 // the tile's LDS reads are done
  const Tile cur = t;
  if (h + (int)gridDim.x < total) {
    t = setup(h + gridDim.x);
    if (t.rows > 0) issue(t, 0, 0);
  }
  uint16_t* out0 = static_cast<uint16_t*>(a.C) + (size_t)cur.g * a.c_group_stride;
  uint16_t* out1 =
      a.C2 != nullptr ? static_cast<uint16_t*>(a.C2) + (size_t)cur.g * a.c_group_stride : nullptr;
#pragma unroll
  for (int it = 0; it < kOut; ++it) {
    const int id = tid + 512 * it;
    const int r = id >> 5, cv = id & 31;
    const int m = cur.m0 + r, n = cur.n0 + 8 * cv;
    if (m >= a.M || n >= a.N) continue;
    uint16_t* out = m < a.msplit ? out0 : out1;
    const int mr = m < a.msplit ? m : m - a.msplit;
    const size_t ncol = (size_t)(n / a.nseg) * a.nseg_stride + (size_t)(n % a.nseg);
    *reinterpret_cast<u32x4*>(out + (size_t)mr * a.ldc + ncol) = outv[it];
  }
  }  // tiles
}

// ------------------------------------- weight gradients, transposed form
// For groups of many rows the weight gradients run as forward-style GEMMs:
// dW_g = A_g^T B_g with A_g^T stored explicitly (each A column a row,
// reduction index contiguous) and B_g read k-major, the form of the dA and
// dX GEMMs.  The transposed operand holds group g's rows as columns
// kpad[g] .. kpad[g] + K_g, zero up to the next multiple of BK.

// kpad[g]: first column of group g in the transposed operands (a multiple
// of BK); kpad[G]: the padded total.
__global__ void kpad_kernel(const int32_t* offsets, int G, int32_t* kpad) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int acc = 0;
  for (int g = 0; g < G; ++g) {
    kpad[g] = acc;
    acc += (offsets[g + 1] - offsets[g] + BK - 1) / BK * BK;
  }
  kpad[G] = acc;
}

// S [rows][C] (leading dimension lds) -> T [C][ldt] (bf16): row r of group
// g becomes column kpad[g] + r - offsets[g]; each group's padding columns
// are zero.  One block per 64 x 64 tile of T; blocks past kpad[G] exit.
__global__ __launch_bounds__(256) void transpose_groups_kernel(const uint16_t* S, int lds, int C,
                                                               const int32_t* offsets,
                                                               const int32_t* kpad, int G,
                                                               uint16_t* T, int ldt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 8];   // 144-byte rows
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p0 >= kpad[G]) return;
  int lo = 0, hi = G;                      // kpad[lo] <= p0 < kpad[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (kpad[mid] <= p0) lo = mid;
    else hi = mid;
  }
  const int r0 = offsets[lo] + (p0 - kpad[lo]);
  const int nrows = offsets[lo + 1] - r0;  // source rows left in the group (> 0)
#pragma unroll
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int r = q >> 3, cc = (q & 7) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nrows && c0 + cc < C) v = *reinterpret_cast<const u32x4*>(S + (size_t)(r0 + r) * lds + c0 + cc);
    *reinterpret_cast<u32x4*>(&tile[r][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int c = q >> 3, pc = (q & 7) * 8;
    if (c0 + c >= C) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = (uint32_t)tile[pc + 2 * k][c] | ((uint32_t)tile[pc + 2 * k + 1][c] << 16);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(T + (size_t)(c0 + c) * ldt + p0 + pc) = v;
  }
}

struct KGemmArgs {
  const void* AT;          // [M][ldat]: the transposed operand
  int ldat;
  const void* B;           // [rows][ldb]: rows offsets[g] .. of group g, k-major
  int ldb;
  const int32_t* offsets;  // [G+1] group rows
  const int32_t* kpad;     // [G+1] group columns in AT
  int G, M, N;
  void* C;                 // group g: [M][ldc] at C + g * c_group_stride
  int ldc;
  size_t c_group_stride;
};

// One block per (group, 256 x 256 output tile), in the XCD-contiguous,
// patch-rotated order of the forward GEMMs.  A group without rows writes
// zeros.
__global__ __launch_bounds__(512) void grouped_kgemm_kernel(KGemmArgs k) {
  __shared__ u32x4 sA[2][(256 + kExtRows) * 8];
  __shared__ u32x4 sB[2][256 * 8];
  const int mtn = (k.M + 255) / 256, ntn = (k.N + 255) / 256;
  const int per = mtn * ntn, total = k.G * per;
  const int h = blockIdx.x;
  if (h >= total) return;
  const int full = total - total % 8;
  const int L = h < full ? (h % 8) * (full / 8) + h / 8 : h;
  const int g = L / per, l = L - g * per;
  const int nb = l / (mtn * kPatchN);
  const int rem = l - nb * mtn * kPatchN;
  const int nbe = ntn - nb * kPatchN < kPatchN ? ntn - nb * kPatchN : kPatchN;
  const int mt = (rem / nbe + nb) % mtn;
  const int nt = nb * kPatchN + rem % nbe;
  const int kg = k.offsets[g + 1] - k.offsets[g];
  const int kp = k.kpad[g + 1] - k.kpad[g];
  uint16_t* C = static_cast<uint16_t*>(k.C) + (size_t)g * k.c_group_stride;
  const int row0 = mt * 256, rows = k.M - row0 < 256 ? k.M - row0 : 256, n0 = nt * 256;
  if (kp == 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int id = threadIdx.x; id < 256 * 32; id += 512) {
      const int r = id >> 5, col = n0 + 8 * (id & 31);
      if (r < rows && col < k.N) *reinterpret_cast<u32x4*>(C + (size_t)(row0 + r) * k.ldc + col) = z;
    }
    return;
  }
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(k.AT) + k.kpad[g];
  a.lda = k.ldat;
  a.B0 = static_cast<const uint16_t*>(k.B) + (size_t)k.offsets[g] * k.ldb;
  a.B1 = a.B0;
  a.ldb = k.ldb;
  a.kseg = kg;             // the group's rows: B rows past them read 0
  a.Kdim = kp;
  a.Ndim = k.N;
  a.C = C;
  a.ldc = k.ldc;
  a.G = 1;
  a.M = k.M;
  gemm_tile<EPI_NONE, 256, 256, 2, 4, (256 + kExtRows) * 8, 256 * 8, true, true>(a, 0, row0, rows, nt, sA, sB);
}

// --------------------------------------------------------------- fp32
// fp32 problems (the small fp32 configuration): a plain LDS-tiled kernel on
// the vector ALUs.  One 256-thread block per 32-row x 64-column output tile
// of one group; K advances 32 at a time through LDS, loaded along k
// (contiguous in both operands).  Thread (ty, tx) accumulates rows ty and
// ty+16, columns tx + 16j, for gate (and up) weights.
constexpr int kF32Rows = 32;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmArgs a, int BMr) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  __shared__ float sa[kF32Rows][33];
  __shared__ float sg[64][33];
  __shared__ float su[GATED ? 64 : 1][33];
  int g, row0, rows;
  if (!find_tile(a, blockIdx.x, BMr, g, row0, rows)) return;
  const int n0 = blockIdx.y * 64;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* A = static_cast<const float*>(a.A);
  const float* Bg = static_cast<const float*>(a.B0) + (size_t)g * a.b_group_stride;
  const float* Bu = GATED ? static_cast<const float*>(a.B1) + (size_t)g * a.b_group_stride : nullptr;
  float acc[2][4], accu[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = accu[i][j] = 0.0f;
  for (int k0 = 0; k0 < a.Kdim; k0 += 32) {
    // A: 32 rows x 32 k (4 a thread); B: 64 columns x 32 k (8 a thread)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, r = e >> 5, kk = e & 31, k = k0 + kk;
      sa[r][kk] = r < rows && k < a.Kdim ? A[(size_t)(row0 + r) * a.lda + k] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = tid + 256 * q, c = e >> 5, kk = e & 31, k = k0 + kk, col = n0 + c;
      float vg = 0.0f, vu = 0.0f;
      if (col < a.Ndim && k < a.Kdim) {
        const int seg = k / a.kseg;
        const size_t off = (size_t)seg * a.kseg_stride + (size_t)col * a.ldb + (k - seg * a.kseg);
        vg = Bg[off];
        if constexpr (GATED) vu = Bu[off];
      }
      sg[c][kk] = vg;
      if constexpr (GATED) su[c][kk] = vu;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float x0 = sa[ty][kk], x1 = sa[ty + 16][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = sg[tx + 16 * j][kk];
        acc[0][j] = fmaf(x0, w, acc[0][j]);
        acc[1][j] = fmaf(x1, w, acc[1][j]);
        if constexpr (GATED) {
          const float wu = su[tx + 16 * j][kk];
          accu[0][j] = fmaf(x0, wu, accu[0][j]);
          accu[1][j] = fmaf(x1, wu, accu[1][j]);
        }
      }
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(a.C);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = ty + 16 * i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx + 16 * j;
      if (col < a.Ndim) C[(size_t)(row0 + r) * a.ldc + col] = epilogue<EPI>(acc[i][j], accu[i][j]);
    }
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
// 128x64); groups of a few hundred rows use 128-row tiles, which double the
// number of blocks; groups of a few rows (decode-sized batches) use 32-row
// tiles so the matrix cores do not multiply mostly-empty rows.
struct TileShape { int bm; };

TileShape pick_tiles(int rows_per_group) { return TileShape{rows_per_group >= 1024 ? 256 : rows_per_group >= 128 ? 128 : 32}; }

template <int EPI, bool BT = false>
hipError_t launch_bf16(const GemmArgs& a, int bm, int mtiles, hipStream_t s) {
  constexpr int BNH = gated<EPI>() ? 128 : 256;
  dim3 grid(mtiles * ((a.Ndim + BNH - 1) / BNH));
  if (bm == 256)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI, BT>), grid, dim3(512), 0, s, a);
  else if (bm == 128) {
    if constexpr (EPI == EPI_NONE && !BT)
      hipLaunchKernelGGL((grouped_gemm_bf16_mid_narrow_kernel<EPI>),
                         dim3(2 * mtiles * ((a.Ndim + 127) / 128)), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((grouped_gemm_bf16_mid_kernel<EPI, BT>), grid, dim3(512), 0, s, a);
  }
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_small_kernel<EPI, BT>), grid, dim3(256), 0, s, a);
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
  dim3 grid(mtiles, (a.Ndim + 63) / 64);
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
  // fp32 problems: one block per 32 rows; bf16: tiles sized to the mean
  // group (all groups share one tile height so the plan is one prefix sum)
  const int bm = bf16 ? pick_tiles(rows_alloc / p.N).bm : kF32Rows;
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
    const int sbm = bf16 ? pick_tiles(p.T).bm : kF32Rows;
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

// ----------------------------------------------------------- backward
// The expert FFN backward, from the forward's rows and the output
// gradients dY (see the header of this file for the forward GEMMs):
//   dA  = dY W_down                      (k-major W_down)
//   G, U recomputed by GEMM-1; its backward epilogue writes the stored
//        activation a and dG = dA v SiLU'(g), dU = dA SiLU(g)   (ReLU: dG)
//   dX  = [dG dU] [W_gate; W_up]         (k-major weights, two segments)
//   dW_down[e] = dY_e^T a_e,  [dW_gate; dW_up][e] = [dG dU]_e^T X_e
// and the same for the shared experts over all tokens with dY = d_out.
namespace {

WgradArgs wgrad_args(const void* A, int lda, const void* B, int ldb, const int32_t* offsets, int G,
                     int Krows, int M, int N, void* C, void* C2, int msplit, size_t c_group_stride,
                     int ldc, int nseg, size_t nseg_stride) {
  WgradArgs w{};
  w.A = A;
  w.lda = lda;
  w.B = B;
  w.ldb = ldb;
  w.offsets = offsets;
  w.G = G;
  w.Krows = Krows;
  w.M = M;
  w.N = N;
  w.C = C;
  w.C2 = C2;
  w.msplit = msplit;
  w.c_group_stride = c_group_stride;
  w.ldc = ldc;
  w.nseg = nseg;
  w.nseg_stride = nseg_stride;
  return w;
}

// compute units of the current device (cached per device)
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t run_wgrad(const WgradArgs& w, hipStream_t s) {
  const long long tiles = (long long)w.G * ((w.M + 255) / 256) * ((w.N + 255) / 256);
  if (tiles == 0) return hipSuccess;
  // one 512-thread block per compute unit (128 KB of LDS each), rounded
  // down to a multiple of 8 XCDs
  long long blocks = cu_count() / 8 * 8;
  if (blocks < 8) blocks = 8;
  if (blocks > tiles) blocks = tiles;
  hipLaunchKernelGGL(grouped_wgrad_kernel, dim3((unsigned)blocks), dim3(512), 0, s, w);
  return hipGetLastError();
}

hipError_t run_kgemm(const void* AT, int ldat, const void* B, int ldb, const int32_t* offsets,
                     const int32_t* kpad, int G, int M, int N, void* C, int ldc, size_t c_stride,
                     hipStream_t s) {
  KGemmArgs k{AT, ldat, B, ldb, offsets, kpad, G, M, N, C, ldc, c_stride};
  const long long blocks = (long long)G * ((M + 255) / 256) * ((N + 255) / 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_kgemm_kernel, dim3((unsigned)blocks), dim3(512), 0, s, k);
  return hipGetLastError();
}

hipError_t run_transpose(const void* S, int lds, int C, const int32_t* offsets, const int32_t* kpad,
                         int G, void* T, int ldt, hipStream_t s) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(ldt / 64));
  hipLaunchKernelGGL(transpose_groups_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(S),
                     lds, C, offsets, kpad, G, static_cast<uint16_t*>(T), ldt);
  return hipGetLastError();
}

hipError_t run_bwd_epi(const GemmArgs& a, bool swiglu, int bm, int mtiles, hipStream_t s) {
  return swiglu ? launch_bf16<EPI_SWIGLU_BWD>(a, bm, mtiles, s)
                : launch_bf16<EPI_RELU_BWD>(a, bm, mtiles, s);
}

}  // namespace

hipError_t launch_grouped_ffn_backward(const moe_problem_t& p, int rows_alloc, const FfnBwdBuffers& b,
                                       hipStream_t s) {
  const bool swiglu = p.act == MOE_ACT_SWIGLU;
  const int dff = p.d_ff, d = p.d;
  const int bm = pick_tiles(rows_alloc / p.N).bm;
  const int tail_rows = bm == 256 ? kTailRows : 0;
  const int ext_rows = bm == 256 ? kExtRows : 0;
  const int mtiles_max = (rows_alloc + bm - 1) / bm + p.N + (tail_rows > 0 ? p.N : 0);
  int32_t* tiles = b.tiles;
  int32_t* tails = tiles + (p.N + 2);
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, b.offsets, p.N, bm, tail_rows,
                     ext_rows, tiles, tails);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // routed experts: dA = dY W_down
  GemmArgs base{};
  base.offsets = b.offsets;
  base.tiles = tiles;
  base.tails = tails;
  base.tail_rows = tail_rows;
  base.ext_rows = ext_rows;
  base.G = p.N;
  base.rows_alloc = rows_alloc;
  GemmArgs n1 = base;
  n1.A = b.dy_perm;
  n1.lda = d;
  n1.B0 = b.w_down;
  n1.b_group_stride = (size_t)d * dff;
  n1.ldb = dff;
  n1.Kdim = d;
  n1.kseg = d;
  n1.Ndim = dff;
  n1.C = b.dA;
  n1.ldc = dff;
  if ((e = launch_bf16<EPI_NONE, true>(n1, bm, mtiles_max, s)) != hipSuccess) return e;
  // GEMM-1 again, backward epilogue: a and [dG dU]
  GemmArgs r1 = base;
  r1.A = b.x_perm;
  r1.lda = d;
  r1.B0 = b.w_gate;
  r1.B1 = b.w_up;
  r1.b_group_stride = (size_t)dff * d;
  r1.ldb = d;
  r1.Kdim = d;
  r1.kseg = d;
  r1.Ndim = dff;
  r1.C = b.act;
  r1.ldc = dff;
  r1.D = b.dA;
  r1.ldd = dff;
  r1.C2 = b.dgu;
  r1.ldc2 = swiglu ? 2 * dff : dff;
  if ((e = run_bwd_epi(r1, swiglu, bm, mtiles_max, s)) != hipSuccess) return e;
  // dX = [dG dU] [W_gate; W_up]
  GemmArgs n2 = base;
  n2.A = b.dgu;
  n2.lda = swiglu ? 2 * dff : dff;
  n2.B0 = b.w_gate;
  n2.B1 = b.w_up;
  n2.b_group_stride = (size_t)dff * d;
  n2.ldb = d;
  n2.Kdim = swiglu ? 2 * dff : dff;
  n2.kseg = dff;
  n2.Ndim = d;
  n2.C = b.dx_perm;
  n2.ldc = d;
  if ((e = launch_bf16<EPI_NONE, true>(n2, bm, mtiles_max, s)) != hipSuccess) return e;
  // weight gradients
  const int gu = swiglu ? 2 : 1;
  if (b.kpad != nullptr) {
    // transposed form: dW_down = dY^T a, [dW_gate; dW_up] = [dG dU]^T X
    hipLaunchKernelGGL(kpad_kernel, dim3(1), dim3(64), 0, s, b.offsets, p.N, b.kpad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = run_transpose(b.dy_perm, d, d, b.offsets, b.kpad, p.N, b.dyT, b.ldt, s)) != hipSuccess) return e;
    if ((e = run_kgemm(b.dyT, b.ldt, b.act, dff, b.offsets, b.kpad, p.N, d, dff, b.dw_down, dff,
                       (size_t)d * dff, s)) != hipSuccess)
      return e;
    if ((e = run_transpose(b.dgu, gu * dff, gu * dff, b.offsets, b.kpad, p.N, b.dguT, b.ldt, s)) !=
        hipSuccess)
      return e;
    if ((e = run_kgemm(b.dguT, b.ldt, b.x_perm, d, b.offsets, b.kpad, p.N, dff, d, b.dw_gate, d,
                       (size_t)dff * d, s)) != hipSuccess)
      return e;
    if (swiglu &&
        (e = run_kgemm(static_cast<const uint16_t*>(b.dguT) + (size_t)dff * b.ldt, b.ldt, b.x_perm, d,
                       b.offsets, b.kpad, p.N, dff, d, b.dw_up, d, (size_t)dff * d, s)) != hipSuccess)
      return e;
  } else {
    if ((e = run_wgrad(wgrad_args(b.dy_perm, d, b.act, dff, b.offsets, p.N, 0, d, dff, b.dw_down,
                                  nullptr, d, (size_t)d * dff, dff, dff, 0),
                       s)) != hipSuccess)
      return e;
    if ((e = run_wgrad(wgrad_args(b.dgu, gu * dff, b.x_perm, d, b.offsets, p.N, 0, gu * dff, d,
                                  b.dw_gate, b.dw_up, dff, (size_t)dff * d, d, d, 0),
                       s)) != hipSuccess)
      return e;
  }

  if (p.n_shared == 0) return hipSuccess;
  // shared experts over all T tokens, dY = d_out
  const int dffs = p.d_ff_shared, wsw = p.n_shared * dffs;
  const int sbm = pick_tiles(p.T).bm;
  const int s_tail = sbm == 256 ? kTailRows : 0;
  const int s_ext = sbm == 256 ? kExtRows : 0;
  int mt = (p.T + sbm - 1) / sbm;
  if (s_tail > 0) {
    int f, t;
    split_rows(p.T, sbm, s_tail, s_ext, f, t);
    mt = f + t;
  }
  GemmArgs sb{};
  sb.G = 1;
  sb.M = p.T;
  sb.rows_alloc = p.T;
  sb.tail_rows = s_tail;
  sb.ext_rows = s_ext;
  for (int k = 0; k < p.n_shared; ++k) {
    GemmArgs a1 = sb;
    a1.A = b.d_out;
    a1.lda = d;
    a1.B0 = static_cast<const uint16_t*>(b.ws_down) + (size_t)k * d * dffs;
    a1.ldb = dffs;
    a1.Kdim = d;
    a1.kseg = d;
    a1.Ndim = dffs;
    a1.C = static_cast<uint16_t*>(b.dA_s) + (size_t)k * dffs;
    a1.ldc = wsw;
    if ((e = launch_bf16<EPI_NONE, true>(a1, sbm, mt, s)) != hipSuccess) return e;
  }
  GemmArgs sr = sb;
  sr.A = b.u;
  sr.lda = d;
  sr.B0 = b.ws_gate;
  sr.B1 = b.ws_up;
  sr.ldb = d;
  sr.Kdim = d;
  sr.kseg = d;
  sr.Ndim = wsw;
  sr.C = b.act_s;
  sr.ldc = wsw;
  sr.D = b.dA_s;
  sr.ldd = wsw;
  sr.C2 = b.dgu_s;
  sr.ldc2 = swiglu ? 2 * wsw : wsw;
  if ((e = run_bwd_epi(sr, swiglu, sbm, mt, s)) != hipSuccess) return e;
  GemmArgs s2 = sb;
  s2.A = b.dgu_s;
  s2.lda = swiglu ? 2 * wsw : wsw;
  s2.B0 = b.ws_gate;
  s2.B1 = b.ws_up;
  s2.ldb = d;
  s2.Kdim = swiglu ? 2 * wsw : wsw;
  s2.kseg = wsw;
  s2.Ndim = d;
  s2.C = b.dx_shared;
  s2.ldc = d;
  if ((e = launch_bf16<EPI_NONE, true>(s2, sbm, mt, s)) != hipSuccess) return e;
  if ((e = run_wgrad(wgrad_args(b.d_out, d, b.act_s, wsw, nullptr, 1, p.T, d, wsw, b.dws_down,
                                nullptr, d, 0, dffs, dffs, (size_t)d * dffs),
                     s)) != hipSuccess)
    return e;
  return run_wgrad(wgrad_args(b.dgu_s, swiglu ? 2 * wsw : wsw, b.u, d, nullptr, 1, p.T,
                              swiglu ? 2 * wsw : wsw, d, b.dws_gate, b.dws_up, wsw, 0, d, d, 0),
                   s);
}

}  // namespace moe
