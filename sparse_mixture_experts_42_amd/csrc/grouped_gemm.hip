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
// EPI_NONE_T stores the plain product transposed (the weight gradients).
enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3, EPI_RELU_BWD = 4, EPI_NONE_T = 5 };

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
  // persistent launches: work-queue counters (kQueueInts, zero at launch),
  // or null for one block per tile
  int32_t* queue;
  // forward SwiGLU / ReLU epilogues: also keep the fp32 pre-activations,
  // P [rows][ldp] with g at column c and the up projection at Ndim + c; or
  // null
  float* P;
  int ldp;
  // EPI_NONE_T: output column n < ct_split is row n of C, column n >= ct_split
  // row n - ct_split of C2 (both with leading dimension ldc); output rows
  // past M are not stored
  int ct_split;
  // persistent plain GEMMs: split-K of the tail tiles (null: none), partial
  // sums [kSplitSlots][8 waves][32 values][64 lanes] fp32 and kSplitSlots
  // counters, one per tail tile (zero at launch; the last piece of a tile
  // sets its counter to zero again)
  float* split_part;
  int32_t* split_cnt;
  // order of the full tiles over the XCDs (xcd_pos): 0 = one contiguous
  // run of the patch order per XCD; P > 0 = runs dealt in chunks of P tiles
  // round-robin, so the 8 XCDs work on neighbouring chunks at once
  int xcd_chunk;
  // persistent grouped launches without split-K: each group's tail tiles
  // run after the full tiles of their 32 columns (find_tile_fold_p) instead
  // of after all full tiles
  int fold_tails;
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

// The tile plan -- group row offsets and the prefixes of full and tail
// tiles -- seen through an accessor, so that the lookups below serve the
// plan in memory (PtrPlan) and a plan held in registers alike.
struct PtrPlan {
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* tails;
  __host__ __device__ int offset(int i) const { return offsets[i]; }
  __host__ __device__ int tile(int i) const { return tiles[i]; }
  __host__ __device__ int tail(int i) const { return tails[i]; }
};
__host__ __device__ inline PtrPlan ptr_plan(const GemmArgs& a) {
  return PtrPlan{a.offsets, a.tiles, a.tails};
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
constexpr int kXcdChunk = 32;   // chunk of the interleaved XCD order: one XCD's 32 CUs
constexpr int kTailRows = 64;   // rows of a tail tile of the 256-row kernels

// Full-height tiles of all groups (single-group form: from M).
template <typename P>
__host__ __device__ inline int full_tiles_total_p(const GemmArgs& a, const P& pl, int BM) {
  if (a.offsets != nullptr) return pl.tile(a.G);
  int f, t;
  split_rows(a.M, BM, a.tail_rows, a.ext_rows, f, t);
  return f;
}
__host__ __device__ inline int full_tiles_total(const GemmArgs& a, int BM) {
  return full_tiles_total_p(a, ptr_plan(a), BM);
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
//
// Position t of XCD y's run (q tiles per XCD) is logical tile xcd_pos(y, t,
// q, P).  With P = 0 the run is the contiguous range [y q, y q + q).  With
// P > 0 the whole chunks of P tiles are dealt round-robin (chunk c of XCD y
// is logical chunk 8c + y) and the q mod P leftover positions of each XCD
// form contiguous runs after them.  At a given time the XCDs then work on 8
// neighbouring chunks, mostly one or two groups, so an activation panel that
// several XCDs read (one per patch of 4 n-tiles) is fetched from HBM once and
// served to the other XCDs by the shared Infinity Cache; with contiguous
// runs each XCD streams its own group, and a group's activations are
// re-read from HBM by each of its patches once they outgrow that cache.
__host__ __device__ inline int xcd_pos(int y, int t, int q, int P) {
  if (P <= 0) return y * q + t;
  const int qc = q / P * P;
  if (t < qc) return ((t / P) * 8 + y) * P + t % P;
  return 8 * qc + y * (q - qc) + (t - qc);
}

template <typename P>
__host__ __device__ inline void find_tile_2d_p(const GemmArgs& a, const P& pl, int BM, int ntiles,
                                               int h, int real, int& g, int& row0, int& rows,
                                               int& nt) {
  int mt_g, base;
  const int full = real - real % 8;
  const int L = h < full ? xcd_pos(h % 8, h / 8, full / 8, a.xcd_chunk) : h;
  if (a.offsets == nullptr) {
    g = 0;
    mt_g = real / ntiles;
    base = 0;
  } else {
    int lo = 0, hi = a.G;          // tiles[lo]*ntiles <= L < tiles[hi]*ntiles
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pl.tile(mid) * ntiles <= L) lo = mid;
      else hi = mid;
    }
    g = lo;
    mt_g = pl.tile(g + 1) - pl.tile(g);
    base = pl.tile(g) * ntiles;
  }
  const int l = L - base;
  const int nb = l / (mt_g * kPatchN);
  const int rem = l - nb * mt_g * kPatchN;
  const int nbe = ntiles - nb * kPatchN < kPatchN ? ntiles - nb * kPatchN : kPatchN;
  const int mt = (rem / nbe + nb) % mt_g;
  nt = nb * kPatchN + rem % nbe;
  row0 = (a.offsets == nullptr ? 0 : pl.offset(g)) + mt * BM;
  const int end = a.offsets == nullptr ? a.M : pl.offset(g + 1);
  rows = end - row0;
  if (mt < mt_g - 1 && rows > BM) rows = BM;
}
__host__ __device__ inline void find_tile_2d(const GemmArgs& a, int BM, int ntiles, int h, int real,
                                             int& g, int& row0, int& rows, int& nt) {
  find_tile_2d_p(a, ptr_plan(a), BM, ntiles, h, real, g, row0, rows, nt);
}

// Tail tile h (counted from the first tail block): n-tile fastest.  Returns
// false past the last tail tile.
template <typename P>
__host__ __device__ inline bool find_tail_p(const GemmArgs& a, const P& pl, int BM, int ntiles, int h,
                                            int& g, int& row0, int& rows, int& nt) {
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
    if (ti >= pl.tail(a.G)) return false;
    int lo = 0, hi = a.G;          // tails[lo] <= ti < tails[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pl.tail(mid) <= ti) lo = mid;
      else hi = mid;
    }
    g = lo;
    row0 = pl.offset(g) + (pl.tile(g + 1) - pl.tile(g)) * BM;
    end = pl.offset(g + 1);
  }
  rows = end - row0;
  return rows > 0;
}
__host__ __device__ inline bool find_tail(const GemmArgs& a, int BM, int ntiles, int h, int& g,
                                          int& row0, int& rows, int& nt) {
  return find_tail_p(a, ptr_plan(a), BM, ntiles, h, g, row0, rows, nt);
}

// The 256-row plan of a grouped launch with the tail tiles folded in: group
// g walks its n-tiles in runs of 8 patches (kFoldRun = 32 n-tiles): the full
// tiles of the run's patches (each patch full_g x kPatchN tiles, rotated as
// in find_tile_2d_p), then, if the group has a tail tile, the run's tail
// tiles, one per n-tile, padded with empty slots to kFoldRun.  A run's full
// tiles are 8 chunks of 32 tiles when full_g = 8 and its tail tiles one more,
// so the chunks stay aligned; dealt to the 8 XCDs (xcd_chunk = 32) a run's
// full tiles run at once and its tail chunk comes next, so a tail tile reads
// its weight panel shortly after the full tiles of its column did, from the
// Infinity Cache, instead of streaming it from HBM after every full tile has
// run.  Slot h of [0, fold_span()).  bm is 256 or kTailRows; rows as in
// find_tile_2d_p and find_tail_p.  Returns false for a padding slot.
constexpr int kFoldRun = 8 * kPatchN;
__host__ __device__ inline int fold_tail_slots(int ntiles) {
  return (ntiles + kFoldRun - 1) / kFoldRun * kFoldRun;
}
template <typename P>
__host__ __device__ inline int fold_span(const P& pl, int G, int ntiles) {
  return pl.tile(G) * ntiles + pl.tail(G) * fold_tail_slots(ntiles);
}
template <typename P>
__host__ __device__ inline bool find_tile_fold_p(const GemmArgs& a, const P& pl, int ntiles, int h,
                                                 int span, int& g, int& row0, int& rows, int& nt,
                                                 int& bm) {
  const int full = span - span % 8;
  const int L = h < full ? xcd_pos(h % 8, h / 8, full / 8, a.xcd_chunk) : h;
  const int ts = fold_tail_slots(ntiles);
  int lo = 0, hi = a.G;   // slots before group lo <= L < slots before group hi
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pl.tile(mid) * ntiles + pl.tail(mid) * ts <= L) lo = mid;
    else hi = mid;
  }
  g = lo;
  const int mt_g = pl.tile(g + 1) - pl.tile(g);
  const int t_g = pl.tail(g + 1) - pl.tail(g);
  const int l = L - (pl.tile(g) * ntiles + pl.tail(g) * ts);
  const int run = l / ((mt_g + t_g) * kFoldRun);    // runs before the last are kFoldRun wide
  const int c0 = run * kFoldRun;
  const int width = ntiles - c0 < kFoldRun ? ntiles - c0 : kFoldRun;
  const int r = l - run * (mt_g + t_g) * kFoldRun;
  const int end = pl.offset(g + 1);
  if (r < mt_g * width) {
    const int pi = r / (mt_g * kPatchN);            // patches before the last are kPatchN wide
    const int rem = r - pi * mt_g * kPatchN;
    const int nb = c0 / kPatchN + pi;
    const int nbe = ntiles - nb * kPatchN < kPatchN ? ntiles - nb * kPatchN : kPatchN;
    const int mt = (rem / nbe + nb) % mt_g;
    nt = nb * kPatchN + rem % nbe;
    row0 = pl.offset(g) + mt * 256;
    rows = end - row0;
    if (mt < mt_g - 1 && rows > 256) rows = 256;
    bm = 256;
    return rows > 0;
  }
  const int j = r - mt_g * width;
  nt = c0 + j;
  row0 = pl.offset(g) + mt_g * 256;
  rows = end - row0;
  bm = kTailRows;
  return j < width && rows > 0;
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

// Backward of the activation at one element, from the pre-activations g
// (and v) and dA: a = SiLU(g) v, dG = dA v SiLU'(g), dU = dA SiLU(g), with
// SiLU'(g) = s (1 + g (1 - s)), s = sigmoid(g); ReLU: a = max(g, 0),
// dG = dA [g > 0].  The recompute GEMM's epilogue and act_bwd_kernel both
// use these, so the two backward paths round identically.
struct ActBwd {
  float a, dg, du;
};
__device__ __forceinline__ ActBwd swiglu_bwd_point(float gv, float up, float da) {
  const float sg = sigmoid_fast(gv);
  const float sl = gv * sg;
  return ActBwd{sl * up, da * up * sg * (1.0f + gv * (1.0f - sg)), da * sl};
}
__device__ __forceinline__ ActBwd relu_bwd_point(float gv, float da) {
  return ActBwd{gv > 0.0f ? gv : 0.0f, gv > 0.0f ? da : 0.0f, 0.0f};
}

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
struct NoPre {
  __device__ void operator()(int) const {}
};
template <typename P> struct IsNoPre { static constexpr bool value = false; };
template <> struct IsNoPre<NoPre> { static constexpr bool value = true; };

// Forward epilogue of the 256-column tiles (8 waves of 2 x 4): lane holds
// column lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32
// accumulator.  Neighbouring lanes (columns c and c+1) swap one value of
// each row pair, so that the even lane holds row r and the odd lane row
// r+1, both at columns (c, c+1); each lane then stores one bf16 pair (4
// bytes) through a buffer descriptor over the tile's rows, so stores to
// rows past the group fall outside it and are dropped without a branch.
template <int EPI, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_forward_tile(const GemmArgs& a, f32x16 (&acc)[TM][TN], int row0,
                                                   int rows, int n0, int wm, int wn, int lane) {
  constexpr bool GATED = gated<EPI>();
  constexpr int OUT_TN = GATED ? TN / 2 : TN;
  uint16_t* C = static_cast<uint16_t*>(a.C);
  const bool odd = (lane & 1) != 0;
  const int pc = (GATED ? wn * (WTN / 2) : wn * WTN) + (lane & 31) - (odd ? 1 : 0);
  const uint32_t lane_row = (uint32_t)(wm * WTM + 4 * (lane >> 5) + (odd ? 1 : 0));
  const __amdgpu_buffer_rsrc_t rC =
      make_rsrc(C + (size_t)row0 * a.ldc + n0, (uint32_t)((size_t)rows * a.ldc * 2 - (size_t)n0 * 2));
  // the fp32 pre-activations, when kept: g pairs (and up pairs) as 8-byte
  // stores through descriptors over the tile's rows, like the output; they
  // are read once, by the backward, so the stores are non-temporal and do
  // not push the operands the GEMM re-reads out of the caches
  constexpr bool KEEP = EPI == EPI_SWIGLU || EPI == EPI_RELU;
  const bool keep = KEEP && a.P != nullptr;
  __amdgpu_buffer_rsrc_t rPg = rC, rPu = rC;
  if (keep) {
    const size_t pbytes = (size_t)rows * a.ldp * 4;
    rPg = make_rsrc(a.P + (size_t)row0 * a.ldp + n0, (uint32_t)(pbytes - (size_t)n0 * 4));
    if constexpr (GATED)
      rPu = make_rsrc(a.P + (size_t)row0 * a.ldp + a.Ndim + n0,
                      (uint32_t)(pbytes - (size_t)(a.Ndim + n0) * 4));
  }
  auto pair_swap = [&](float x0, float x1, bool odd_lane) {
    const float send = odd_lane ? x0 : x1;
    const float got = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
    f32x2 pr;
    pr[0] = odd_lane ? got : x0;
    pr[1] = odd_lane ? x1 : got;
    return pr;
  };
  // Ndim is a multiple of 64: a 32-column block is valid or not as a whole
  {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < OUT_TN; ++j) {
        if (n0 + pc + 32 * j >= a.Ndim) continue;
        const uint32_t vC = (lane_row * a.ldc + pc + 32 * j) * 2u;
        if (keep) {
          const uint32_t vP = (lane_row * a.ldp + pc + 32 * j) * 4u;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const int rr = 32 * i + 8 * (v >> 2) + (v & 3);
            const f32x2 pg = pair_swap(acc[i][j][v], acc[i][j][v + 1], odd);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pg), rPg, vP,
                                                  rr * a.ldp * 4, 2);
            if constexpr (GATED) {
              const f32x2 pu = pair_swap(acc[i][j + TN / 2][v], acc[i][j + TN / 2][v + 1], odd);
              __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pu), rPu, vP,
                                                    rr * a.ldp * 4, 2);
            }
          }
        }
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float x[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float g = acc[i][j][v + q];
            if constexpr (EPI == EPI_SWIGLU) x[q] = silu_fast(g) * acc[i][j + TN / 2][v + q];
            else if constexpr (EPI == EPI_RELU) x[q] = g > 0.0f ? g : 0.0f;
            else x[q] = g;
          }
          // quad_perm [1,0,3,2]: each lane receives its neighbour's value
          const float send = odd ? x[0] : x[1];
          const float got = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
          f32x2 pr;
          pr[0] = odd ? got : x[0];
          pr[1] = odd ? x[1] : got;
          const int rr = 32 * i + 8 * (v >> 2) + (v & 3);   // uniform part of the row
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)),
                                                rC, vC, rr * a.ldc * 2, 0);
        }
      }
  }
}

// Transposed store of a plain tile: output element (m, n) goes to row n of
// C (n < ct_split) or of C2 (row n - ct_split), at column m.  A lane holds
// four consecutive m of one n in each group of four accumulator values.
// Stored straight from the accumulators, each store instruction would touch
// 32 rows at 16 bytes each; instead each wave passes its WTN x WTM block
// through its own WTN x WTM x 2-byte LDS region (bf16, rows n, the 16-byte
// chunk c of row n at slot c ^ (n % chunks)), then stores whole 16-byte
// pieces, a wave instruction covering 64 * 16 / (2 WTM) rows contiguously.
template <int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_transposed_tile(const GemmArgs& a, f32x16 (&acc)[TM][TN], int row0,
                                                      int rows, int n0, int wm, int wn, int lane,
                                                      u32x4* region) {
  constexpr int CH = WTM / 8;                 // 16-byte chunks per LDS row
  static_assert(CH == 16 && WTN % 32 == 0, "128 m per wave");
  uint32_t* r32 = reinterpret_cast<uint32_t*>(region);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nl = 32 * j + (lane & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * i + q;              // m = 32 i + 8 q + 4 (lane / 32) + 0..3
        f32x2 lo, hi;
        lo[0] = acc[i][j][4 * q];
        lo[1] = acc[i][j][4 * q + 1];
        hi[0] = acc[i][j][4 * q + 2];
        hi[1] = acc[i][j][4 * q + 3];
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        *reinterpret_cast<u32x2*>(r32 + (nl * CH + (c ^ (nl % CH))) * 4 + 2 * (lane >> 5)) = w;
      }
  }
  // the wave reads back what it wrote: 16 lanes a row, 4 rows an instruction
  const int m0 = row0 + wm * WTM;
  const int c = lane & 15;
  const int m = m0 + 8 * c;
#pragma unroll
  for (int it = 0; it < WTN / 4; ++it) {
    const int nl = 4 * it + (lane >> 4);
    const u32x4 v = region[nl * CH + (c ^ (nl % CH))];
    const int n = n0 + wn * WTN + nl;
    if (n >= a.Ndim || m >= row0 + rows) continue;
    uint16_t* row = n < a.ct_split ? static_cast<uint16_t*>(a.C) + (size_t)n * a.ldc
                                   : static_cast<uint16_t*>(a.C2) + (size_t)(n - a.ct_split) * a.ldc;
    *reinterpret_cast<u32x4*>(row + m) = v;
  }
}

// PIPE tiles may continue a persistent block's previous tile: stage 0 uses
// LDS buffer b0 (stage k buffer (k + b0) & 1), `issued` says its loads are
// already in flight, and pre(buf) runs after the main loop, once every wave
// is past the last stage barrier, with buf the LDS buffer that is free
// (where the next tile's stage 0 goes).
template <int EPI, int BM, int BN, int WGM, int WGN, int SAN, int SBN, bool BT = false, bool PIPE = false,
          typename Pre = NoPre>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int g, int row0, int rows, int by,
                                          u32x4 (&sA)[2][SAN], u32x4 (&sB)[2][SBN], int b0 = 0,
                                          bool issued = false, const Pre& pre = Pre{}) {
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
  static_assert(!BT || ((EPI == EPI_NONE || EPI == EPI_NONE_T) && BN == 256),
                "k-major B: plain epilogue, 256 columns");
  constexpr int BNH = GATED ? BN / 2 : BN;        // output columns per tile

  // In a persistent caller's loop (which passes a Pre step) the thread index
  // is made opaque to the compiler, so that the loop recomputes the per-lane
  // addressing of each tile instead of keeping that of every tile shape live
  // across it.  Elsewhere it stays visible: the compiler then proves that the
  // transposing LDS reads of one stage miss the direct loads into the other,
  // and waits for no load mid-stage.
  int tid = threadIdx.x;
  if constexpr (!IsNoPre<Pre>::value) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
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
      // the descriptor ends at column Ndim of the segment's last row, so a
      // group whose columns start inside a wider row reads nothing past them
      const __amdgpu_buffer_rsrc_t rBT =
          make_rsrc(base, (uint32_t)((size_t)(a.kseg - 1) * a.ldb + a.Ndim - n0) * 2u);
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
    if (!issued) issue_part(0, true, b0, 0, NL);
    advance();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    read_frags(fa[0], fb[0], b0, 0);
    // k-steps 0, 1, 2 and the first half of 3 of stage kt; loads l0.. of
    // stage kt+1 are issued during k-steps 0 and 1 (the first ones already
    // went out after the previous barrier)
    auto body = [&](int kt, int l0) {
      const int buf = (kt + b0) & 1;
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
      kstep(fa[1], fb[1], H, TM, fa[0], fb[0], (kt + b0) & 1, 0, true, 1, kt + 1, kt + 1 < nk,
            (kt + 1 + b0) & 1, 0, LB);
      body(kt, LB);
    }
    kstep(fa[1], fb[1], H, TM, fa[0], fb[0], 0, 0, false, 1, 0, false, 0, 0, 0);
    // the empty loads of the last stage still write the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    pre((nk + b0) & 1);
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
          const float da = __builtin_bit_cast(float, q ? (dp & 0xffff0000u) : (dp << 16));
          const ActBwd r = swiglu_bwd_point(gv, uv, da);
          pa[q] = r.a;
          pg[q] = r.dg;
          pu[q] = r.du;
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
  if constexpr (PIPE && (EPI == EPI_NONE || EPI == EPI_SWIGLU || EPI == EPI_RELU)) {
    store_forward_tile<EPI, TM, TN, WTM, WTN>(a, acc, row0, rows, n0, wm, wn, lane);
    return;
  }
  if constexpr (EPI == EPI_NONE_T) {
    // every wave is past its last fragment read before any region is written
    __syncthreads();
    constexpr int RU4 = WTM * WTN * 2 / 16;   // 16-byte units per region
    constexpr int NA = 2 * SAN / RU4;         // regions in sA
    static_assert(NA >= NW || (NW - NA) * RU4 <= 2 * SBN, "a region per wave");
    u32x4* region = wave < NA ? &sA[0][0] + wave * RU4 : &sB[0][0] + (wave - NA) * RU4;
    store_transposed_tile<TM, TN, WTM, WTN>(a, acc, row0, rows, n0, wm, wn, lane, region);
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
            const ActBwd rb = EPI == EPI_SWIGLU_BWD ? swiglu_bwd_point(gv, acc[i][j + TN / 2][v + q], da)
                                                    : relu_bwd_point(gv, da);
            pa[q] = rb.a;
            pg[q] = rb.dg;
            pu[q] = rb.du;
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
          if constexpr (EPI == EPI_SWIGLU || EPI == EPI_RELU) {
            if (a.P != nullptr && r < rows) {
              float* prow = a.P + (size_t)(row0 + r) * a.ldp;
              prow[col] = acc[i][j][v + q];
              if constexpr (EPI == EPI_SWIGLU) prow[a.Ndim + col] = acc[i][j + TN / 2][v + q];
            }
          }
        }
      }
    }
  }
}

// Groups of many rows: 256x256 tiles on 8 waves (128x64 each).  A group's
// last tile grows to 320 rows (160x64 per wave) when the group ends at most
// 64 rows past a multiple of 256, and groups of at most 64 rows get a 64-row
// tail tile (32x64 per wave).
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

// Persistent launches split the 1-D tile space [0, total) into 9 queues:
// queue y < 8 holds the y-th run of q = full/8 tiles of the patch order
// (full = full tiles rounded down to a multiple of 8), queue 8 the rest.
// Position t of queue y is tile slot h (find_tile_2d / find_tail), or -1
// past the queue's end.
__host__ __device__ inline int queue_slot(int y, int t, int q, int full, int rest) {
  if (y < 8) return t < q ? 8 * t + y : -1;
  return t < rest ? full + t : -1;
}

// Split-K of the tail tiles of a persistent plain GEMM: the number of
// pieces per tail tile (1: none) for `tail_tiles` tail tiles, `blocks`
// blocks and nk stages, so that about one piece per block remains, each of
// at least 4 stages, and the pieces fit kSplitSlots partial-sum slots.
__host__ __device__ inline int split_pieces(int tail_tiles, int blocks, int nk) {
  if (tail_tiles <= 0) return 1;
  const int nb = blocks < kSplitSlots ? blocks : kSplitSlots;
  int S = nb / tail_tiles;
  if (S > 4) S = 4;
  if (S > nk / 4) S = nk / 4;
  return S < 1 ? 1 : S;
}
// Piece p of S of a tail tile: stages kt0 .. kt0+n-1 of 0 .. nk-1.
__host__ __device__ inline void split_range(int p, int S, int nk, int& kt0, int& n) {
  kt0 = p * nk / S;
  n = (p + 1) * nk / S - kt0;
}

// Tail tiles of all groups (single-group form: from M).
template <typename P>
__host__ __device__ inline int tail_tiles_total_p(const GemmArgs& a, const P& pl, int BM) {
  if (a.offsets != nullptr) return pl.tail(a.G);
  int f, t;
  split_rows(a.M, BM, a.tail_rows, a.ext_rows, f, t);
  return t;
}
__host__ __device__ inline int tail_tiles_total(const GemmArgs& a, int BM) {
  return tail_tiles_total_p(a, ptr_plan(a), BM);
}

// ------------------------------------------ ring-pipelined persistent GEMM
// Persistent forward GEMM of 256x256 tiles (and 64-row tail tiles) on 8
// waves, whose main loop keeps the weight loads two stages ahead.
//
// The grouped GEMM's stage time is set by how long a stage's loads take to
// arrive.  Within one XCD, the 32 blocks of a patch share every operand
// panel, so most of a stage's 64 KB comes from the L2, but the weight panels
// are streamed from HBM, and with two LDS stages a load has at most one
// stage to arrive.  Here the LDS is five 32-KB slots (all of the CU's 160
// KB): two for the activations (loaded one stage ahead) and three for the
// weights (loaded two stages ahead).  The plan has no extended 320-row
// tiles: their taller activation slots would leave room for only two weight
// slots, and measured, such tiles gave back what they save in traffic.
//
// The loads are direct-to-LDS buffer loads issued in inline asm.  The
// compiler, which does not see that they write the LDS, then inserts no
// waits of its own for them, and the kernel waits itself: at the barrier of
// stage kt it needs A(kt+1) and B(kt+1), while B(kt+2), issued after
// A(kt+1), may stay in flight.  Loads complete in issue order as far as
// vmcnt is concerned, so that wait is vmcnt(number of B loads per wave).
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kPoolU4 = 160 * 1024 / 16;   // the LDS pool in 16-byte units

// Buffer resource words over [base, base + bytes) (the resource make_rsrc
// builds): loads past the end return 0.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 d;
  d[0] = (int)(uint32_t)p;
  d[1] = (int)(uint32_t)(p >> 32);
  d[2] = (int)bytes;
  d[3] = 0x00020000;
  return d;
}

// 16 bytes per lane from global memory to LDS at lds + 16 * lane.  M0 holds
// the LDS address (set by the compiler for the asm operand); one wait state
// separates its write from the load that reads it.
__device__ __forceinline__ void lds_load16(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
// The same load marked non-temporal: for data read once (a decode-sized
// layer's expert weights), streamed past the caches.
__device__ __forceinline__ void lds_load16_nt(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Pool layout: two A slots, then three B slots, 32 KB each (256 tile rows
// of 128 bytes).
struct RingLayout {
  static constexpr int kBAhead = 2;   // stages B is loaded ahead
  static constexpr int kBSlots = 3;
  static constexpr uint32_t kSlot = 256 * 128;
  __device__ static constexpr uint32_t a_off(int s) { return (uint32_t)s * kSlot; }
  __device__ static constexpr uint32_t b_off(int s) { return (2 + (uint32_t)s) * kSlot; }
  static_assert((2 + kBSlots) * kSlot <= kPoolU4 * 16, "the slots fit the pool");
};
// The claimed tile reaches every wave through the pool's last 16 bytes, in
// the third B slot, which the loads first write during stage 0 of a tile,
// after its first barrier.
constexpr int kNextU4 = kPoolU4 - 1;

// Per-lane load addressing of one tile (the lane mapping and row layout of
// gemm_tile): load i of wave w fills tile rows 8q .. 8q+7, q = w*AI + i (A)
// or w*BI + i (B), lane l row 8q + l/8 at 16-byte slot l%8, which holds
// logical chunk (l%8) ^ ((8q + l/8) >> 1 & 7).
template <int EPI, int BM, int NW = 8>
struct RingAddr {
  static constexpr int BN = 256, AI = BM / 8 / NW, BI = BN / 8 / NW;
  static constexpr int BNH = gated<EPI>() ? BN / 2 : BN;
  const uint16_t* a_base;
  uint32_t a_bytes, a_voff_e, a_voff_o, a_step;
  const uint16_t* b_base;   // column tile n0, segment 0
  uint32_t b_bytes, b_voff_e, b_voff_o, b_step;
  int wave;
  int kt0;                  // first stage of the tile's k range (split-K pieces)
  __device__ __forceinline__ RingAddr(const GemmArgs& a, int g, int row0, int rows, int by, int wave_,
                                      int lane, int kt0_ = 0) {
    wave = wave_;
    kt0 = kt0_;
    const int lrow = lane >> 3;
    const int ce = (lane & 7) ^ (lrow >> 1), co = (lane & 7) ^ (4 + (lrow >> 1));
    a_base = static_cast<const uint16_t*>(a.A) + (size_t)row0 * a.lda;
    a_bytes = (uint32_t)rows * a.lda * 2;
    a_voff_e = (uint32_t)((wave * AI * 8 + lrow) * a.lda + ce * 8) * 2;
    a_voff_o = (uint32_t)((wave * AI * 8 + lrow) * a.lda + co * 8) * 2;
    a_step = 8u * a.lda * 2;
    const int n0 = by * BNH;
    b_base = static_cast<const uint16_t*>(a.B0) + (size_t)g * a.b_group_stride;
    int b_local0 = wave * (BN / NW);
    if constexpr (gated<EPI>()) {
      if (wave >= NW / 2) {
        b_base = static_cast<const uint16_t*>(a.B1) + (size_t)g * a.b_group_stride;
        b_local0 -= BN / 2;
      }
    }
    b_base += (size_t)n0 * a.ldb;
    const int b_valid = a.Ndim - n0 < BNH ? a.Ndim - n0 : BNH;
    b_bytes = (uint32_t)b_valid * a.ldb * 2;
    b_voff_e = (uint32_t)((b_local0 + lrow) * a.ldb + ce * 8) * 2;
    b_voff_o = (uint32_t)((b_local0 + lrow) * a.ldb + co * 8) * 2;
    b_step = 8u * a.ldb * 2;
  }
  // load i of the A rows of stage kt into the slot at LDS address slot_lds
  __device__ __forceinline__ void load_a(int kt, bool live, uint32_t slot_lds, int i) const {
    const bool odd = ((wave * AI + i) & 1) != 0;
    lds_load16(rsrc_words(a_base, live ? a_bytes : 0u), slot_lds + (uint32_t)((wave * AI + i) * 1024),
               (odd ? a_voff_o : a_voff_e) + (uint32_t)i * a_step + (uint32_t)(kt0 + kt) * 128u);
  }
  // where the B rows of stage kt start: K segment seg of B (the shared
  // experts' down projection is segmented), k offset within it in bytes
  __device__ __forceinline__ void b_stage(const GemmArgs& a, int kt, const uint16_t*& base,
                                          uint32_t& koff) const {
    const int kb = (kt0 + kt) * 64;
    const int seg = a.kseg == a.Kdim ? 0 : kb / a.kseg;
    base = b_base + (size_t)seg * a.kseg_stride;
    koff = (uint32_t)(kb - seg * a.kseg) * 2u;
  }
  // load i of the B rows of a stage located by b_stage
  __device__ __forceinline__ void load_b(const uint16_t* base, uint32_t koff, bool live, uint32_t slot_lds,
                                         int i) const {
    const bool odd = ((wave * BI + i) & 1) != 0;
    lds_load16(rsrc_words(base, live ? b_bytes : 0u), slot_lds + (uint32_t)((wave * BI + i) * 1024),
               (odd ? b_voff_o : b_voff_e) + (uint32_t)i * b_step + koff);
  }
};

// Loads that start a tile, in this order: A(0), B(0), B(1).
template <int EPI, int BM>
__device__ __forceinline__ void ring_stage0(const GemmArgs& a, const RingAddr<EPI, BM>& ad, int nk,
                                            uint32_t pool_lds) {
  using AD = RingAddr<EPI, BM>;
  using L = RingLayout;
#pragma unroll
  for (int i = 0; i < AD::AI; ++i) ad.load_a(0, true, pool_lds + L::a_off(0), i);
  const uint16_t* bb;
  uint32_t bk;
  ad.b_stage(a, 0, bb, bk);
#pragma unroll
  for (int i = 0; i < AD::BI; ++i) ad.load_b(bb, bk, true, pool_lds + L::b_off(0), i);
  ad.b_stage(a, 1, bb, bk);
#pragma unroll
  for (int i = 0; i < AD::BI; ++i) ad.load_b(bb, bk, nk > 1, pool_lds + L::b_off(1), i);
}

// The k range of a tile: stages kt0 .. kt0+nk-1.  A tail tile of a plain
// (EPI_NONE) GEMM may run as S split-K pieces; piece `piece` of tail tile
// `tt` then leaves fp32 partial sums in a.split_part, and the piece that
// finishes last adds them up in piece order and stores the tile.
struct KRange {
  int kt0, nk;
  int S, piece, tt;
};

// One tile.  `issued`: its first loads (ring_stage0) are already in flight.
// pre() runs after the main loop, once every wave is past the last stage
// barrier and every wave's loads have landed; then no wave reads the pool
// any more, and pre() may start the next tile's loads.
template <int EPI, int BM, typename Pre>
__device__ __forceinline__ void ring_tile(const GemmArgs& a, int g, int row0, int rows, int by,
                                          u32x4 (&pool)[kPoolU4], bool issued, const Pre& pre,
                                          const KRange& kr) {
  using AD = RingAddr<EPI, BM>;
  using L = RingLayout;
  constexpr int WGN = 4, BN = 256;
  constexpr int WTM = BM / 2, WTN = BN / WGN;     // wave tile: 128x64 or 32x64
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr bool GATED = gated<EPI>();
  constexpr int NL = AD::AI + AD::BI;             // loads per wave per stage: A first, then B
  constexpr int FI = AD::BI;                      // loads that may stay in flight at a barrier
  static_assert(!GATED || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  // opaque thread index: the persistent loop recomputes each tile's per-lane
  // addressing instead of keeping that of every tile height live across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  by = __builtin_amdgcn_readfirstlane(by);
  const int wm = wave / WGN, wn = wave % WGN;
  const int n0 = by * AD::BNH;
  const AD ad(a, g, row0, rows, by, wave, lane, kr.kt0);
  const uint32_t pool_lds = (uint32_t)(uintptr_t)(lds_t*)&pool[0];
  const int nk = kr.nk;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto brow = [&](int j) {
    if constexpr (GATED)
      return j < TN / 2 ? wn * (WTN / 2) + 32 * j : BN / 2 + wn * (WTN / 2) + 32 * (j - TN / 2);
    else
      return wn * WTN + 32 * j;
  };
  // fragment r of k-step rkk from A slot sa and B slot sb, in the order the
  // matrix instructions of row 0 need them first: A row 0, the B columns,
  // then A rows 1..
  auto read_one = [&](bf16x8 (&ra)[TM], bf16x8 (&rb)[TN], int sa, int sb, int rkk, int r) {
    const int c = rkk * 2 + (lane >> 5);
    const int ia = r == 0 ? 0 : (r <= TN ? -1 : r - TN);
    if (ia >= 0)
      ra[ia] = __builtin_bit_cast(bf16x8, pool[L::a_off(sa) / 16 + swz(wm * WTM + ia * 32 + (lane & 31), c)]);
    else
      rb[r - 1] = __builtin_bit_cast(bf16x8, pool[L::b_off(sb) / 16 + swz(brow(r - 1) + (lane & 31), c)]);
  };
  // load l of those issued during stage kt: A(kt+1) into A slot sa_n, then
  // B(kt + kBAhead) into B slot sb_n; bb / bk locate those B rows
  const uint16_t* bb = nullptr;
  uint32_t bk = 0;
  auto issue = [&](int kt, int l, int sa_n, int sb_n) {
    if (l < AD::AI) ad.load_a(kt + 1, kt + 1 < nk, pool_lds + L::a_off(sa_n), l);
    else ad.load_b(bb, bk, kt + L::kBAhead < nk, pool_lds + L::b_off(sb_n), l - AD::AI);
  };
  // matrix instructions of rows i0..i1 of one k-step in a fixed order: after
  // instruction s, fragment s / RS of the next k-step when s % RS == 0, and
  // load l0 + s / 2 of the stage when s is odd; leftovers at the end
  auto kstep = [&](const bf16x8 (&fa_)[TM], const bf16x8 (&fb_)[TN], int i0, int i1, bf16x8 (&ra)[TM],
                   bf16x8 (&rb)[TN], int sa, int sb, int rkk, bool rd, int RS, int kt, int l0, int l1,
                   int sa_n, int sb_n) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i < i0 || i >= i1) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_[i], fb_[j], acc[i][j], 0, 0, 0);
        if (rd && s % RS == 0 && s / RS < TM + TN) read_one(ra, rb, sa, sb, rkk, s / RS);
        if ((s & 1) && l0 + s / 2 < l1) issue(kt, l0 + s / 2, sa_n, sb_n);
        __builtin_amdgcn_sched_barrier(0);
        ++s;
      }
    }
#pragma unroll
    for (int t = 0; t < TM + TN; ++t)
      if (rd && t * RS >= s) read_one(ra, rb, sa, sb, rkk, t);
#pragma unroll
    for (int t = 0; t < NL; ++t)
      if (l0 + t < l1 && 2 * t + 1 >= s) issue(kt, l0 + t, sa_n, sb_n);
  };

  constexpr int H = TM / 2;
  bf16x8 fa[2][TM], fb[2][TN];
  if (!issued) ring_stage0<EPI, BM>(a, ad, nk, pool_lds);
  // A(0) and B(0) landed; B(1) may be in flight
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(FI) : "memory");
  __syncthreads();
  int ra2 = 0, rb = 0;   // slots of stage kt: kt % 2 (A) and kt % kBSlots (B)
#pragma unroll
  for (int t = 0; t < TM + TN; ++t) read_one(fa[0], fb[0], 0, 0, 0, t);
  // k-steps 0, 1, 2 and the first half of 3 of stage kt; its loads go out
  // during k-steps 0 and 1
  auto body = [&](int kt) {
    const int sa_n = ra2 ^ 1;
    const int sb_n = rb == 0 ? 2 : rb - 1;   // (kt + 2) % 3
    ad.b_stage(a, kt + L::kBAhead, bb, bk);
    constexpr int LM = TM * TN / 2 < NL ? TM * TN / 2 : NL;
    kstep(fa[0], fb[0], 0, TM, fa[1], fb[1], ra2, rb, 1, true, 2, kt, 0, LM, sa_n, sb_n);
    kstep(fa[1], fb[1], 0, TM, fa[0], fb[0], ra2, rb, 2, true, 2, kt, LM, NL, sa_n, sb_n);
    kstep(fa[0], fb[0], 0, TM, fa[1], fb[1], ra2, rb, 3, true, 2, kt, 0, 0, sa_n, sb_n);
    kstep(fa[1], fb[1], 0, H, fa[0], fb[0], 0, 0, 0, false, 1, kt, 0, 0, sa_n, sb_n);
  };
  body(0);
  for (int kt = 1; kt < nk; ++kt) {
    // stage kt's operands landed: every load but the B loads of stage kt+1
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(FI) : "memory");
    __syncthreads();
    ra2 ^= 1;
    rb = rb + 1 == L::kBSlots ? 0 : rb + 1;
    // second half of k-step 3 of stage kt-1, reading the first fragments of
    // stage kt
    kstep(fa[1], fb[1], H, TM, fa[0], fb[0], ra2, rb, 0, true, 1, kt, 0, 0, 0, 0);
    body(kt);
  }
  kstep(fa[1], fb[1], H, TM, fa[0], fb[0], 0, 0, 0, false, 1, 0, 0, 0, 0, 0);
  // the empty loads of the last stages still write the pool; once every
  // wave's have landed, no wave touches the pool until pre() starts the
  // next tile
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (EPI == EPI_NONE && BM == kTailRows) {
    if (kr.S > 1) {
      // Partial sums of this piece: value r (of 32) of lane l of wave w at
      // [slot][w][r][l], slot = tt * S + piece, so each store instruction
      // writes 256 contiguous bytes.  The stores and, in the last
      // piece, the loads are system-scope atomics: written through to memory
      // and read from it, so pieces on different XCDs (separate L2s) see
      // each other's values.  The counter's add follows the stores' wait.
      float* own = a.split_part + ((size_t)(kr.tt * kr.S + kr.piece) * 8 + wave) * 32 * 64 + lane;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          __hip_atomic_store(own + (16 * j + v) * 64, acc[0][j][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      int32_t* flag = reinterpret_cast<int32_t*>(&pool[kNextU4]) + 1;
      if (tid == 0) *flag = atomicAdd(&a.split_cnt[kr.tt], 1) == kr.S - 1;
      // pre()'s barrier publishes the flag; its loads avoid this word
      pre();
      if (__builtin_amdgcn_readfirstlane(*flag) == 0) return;
      f32x16 sum[TM][TN];
#pragma unroll
      for (int i = 0; i < kr.S; ++i) {
        const float* src = a.split_part + ((size_t)(kr.tt * kr.S + i) * 8 + wave) * 32 * 64 + lane;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = i == kr.piece ? acc[0][j][v]
                                          : __hip_atomic_load(src + (16 * j + v) * 64, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_SYSTEM);
            sum[0][j][v] = i == 0 ? x : sum[0][j][v] + x;
          }
      }
      // the counter is zero again for the next launch that uses it
      if (tid == 0) __hip_atomic_store(&a.split_cnt[kr.tt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      store_forward_tile<EPI, TM, TN, WTM, WTN>(a, sum, row0, rows, n0, wm, wn, lane);
      return;
    }
  }
  pre();
  store_forward_tile<EPI, TM, TN, WTM, WTN>(a, acc, row0, rows, n0, wm, wn, lane);
}

// The tile plan in VGPRs: lane l holds entry l + 64 r (r < 5) of the group
// offsets and of the full- and tail-tile prefixes, so a lookup is a
// readlane (uniform index) and needs no memory access.  Up to 320 entries:
// G <= 256 groups.
struct RegPlan {
  int off[5], til[5], tal[5];
  __device__ __forceinline__ static int pick(const int (&v)[5], int j) {
    const int r = j >> 6;
    const int x = r == 0 ? v[0] : r == 1 ? v[1] : r == 2 ? v[2] : r == 3 ? v[3] : v[4];
    return __builtin_amdgcn_readlane(x, j & 63);
  }
  __device__ __forceinline__ int offset(int i) const { return pick(off, i); }
  __device__ __forceinline__ int tile(int i) const { return pick(til, i); }
  __device__ __forceinline__ int tail(int i) const { return pick(tal, i); }
};

// Persistent forward GEMM over the ring-pipelined tiles: one block per
// compute unit, each taking tiles from work queues until they are empty, so
// no block waits on a second wave of launches.
//
// The tiles are the 1-D tile space of the plan (full tiles, then tail
// tiles).  Its first full tiles (a multiple of 8) are split into 8 equal
// contiguous runs of the patch order, one per XCD: block b sits on XCD b % 8
// (blocks are dealt to the XCDs round-robin) and takes tiles from
// queue[b % 8], so one XCD's compute units work through neighbouring patches
// and share their panels in that XCD's L2.  A block whose run is used up
// takes the other runs' remaining tiles, then queue[8]: the leftover full
// tiles and the tail tiles.  Counters are bumped by one lane with a global
// atomic; they start at zero (the plan kernel clears them).
//
// Thread 0 keeps the queue state in registers and reserves its next
// position in the own run one tile ahead.  After the main loop of a tile,
// the block claims and decodes the next one and issues its first loads,
// which are then in flight during the current tile's epilogue.
template <int EPI>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_ring_kernel(GemmArgs ga) {
  __shared__ u32x4 pool[kPoolU4];
  constexpr int BNH = gated<EPI>() ? 128 : 256;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const GemmArgs a = ga;
  RegPlan pl;
#pragma unroll
  for (int r = 0; r < 5; ++r) {
    const int i = lane + 64 * r;
    const bool in = a.offsets != nullptr && i <= a.G;
    pl.off[r] = in ? a.offsets[i] : 0;
    pl.til[r] = in ? a.tiles[i] : 0;
    pl.tal[r] = in ? a.tails[i] : 0;
  }
  int32_t* s_next = reinterpret_cast<int32_t*>(&pool[kNextU4]);
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total_p(a, pl, 256) * ntiles;
  const int tail_tiles = tail_tiles_total_p(a, pl, 256) * ntiles;
  const int nk = a.Kdim / BK;
  // Tail tiles (64 rows) are few and, with a long K, slow for their work:
  // they mostly stream their weight panel.  When they would leave most
  // blocks idle at the end, a plain GEMM splits each into S k-ranges, so
  // that about one piece per block remains (S * tail_tiles <= kSplitSlots).
  const int S = EPI == EPI_NONE && a.split_part != nullptr ? split_pieces(tail_tiles, gridDim.x, nk) : 1;
  const int total = real + tail_tiles * S;
  // without split-K, a grouped launch may run its tail tiles among the full
  // tiles: the patch order then spans every tile
  const bool fold = a.fold_tails != 0 && S == 1 && a.offsets != nullptr;
  const int span = fold ? fold_span(pl, a.G, ntiles) : real;
  const int full = span - span % 8;
  const int q = full / 8;
  const int rest = (fold ? span : total) - full;
  const int xcd = blockIdx.x & 7;
  int32_t* queue = a.queue;

  // thread 0's queue state: the queue being drained (0: own run, 1..7 the
  // next XCDs' runs, 8: leftovers and tails, 9: none) and the position in
  // the own run requested at the previous claim (-1: none), whose value is
  // used one tile later, when it has long arrived
  int cur = 0, pending = -1;
  // Only thread 0 claims.  The compiler cannot tell, and would aggregate
  // each atomic over the wave: it then rebuilds a per-lane result from the
  // returned value right after the atomic, so the reservation one tile ahead
  // would be waited for at once.  An offset it cannot prove uniform (zero at
  // run time) keeps the atomics plain; the reserved position is then waited
  // for only where it is used, a tile later.
  int zero = 0;
  asm volatile("" : "+v"(zero));
  auto claim = [&]() -> int {
    int spec = pending;
    int h = -1;
    while (cur < 9) {
      const int y = cur < 8 ? (xcd + cur) & 7 : 8;
      const int t = (cur == 0 && spec >= 0) ? spec : atomicAdd(&queue[y + zero], 1);
      spec = -1;
      h = queue_slot(y, t, q, full, rest);
      if (h >= 0) break;
      ++cur;
    }
    pending = cur == 0 ? atomicAdd(&queue[xcd + zero], 1) : -1;
    return h;
  };
  // a tile of the 1-D space: coordinates, height class (256, 64) and k
  // range; false when it holds no rows (block-uniform results)
  auto decode = [&](int h, int& g, int& row0, int& rows, int& by, int& bm, KRange& kr) -> bool {
    bool ok = true;
    kr = KRange{0, nk, 1, 0, 0};
    if (fold) {
      ok = find_tile_fold_p(a, pl, ntiles, h, span, g, row0, rows, by, bm);
    } else if (h < real) {
      find_tile_2d_p(a, pl, 256, ntiles, h, real, g, row0, rows, by);
      bm = 256;
    } else {
      bm = kTailRows;
      const int tt = (h - real) / S, piece = (h - real) - tt * S;
      ok = find_tail_p(a, pl, 256, ntiles, tt, g, row0, rows, by);
      int k0, n;
      split_range(piece, S, nk, k0, n);
      kr = KRange{k0, n, S, piece, tt};
    }
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    rows = __builtin_amdgcn_readfirstlane(rows);
    by = __builtin_amdgcn_readfirstlane(by);
    bm = __builtin_amdgcn_readfirstlane(bm);
    kr.kt0 = __builtin_amdgcn_readfirstlane(kr.kt0);
    kr.nk = __builtin_amdgcn_readfirstlane(kr.nk);
    kr.S = __builtin_amdgcn_readfirstlane(kr.S);
    kr.piece = __builtin_amdgcn_readfirstlane(kr.piece);
    kr.tt = __builtin_amdgcn_readfirstlane(kr.tt);
    return __builtin_amdgcn_readfirstlane((int)ok) != 0;
  };

  if (tid == 0) *s_next = claim();
  __syncthreads();
  int h = __builtin_amdgcn_readfirstlane(*s_next);
  int g = 0, row0 = 0, rows = 0, by = 0, bm = 0;
  KRange kr{0, nk, 1, 0, 0};
  bool work = h >= 0 && decode(h, g, row0, rows, by, bm, kr);
  bool issued = false;
  const uint32_t pool_lds = (uint32_t)(uintptr_t)(lds_t*)&pool[0];
  while (h >= 0) {
    int h_next = -1, g2 = 0, r2 = 0, n2 = 0, y2 = 0, bm2 = 0;
    KRange kr2{0, nk, 1, 0, 0};
    bool next_work = false;
    // claim the next tile, decode it and start its loads
    auto pre = [&]() {
      if (tid == 0) *s_next = claim();
      __syncthreads();
      h_next = __builtin_amdgcn_readfirstlane(*s_next);
      next_work = h_next >= 0 && decode(h_next, g2, r2, n2, y2, bm2, kr2);
      if (next_work) {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int w = __builtin_amdgcn_readfirstlane(t >> 6);
        if (bm2 == 256)
          ring_stage0<EPI, 256>(a, RingAddr<EPI, 256>(a, g2, r2, n2, y2, w, t & 63), nk, pool_lds);
        else
          ring_stage0<EPI, kTailRows>(a, RingAddr<EPI, kTailRows>(a, g2, r2, n2, y2, w, t & 63, kr2.kt0),
                                      kr2.nk, pool_lds);
      }
    };
    if (!work) {
      // a tile slot without rows: every wave has read s_next before thread
      // 0 writes it again
      __syncthreads();
      pre();
    } else if (bm == 256) {
      ring_tile<EPI, 256>(a, g, row0, rows, by, pool, issued, pre, kr);
    } else {
      ring_tile<EPI, kTailRows>(a, g, row0, rows, by, pool, issued, pre, kr);
    }
    issued = next_work;
    work = next_work;
    h = h_next;
    g = g2;
    row0 = r2;
    rows = n2;
    by = y2;
    bm = bm2;
    kr = kr2;
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


// -------------------------------------------- streaming GEMM, small groups
// Groups of a few rows (decode-sized batches).  These GEMMs stream the
// touched experts' weights from HBM once and do little arithmetic per
// byte; what limits them is how evenly the weight bytes spread over the
// CUs and how many are in flight.  Each block is one wave and one tile of
// 32 rows x 64 weight rows (SwiGLU: 32 gate + 32 up rows, 32 output
// columns), so a layer has four times the tiles of 256-row weight panels
// and the last round of tiles is short.  The LDS holds kStreamSlots stages
// of 4 KB of activation rows and 8 KB of weight rows; both are loaded
// kStreamSlots - 1 stages ahead (36 loads of 1 KB in flight per wave), three
// blocks per CU.  The weights are read once, so their loads are
// non-temporal.  Each output element sums its k in the same order as the
// 32-row tiles of gemm_tile.
constexpr int kStreamSlots = 4;

template <int EPI>
__global__ __launch_bounds__(64) void grouped_gemm_bf16_stream_kernel(GemmArgs a) {
  constexpr int BM = 32, BN = 64, NS = kStreamSlots, D = NS - 1;
  constexpr bool GATED = gated<EPI>();
  constexpr int BNH = GATED ? BN / 2 : BN;             // output columns per tile
  constexpr int TN = 2;                                // 32x32 accumulators
  constexpr uint32_t ASLOT = BM * 128, BSLOT = BN * 128;
  constexpr int AI = BM / 8, BI = BN / 8, NL = AI + BI;   // 1-KB loads per stage
  static_assert((D - 1) * NL <= 63, "vmcnt counts at most 63 loads");
  __shared__ u32x4 pool[NS * (ASLOT + BSLOT) / 16];
  const int ntiles = (a.Ndim + BNH - 1) / BNH;
  const int real = full_tiles_total(a, BM) * ntiles;
  const int h = blockIdx.x;
  if (h >= real) return;
  int g, row0, rows, by;
  find_tile_2d(a, BM, ntiles, h, real, g, row0, rows, by);
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  by = __builtin_amdgcn_readfirstlane(by);
  const int lane = threadIdx.x & 63;
  const int n0 = by * BNH;
  // load i fills tile rows 8i .. 8i+7: lane l row 8i + l/8 at 16-byte slot
  // l%8, which holds logical chunk (l%8) ^ ((8i + l/8) >> 1 & 7)
  const int lrow = lane >> 3;
  const int ce = (lane & 7) ^ (lrow >> 1), co = (lane & 7) ^ (4 + (lrow >> 1));
  const uint16_t* a_base = static_cast<const uint16_t*>(a.A) + (size_t)row0 * a.lda;
  const uint32_t a_bytes = (uint32_t)rows * a.lda * 2;
  const uint32_t a_voff_e = (uint32_t)(lrow * a.lda + ce * 8) * 2, a_voff_o = (uint32_t)(lrow * a.lda + co * 8) * 2;
  // B rows: gated, rows 0-31 the gate rows and 32-63 the up rows of output
  // columns n0 .. n0+31; plain, rows 0-63 of columns n0 .. n0+63
  const int b_valid = a.Ndim - n0 < BNH ? a.Ndim - n0 : BNH;
  const uint16_t* b0 = static_cast<const uint16_t*>(a.B0) + (size_t)g * a.b_group_stride + (size_t)n0 * a.ldb;
  const uint16_t* b1 = GATED ? static_cast<const uint16_t*>(a.B1) + (size_t)g * a.b_group_stride +
                                   (size_t)n0 * a.ldb
                             : b0;
  const uint32_t b_bytes = (uint32_t)b_valid * a.ldb * 2;
  const uint32_t b_voff_e = (uint32_t)(lrow * a.ldb + ce * 8) * 2, b_voff_o = (uint32_t)(lrow * a.ldb + co * 8) * 2;
  const uint32_t pool_lds = (uint32_t)(uintptr_t)(lds_t*)&pool[0];
  auto a_off = [](int s) { return (uint32_t)s * ASLOT; };
  auto b_off = [](int s) { return NS * ASLOT + (uint32_t)s * BSLOT; };
  const int nk = a.Kdim / BK;
  // stage kt into slot kt % NS: A rows, then B rows
  auto issue = [&](int kt) {
    const int s = kt % NS;
    const bool live = kt < nk;
    const uint32_t ka = (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_load16(rsrc_words(a_base, live ? a_bytes : 0u), pool_lds + a_off(s) + (uint32_t)i * 1024u,
                 ((i & 1) ? a_voff_o : a_voff_e) + (uint32_t)i * 8u * a.lda * 2u + ka);
    const int kb = live ? kt * 64 : 0;
    const int seg = a.kseg == a.Kdim ? 0 : kb / a.kseg;
    const uint32_t koff = (uint32_t)(kb - seg * a.kseg) * 2u;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      // gated: loads 0-3 the gate rows, 4-7 the up rows (row 8i - 32)
      const bool up = GATED && i >= BI / 2;
      const int r8 = up ? i - BI / 2 : i;
      const uint16_t* base = (up ? b1 : b0) + (size_t)seg * a.kseg_stride;
      lds_load16_nt(rsrc_words(base, live ? b_bytes : 0u), pool_lds + b_off(s) + (uint32_t)i * 1024u,
                    ((i & 1) ? b_voff_o : b_voff_e) + (uint32_t)r8 * 8u * a.ldb * 2u + koff);
    }
  };
  f32x16 acc[1][TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[0][j][v] = 0.0f;
#pragma unroll
  for (int kt = 0; kt < D; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed; the D - 1 stages after it may still be in flight.  One
    // wave: its own program order keeps the slot of stage kt + D, which stage
    // kt - 1 used, free of reads
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((D - 1) * NL) : "memory");
    issue(kt + D);
    const int s = kt % NS;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      const bf16x8 fa = __builtin_bit_cast(bf16x8, pool[a_off(s) / 16 + swz(lane & 31, c)]);
      bf16x8 fb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = __builtin_bit_cast(bf16x8, pool[b_off(s) / 16 + swz(32 * j + (lane & 31), c)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[j], acc[0][j], 0, 0, 0);
    }
  }
  // the empty loads of the last stages still write the pool: drain them
  // before the block ends and another block takes this LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  store_forward_tile<EPI, 1, TN, BM, BN>(a, acc, row0, rows, n0, 0, 0, lane);
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
  // LDS addresses of this wave's part of each operand stage
  const uint32_t ldsA[2] = {(uint32_t)(uintptr_t)(lds_t*)&sA[0][wave * PER * 64],
                            (uint32_t)(uintptr_t)(lds_t*)&sA[1][wave * PER * 64]};
  const uint32_t ldsB[2] = {(uint32_t)(uintptr_t)(lds_t*)&sB[0][wave * PER * 64],
                            (uint32_t)(uintptr_t)(lds_t*)&sB[1][wave * PER * 64]};

  // tile h: group, output tile origin, the group's rows and operand descriptors
  struct Tile {
    int g, m0, n0, rows;
    i32x4 rA, rB;
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
    t.rA = rsrc_words(static_cast<const uint16_t*>(a.A) + (size_t)r0 * a.lda + t.m0,
                      (uint32_t)(abytes > 0 ? abytes : 0));
    t.rB = rsrc_words(static_cast<const uint16_t*>(a.B) + (size_t)r0 * a.ldb + t.n0,
                      (uint32_t)(bbytes > 0 ? bbytes : 0));
    return t;
  };
  // The loads are inline asm, so the compiler, which does not see that they
  // write LDS, adds no waits for them before the transposing reads of the
  // other buffer; the stage's explicit vmcnt(0) and barrier order them.
  auto issue = [&](const Tile& t, int kt, int buf) __attribute__((always_inline)) {
    const uint32_t ka = (uint32_t)kt * BK * (uint32_t)a.lda * 2u;
    const uint32_t kb = (uint32_t)kt * BK * (uint32_t)a.ldb * 2u;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      lds_load16(t.rA, ldsA[buf] + i * 1024u, kmajor_voff(wave * PER + i, lane, a.lda) + ka);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      lds_load16(t.rB, ldsB[buf] + i * 1024u, kmajor_voff(wave * PER + i, lane, a.ldb) + kb);
  };

  // Persistent: block b takes tiles b, b + gridDim, ...  A tile's first
  // operand stage is issued during the previous tile's epilogue, before
  // that tile's output stores, so the load latency and the store drain
  // overlap (one counter covers both on this target).
  int h = blockIdx.x;
  if (h >= total) return;
  Tile t = setup(h);
  if (t.rows > 0) issue(t, 0, 0);
  constexpr int kOut = 256 * 32 / 512;        // 16-byte output pieces per thread
  // Memory operations complete in issue order as vmcnt counts them.  After
  // a tile whose kOut stores per thread all issued (no edge), the next
  // tile's first-stage loads, issued before those stores, are done once at
  // most kOut operations are outstanding: the stores keep draining while
  // the next tile computes.
  bool drain_all = true;
  for (; h < total; h += gridDim.x) {
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (t.rows + BK - 1) / BK;
  if (drain_all)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kOut) : "memory");
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
  drain_all = cur.m0 + 256 > a.M || cur.n0 + 256 > a.N;
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
// One 256-thread block (G <= 256): thread g holds group g's padded size, and
// a block scan in LDS gives the exclusive prefix.
__global__ __launch_bounds__(256) void kpad_kernel(const int32_t* offsets, int G, int32_t* kpad) {
  __shared__ int sc[256];
  const int g = threadIdx.x;
  const int own = g < G ? (offsets[g + 1] - offsets[g] + BK - 1) / BK * BK : 0;
  sc[g] = own;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = g >= off ? sc[g - off] : 0;
    __syncthreads();
    sc[g] += v;
    __syncthreads();
  }
  if (g < G) kpad[g] = sc[g] - own;
  if (g == G - 1) kpad[G] = sc[g];
}

// S [rows][C] (leading dimension lds) -> T [C][ldt] (bf16): row r of group
// g becomes column kpad[g] + r - offsets[g]; each group's padding columns
// are zero.  With offsets null, the S rows 0 .. rows1-1 are one group at
// column 0, zero-filled up to ldt.  One block per 64 x 64 tile of T; blocks
// past the last column exit.
__global__ __launch_bounds__(256) void transpose_groups_kernel(const uint16_t* S, int lds, int C,
                                                               const int32_t* offsets,
                                                               const int32_t* kpad, int G,
                                                               uint16_t* T, int ldt, int rows1) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 8];   // 144-byte rows
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  int r0, nrows;                           // source rows left in the group
  if (offsets == nullptr) {
    r0 = p0;
    nrows = rows1 - p0;
  } else {
    if (p0 >= kpad[G]) return;
    int lo = 0, hi = G;                    // kpad[lo] <= p0 < kpad[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (kpad[mid] <= p0) lo = mid;
      else hi = mid;
    }
    r0 = offsets[lo] + (p0 - kpad[lo]);
    nrows = offsets[lo + 1] - r0;
  }
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

// One weight-gradient problem: per group g, C_g = AT_g B_g reduced over the
// group's rows, with AT the transposed operand and B read k-major.
struct KGemmSet {
  const void* AT;          // [M][ldat]: group g's k columns from kpad[g]
  int ldat;
  const void* B;           // [rows][ldb]: rows offsets[g] .. of group g
  int ldb;
  const int32_t* offsets;  // [G+1] group rows; or null: every group reduces
  const int32_t* kpad;     // over rows 0 .. rows-1, AT columns from 0, and
  int rows;                // takes B columns from g * b_group_cols
  size_t b_group_cols;
  int G, M, N;
  void* C;                 // group g: [M][ldc] at C + g * c_group_stride
  int ldc;
  size_t c_group_stride;
  // transposed output (EPI_NONE_T): group g's output column n < ct_split is
  // row n of C + g * c_group_stride, column n >= ct_split row n - ct_split of
  // C2 + g * c_group_stride; each row holds the M outputs of its column
  void* C2;
  int ct_split;
};

// Blocks 0 .. head-1 take the tiles of set[0] (head: its tile count rounded
// up to a multiple of 8, 0 for none), the rest those of set[1].
struct KGemmArgs {
  KGemmSet set[2];
  int head;
};

__host__ __device__ inline int kgemm_tiles(const KGemmSet& k) {
  return k.G * ((k.M + 255) / 256) * ((k.N + 255) / 256);
}

// One block per (set, group, 256 x 256 output tile).  Within a set the tiles
// run in the XCD-contiguous, patch-rotated order of the forward GEMMs; set 0
// (a few long reductions, e.g. shared experts over every token) comes
// first, so its blocks start at once, spread over the XCDs, while set 1's
// shorter tiles fill the other compute units.  A group without rows writes
// zeros.  EPI is EPI_NONE (output [M][N]) or EPI_NONE_T (output stored
// transposed, [N][M], split at ct_split between C and C2).
template <int EPI>
__global__ __launch_bounds__(512) void grouped_kgemm_kernel(KGemmArgs ka) {
  __shared__ u32x4 sA[2][(256 + kExtRows) * 8];
  __shared__ u32x4 sB[2][256 * 8];
  const bool first = (int)blockIdx.x < ka.head;
  const KGemmSet k = first ? ka.set[0] : ka.set[1];
  const int mtn = (k.M + 255) / 256, ntn = (k.N + 255) / 256;
  const int per = mtn * ntn, total = k.G * per;
  const int h = first ? (int)blockIdx.x : (int)blockIdx.x - ka.head;   // head % 8 == 0
  if (h >= total) return;
  const int full = total - total % 8;
  const int L = h < full ? (h % 8) * (full / 8) + h / 8 : h;
  const int g = L / per, l = L - g * per;
  const int nb = l / (mtn * kPatchN);
  const int rem = l - nb * mtn * kPatchN;
  const int nbe = ntn - nb * kPatchN < kPatchN ? ntn - nb * kPatchN : kPatchN;
  const int mt = (rem / nbe + nb) % mtn;
  const int nt = nb * kPatchN + rem % nbe;
  const int r0 = k.offsets ? k.offsets[g] : 0;
  const int kg = k.offsets ? k.offsets[g + 1] - r0 : k.rows;
  const int kc = k.offsets ? k.kpad[g] : 0;
  const int kp = k.offsets ? k.kpad[g + 1] - kc : (k.rows + BK - 1) / BK * BK;
  uint16_t* C = static_cast<uint16_t*>(k.C) + (size_t)g * k.c_group_stride;
  uint16_t* C2 = EPI == EPI_NONE_T ? static_cast<uint16_t*>(k.C2) + (size_t)g * k.c_group_stride : nullptr;
  const int row0 = mt * 256, rows = k.M - row0 < 256 ? k.M - row0 : 256, n0 = nt * 256;
  if (kp == 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int id = threadIdx.x; id < 256 * 32; id += 512) {
      const int r = id >> 5, col = 8 * (id & 31);
      if constexpr (EPI == EPI_NONE_T) {
        // output column n0 + r: M values from row0 + col
        const int n = n0 + r;
        if (n < k.N && col < rows) {
          uint16_t* dst = n < k.ct_split ? C + (size_t)n * k.ldc : C2 + (size_t)(n - k.ct_split) * k.ldc;
          *reinterpret_cast<u32x4*>(dst + row0 + col) = z;
        }
      } else if (r < rows && n0 + col < k.N) {
        *reinterpret_cast<u32x4*>(C + (size_t)(row0 + r) * k.ldc + n0 + col) = z;
      }
    }
    return;
  }
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(k.AT) + kc;
  a.lda = k.ldat;
  a.B0 = static_cast<const uint16_t*>(k.B) + (size_t)r0 * k.ldb + (k.offsets ? 0 : (size_t)g * k.b_group_cols);
  a.B1 = a.B0;
  a.ldb = k.ldb;
  a.kseg = kg;             // the group's rows: B rows past them read 0
  a.Kdim = kp;
  a.Ndim = k.N;
  a.C = C;
  a.C2 = C2;
  a.ct_split = k.ct_split;
  a.ldc = k.ldc;
  a.G = 1;
  a.M = k.M;
  gemm_tile<EPI, 256, 256, 2, 4, (256 + kExtRows) * 8, 256 * 8, true, true>(a, 0, row0, rows, nt, sA, sB);
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
                                                        int32_t* tiles, int32_t* tails,
                                                        int32_t* queues) {
  __shared__ int32_t s[256], t[256];
  const int g = threadIdx.x;
  // the persistent GEMM launches that follow start from empty queues and
  // zero split-K counters
  if (queues != nullptr)
    for (int i = g; i < kQueueSets * kQueueInts + kSplitSlots; i += 256) queues[i] = 0;
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
  constexpr bool kFwd = !BT && (EPI == EPI_NONE || EPI == EPI_SWIGLU || EPI == EPI_RELU);
  if (bm == 256 && kFwd && a.queue != nullptr) {
    // one block per compute unit, a multiple of the 8 XCDs
    int blocks = cu_count() / 8 * 8;
    if (blocks < 8) blocks = 8;
    // the weights are the streamed operand: they run two stages ahead
    hipLaunchKernelGGL((grouped_gemm_bf16_ring_kernel<kFwd ? EPI : EPI_NONE>), dim3(blocks), dim3(512), 0, s,
                       a);
  } else if (bm == 256)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI, BT>), grid, dim3(512), 0, s, a);
  else if (bm == 128) {
    if constexpr (EPI == EPI_NONE && !BT)
      hipLaunchKernelGGL((grouped_gemm_bf16_mid_narrow_kernel<EPI>),
                         dim3(2 * mtiles * ((a.Ndim + 127) / 128)), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((grouped_gemm_bf16_mid_kernel<EPI, BT>), grid, dim3(512), 0, s, a);
  }
  else if (kFwd)
    hipLaunchKernelGGL((grouped_gemm_bf16_stream_kernel<kFwd ? EPI : EPI_NONE>),
                       dim3(mtiles * ((a.Ndim + BNH / 4 - 1) / (BNH / 4))), dim3(64), 0, s, a);
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

int ffn_row_tile(int rows, int groups, bool bf16) {
  return bf16 ? pick_tiles(rows / groups).bm : kF32Rows;
}

hipError_t launch_grouped_ffn(const moe_problem_t& p, int rows_alloc, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, const void* u, const void* ws_gate,
                              const void* ws_up, const void* ws_down, void* y_perm,
                              void* y_shared, int32_t* tiles, void* act, void* act_shared,
                              float* split, hipStream_t s, float* pre, float* pre_shared) {
  const int gu = p.act == MOE_ACT_SWIGLU ? 2 : 1;
  const bool bf16 = p.dtype == MOE_BF16;
  const int epi1 = p.act == MOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_RELU;
  // fp32 problems: one block per 32 rows; bf16: tiles sized to the mean
  // group (all groups share one tile height so the plan is one prefix sum)
  const int bm = ffn_row_tile(rows_alloc, p.N, bf16);
  // the persistent 256-row kernel runs full and tail tiles, no extended ones
  const int tail_rows = bf16 && bm == 256 ? kTailRows : 0;
  const int ext_rows = 0;
  // grid bound: at most rows/bm + 1 full tiles and one tail tile per group
  const int mtiles_max = (rows_alloc + bm - 1) / bm + p.N + (tail_rows > 0 ? p.N : 0);
  int32_t* tails = tiles + (p.N + 2);
  int32_t* queues = tiles + 2 * (p.N + 2);

  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, offsets, p.N, bm, tail_rows,
                     ext_rows, tiles, tails, queues);
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
  g1.queue = queues;
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
  g1.P = bf16 ? pre : nullptr;
  g1.ldp = gu * p.d_ff;
  // the gate/up GEMM runs its tail tiles right after the full tiles of their
  // columns, with the 8 XCDs on neighbouring chunks of one group, when the
  // groups average 8 row tiles or more, so that a patch fills the 32 CUs of
  // an XCD; with fewer, the patches do not line up with the chunks anyway
  // and the padded tail slots cost more than the re-read weight panels
  const bool fold1 = bm == 256 && rows_alloc >= 8 * 256 * p.N;
  g1.fold_tails = fold1 ? 1 : 0;
  g1.xcd_chunk = fold1 ? kXcdChunk : 0;
  if ((e = run_gemm(g1, epi1, bf16, bm, mtiles_max, s)) != hipSuccess) return e;

  // the down GEMMs may split their tail tiles' k range (one after the other,
  // sharing the partial-sum buffer and the counters, which each launch
  // leaves at zero)
  int32_t* split_cnt = queues + kQueueSets * kQueueInts;
  GemmArgs g2 = g1;
  g2.P = nullptr;
  g2.fold_tails = 0;
  g2.split_part = bf16 ? split : nullptr;
  g2.split_cnt = split_cnt;
  g2.A = act;
  g2.B0 = w_down;
  g2.B1 = nullptr;
  g2.C = y_perm;
  g2.queue = queues + kQueueInts;
  g2.Ndim = p.d;
  g2.Kdim = p.d_ff;
  g2.lda = p.d_ff;
  g2.ldb = p.d_ff;
  g2.ldc = p.d;
  g2.kseg = p.d_ff;
  g2.b_group_stride = (size_t)p.d * p.d_ff;
  // the down GEMM's activations (rows x d_ff) are the large operand: XCDs
  // share them through the Infinity Cache in chunks of one XCD's 32 CUs
  g2.xcd_chunk = kXcdChunk;
  if ((e = run_gemm(g2, EPI_NONE, bf16, bm, mtiles_max, s)) != hipSuccess) return e;

  if (p.n_shared > 0) {
    // all shared experts as one expert of width n_shared*d_ff_shared: the
    // gate/up rows of consecutive experts are contiguous; the down
    // projection is K-segmented, one segment per shared expert
    const int ws_w = p.n_shared * p.d_ff_shared;
    const int sbm = ffn_row_tile(p.T, 1, bf16);
    const int s_tail = bf16 && sbm == 256 ? kTailRows : 0;
    const int s_ext = 0;
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
    s1.queue = queues + 2 * kQueueInts;
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
    s1.P = bf16 ? pre_shared : nullptr;
    s1.ldp = gu * ws_w;
    if ((e = run_gemm(s1, epi1, bf16, sbm, mt, s)) != hipSuccess) return e;
    GemmArgs s2 = s1;
    s2.P = nullptr;
    s2.split_part = bf16 ? split : nullptr;
    s2.split_cnt = split_cnt;
    s2.A = act_shared;
    s2.queue = queues + 3 * kQueueInts;
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
// The activation backward without GEMM-1, from the forward's fp32
// pre-activations P [rows][ldp] (g at column c, v at d_ff + c): the same
// a, dG and dU as the recompute GEMM's epilogue, element for element (same
// accumulators, same swiglu_bwd_point / relu_bwd_point, same bf16 rounding).
// Rows [0, *nrows_dev) (or nrows when nrows_dev is null); 8 columns a thread.
namespace {
template <bool SWIGLU>
__global__ __launch_bounds__(256) void act_bwd_kernel(const float* P, int ldp, const uint16_t* dA,
                                                      int ldd, const int32_t* nrows_dev, int nrows,
                                                      int dff, uint16_t* act, int ldc, uint16_t* dgu,
                                                      int ldc2) {
  const long long R = nrows_dev != nullptr ? *nrows_dev : nrows;
  const int cpr = dff / 8;
  // 8 columns of one row per item; P and dA are read once, so their loads
  // are non-temporal
  auto item = [&](long long r, int c) {
    const float* pg = P + r * ldp + c;
    float g[8], v[8], da[8];
    auto ld4 = [](const float* q, float* out) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(x[j]);
    };
    ld4(pg, &g[0]);
    ld4(pg + 4, &g[4]);
    if constexpr (SWIGLU) {
      ld4(pg + dff, &v[0]);
      ld4(pg + dff + 4, &v[4]);
    }
    const u32x4 dq = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dA + r * ldd + c));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      da[2 * q] = __uint_as_float(dq[q] << 16);
      da[2 * q + 1] = __uint_as_float(dq[q] & 0xffff0000u);
    }
    uint32_t wa[4], wg[4], wu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x2 pa, pgr, pu;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 2 * q + h;
        const ActBwd rb = SWIGLU ? swiglu_bwd_point(g[k], v[k], da[k]) : relu_bwd_point(g[k], da[k]);
        pa[h] = rb.a;
        pgr[h] = rb.dg;
        pu[h] = rb.du;
      }
      wa[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pa, bf16x2));
      wg[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pgr, bf16x2));
      if constexpr (SWIGLU) wu[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pu, bf16x2));
    }
    *reinterpret_cast<u32x4*>(act + r * ldc + c) = u32x4{wa[0], wa[1], wa[2], wa[3]};
    *reinterpret_cast<u32x4*>(dgu + r * ldc2 + c) = u32x4{wg[0], wg[1], wg[2], wg[3]};
    if constexpr (SWIGLU)
      *reinterpret_cast<u32x4*>(dgu + r * ldc2 + dff + c) = u32x4{wu[0], wu[1], wu[2], wu[3]};
  };
  const long long total = R * cpr;
  if (total + (long long)gridDim.x * 256 < (1ll << 31)) {
    // 32-bit item index (the stride cannot overflow it): the division by
    // cpr stays a short 32-bit sequence
    const int tot = (int)total;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < tot; i += gridDim.x * 256) {
      const int r = i / cpr;
      item(r, (i - r * cpr) * 8);
    }
  } else {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (long long)gridDim.x * 256) {
      const long long r = i / cpr;
      item(r, (int)(i - r * cpr) * 8);
    }
  }
}

hipError_t run_act_bwd(bool swiglu, const float* P, int ldp, const void* dA, int ldd,
                       const int32_t* nrows_dev, int nrows_max, int dff, void* act, int ldc,
                       void* dgu, int ldc2, hipStream_t s) {
  const long long total = (long long)nrows_max * (dff / 8);
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const int nrows = nrows_dev != nullptr ? 0 : nrows_max;
  if (swiglu)
    hipLaunchKernelGGL(act_bwd_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, P, ldp,
                       static_cast<const uint16_t*>(dA), ldd, nrows_dev, nrows, dff,
                       static_cast<uint16_t*>(act), ldc, static_cast<uint16_t*>(dgu), ldc2);
  else
    hipLaunchKernelGGL(act_bwd_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, P, ldp,
                       static_cast<const uint16_t*>(dA), ldd, nrows_dev, nrows, dff,
                       static_cast<uint16_t*>(act), ldc, static_cast<uint16_t*>(dgu), ldc2);
  return hipGetLastError();
}
}  // namespace

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

// One launch over set s1 and, when s0 is given, the long tiles of s0 first.
// s1.C2 == null: plain outputs [M][ldc] per group; else both sets stored
// transposed, output column n < ct_split to row n of C, the others to row
// n - ct_split of C2.
hipError_t run_kgemm(const KGemmSet& s1, const KGemmSet* s0, hipStream_t s) {
  KGemmArgs k{};
  k.set[1] = s1;
  if (s0 != nullptr) {
    k.set[0] = *s0;
    k.head = (kgemm_tiles(*s0) + 7) / 8 * 8;
  }
  const long long blocks = (long long)k.head + kgemm_tiles(s1);
  if (blocks == 0) return hipSuccess;
  if (s1.C2 != nullptr)
    hipLaunchKernelGGL(grouped_kgemm_kernel<EPI_NONE_T>, dim3((unsigned)blocks), dim3(512), 0, s, k);
  else
    hipLaunchKernelGGL(grouped_kgemm_kernel<EPI_NONE>, dim3((unsigned)blocks), dim3(512), 0, s, k);
  return hipGetLastError();
}

// the routed experts' set: groups by offsets, AT columns by kpad
KGemmSet kgemm_set(const void* AT, int ldat, const void* B, int ldb, const int32_t* offsets,
                   const int32_t* kpad, int G, int M, int N, void* C, int ldc, size_t c_stride,
                   void* C2 = nullptr, int ct_split = 0) {
  KGemmSet k{};
  k.AT = AT;
  k.ldat = ldat;
  k.B = B;
  k.ldb = ldb;
  k.offsets = offsets;
  k.kpad = kpad;
  k.G = G;
  k.M = M;
  k.N = N;
  k.C = C;
  k.ldc = ldc;
  k.c_group_stride = c_stride;
  k.C2 = C2;
  k.ct_split = ct_split;
  return k;
}

// S [rows][C] -> T [C][ldt] per group (offsets null: rows1 rows, one group)
hipError_t run_transpose(const void* S, int lds, int C, const int32_t* offsets, const int32_t* kpad,
                         int G, void* T, int ldt, hipStream_t s, int rows1 = 0) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(ldt / 64));
  hipLaunchKernelGGL(transpose_groups_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(S),
                     lds, C, offsets, kpad, G, static_cast<uint16_t*>(T), ldt, rows1);
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
  const int bm = ffn_row_tile(rows_alloc, p.N, true);
  const int tail_rows = bm == 256 ? kTailRows : 0;
  const int ext_rows = bm == 256 ? kExtRows : 0;
  const int mtiles_max = (rows_alloc + bm - 1) / bm + p.N + (tail_rows > 0 ? p.N : 0);
  int32_t* tiles = b.tiles;
  int32_t* tails = tiles + (p.N + 2);
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, b.offsets, p.N, bm, tail_rows,
                     ext_rows, tiles, tails, nullptr);
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
  if (b.pre != nullptr)
    e = run_act_bwd(swiglu, b.pre, (swiglu ? 2 : 1) * dff, b.dA, dff, b.offsets + p.N, rows_alloc,
                    dff, b.act, dff, b.dgu, r1.ldc2, s);
  else
    e = run_bwd_epi(r1, swiglu, bm, mtiles_max, s);
  if (e != hipSuccess) return e;
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
  // [dG dU] (rows x 2 d_ff) is the large operand, as the activations are in
  // the forward down GEMM: the XCDs share it through the Infinity Cache
  n2.xcd_chunk = kXcdChunk;
  if ((e = launch_bf16<EPI_NONE, true>(n2, bm, mtiles_max, s)) != hipSuccess) return e;
  const int gu = swiglu ? 2 : 1;
  // shared experts' data gradients over all T tokens, dY = d_out
  const int dffs = p.d_ff_shared, wsw = p.n_shared * dffs;
  if (p.n_shared > 0) {
    const int sbm = ffn_row_tile(p.T, 1, true);
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
    sr.ldc2 = gu * wsw;
    if (b.pre_shared != nullptr)
      e = run_act_bwd(swiglu, b.pre_shared, gu * wsw, b.dA_s, wsw, nullptr, p.T, wsw, b.act_s, wsw,
                      b.dgu_s, sr.ldc2, s);
    else
      e = run_bwd_epi(sr, swiglu, sbm, mt, s);
    if (e != hipSuccess) return e;
    GemmArgs s2 = sb;
    s2.A = b.dgu_s;
    s2.lda = gu * wsw;
    s2.B0 = b.ws_gate;
    s2.B1 = b.ws_up;
    s2.ldb = d;
    s2.Kdim = gu * wsw;
    s2.kseg = wsw;
    s2.Ndim = d;
    s2.C = b.dx_shared;
    s2.ldc = d;
    if ((e = launch_bf16<EPI_NONE, true>(s2, sbm, mt, s)) != hipSuccess) return e;
  }

  // weight gradients
  if (b.kpad != nullptr) {
    // transposed form.  dW_down = dY^T a from dY transposed; [dW_gate;
    // dW_up]^T = X^T [dG dU] from X transposed (d columns rather than the
    // 2 d_ff of [dG dU]), the product stored transposed, split at d_ff.  The
    // shared experts' gradients (every token) run in the same launches as a
    // first set of long tiles: dWs_down[k] = d_out^T a_s[:, k-th d_ff_s
    // columns], [dWs_gate; dWs_up]^T = u^T [dG_s dU_s].
    hipLaunchKernelGGL(kpad_kernel, dim3(1), dim3(256), 0, s, b.offsets, p.N, b.kpad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const bool sh = p.n_shared > 0 && b.dOT != nullptr;
    KGemmSet sd{}, sg{};
    if (sh) {
      if ((e = run_transpose(b.d_out, d, d, nullptr, nullptr, 1, b.dOT, b.ldts, s, p.T)) != hipSuccess) return e;
      sd = kgemm_set(b.dOT, b.ldts, b.act_s, wsw, nullptr, nullptr, p.n_shared, d, dffs, b.dws_down, dffs,
                     (size_t)d * dffs);
      sd.rows = p.T;
      sd.b_group_cols = dffs;
    }
    if ((e = run_transpose(b.dy_perm, d, d, b.offsets, b.kpad, p.N, b.dyT, b.ldt, s)) != hipSuccess) return e;
    if ((e = run_kgemm(kgemm_set(b.dyT, b.ldt, b.act, dff, b.offsets, b.kpad, p.N, d, dff, b.dw_down, dff,
                                 (size_t)d * dff),
                       sh ? &sd : nullptr, s)) != hipSuccess)
      return e;
    if (sh) {
      if ((e = run_transpose(b.u, d, d, nullptr, nullptr, 1, b.uT, b.ldts, s, p.T)) != hipSuccess) return e;
      sg = kgemm_set(b.uT, b.ldts, b.dgu_s, gu * wsw, nullptr, nullptr, 1, d, gu * wsw, b.dws_gate, d, 0,
                     swiglu ? b.dws_up : b.dws_gate, wsw);
      sg.rows = p.T;
    }
    if ((e = run_transpose(b.x_perm, d, d, b.offsets, b.kpad, p.N, b.xT, b.ldt, s)) != hipSuccess) return e;
    if ((e = run_kgemm(kgemm_set(b.xT, b.ldt, b.dgu, gu * dff, b.offsets, b.kpad, p.N, d, gu * dff, b.dw_gate,
                                 d, (size_t)dff * d, swiglu ? b.dw_up : b.dw_gate, dff),
                       sh ? &sg : nullptr, s)) != hipSuccess)
      return e;
    if (sh || p.n_shared == 0) return hipSuccess;
  } else {
    if ((e = run_wgrad(wgrad_args(b.dy_perm, d, b.act, dff, b.offsets, p.N, 0, d, dff, b.dw_down,
                                  nullptr, d, (size_t)d * dff, dff, dff, 0),
                       s)) != hipSuccess)
      return e;
    if ((e = run_wgrad(wgrad_args(b.dgu, gu * dff, b.x_perm, d, b.offsets, p.N, 0, gu * dff, d,
                                  b.dw_gate, b.dw_up, dff, (size_t)dff * d, d, d, 0),
                       s)) != hipSuccess)
      return e;
    if (p.n_shared == 0) return hipSuccess;
  }
  // shared experts' weight gradients by the direct kernel
  if ((e = run_wgrad(wgrad_args(b.d_out, d, b.act_s, wsw, nullptr, 1, p.T, d, wsw, b.dws_down,
                                nullptr, d, 0, dffs, dffs, (size_t)d * dffs),
                     s)) != hipSuccess)
    return e;
  return run_wgrad(wgrad_args(b.dgu_s, gu * wsw, b.u, d, nullptr, 1, p.T, gu * wsw, d, b.dws_gate,
                              b.dws_up, wsw, 0, d, d, 0),
                   s);
}

}  // namespace moe
