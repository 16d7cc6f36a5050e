// Host-side check of the grouped-GEMM tile plan: for random and edge-case
// group sizes, the tiles that split_rows, find_tile_2d and find_tail assign
// to the launched grid cover every row of every group exactly once per
// column tile, stay inside their group and within the tile bodies' heights;
// the persistent launch's queues hand out every tile slot once; and the
// split-K pieces of the tail tiles cover each tile's k range once; and the
// interleaved XCD order (xcd_pos) is a permutation of each launch's tiles.
// Built with hipcc as a host program (no GPU needed) by tests/test_tile_plan.py.
#include "grouped_gemm.hip"
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <random>
using namespace moe;
static int check(const std::vector<int>& sizes, int ntiles, bool single, int BM, int tail, int ext,
                 int chunk = 0) {
  int G = (int)sizes.size();
  std::vector<int32_t> off(G + 1, 0), tiles(G + 2, 0), tails(G + 2, 0);
  for (int g = 0; g < G; ++g) off[g + 1] = off[g] + sizes[g];
  for (int g = 0; g < G; ++g) {
    int f, t;
    split_rows(sizes[g], BM, tail, ext, f, t);
    tiles[g + 1] = tiles[g] + f;
    tails[g + 1] = tails[g] + t;
  }
  GemmArgs a{};
  a.offsets = single ? nullptr : off.data();
  a.tiles = single ? nullptr : tiles.data();
  a.tails = single ? nullptr : tails.data();
  a.tail_rows = tail; a.ext_rows = ext; a.G = G; a.M = single ? sizes[0] : 0;
  a.xcd_chunk = chunk;
  int R = off[G];
  int mtiles_max;
  if (single) { int f, t; split_rows(R, BM, tail, ext, f, t); mtiles_max = f + t; }
  else mtiles_max = (R + BM - 1) / BM + G + (tail > 0 ? G : 0);
  int grid = mtiles_max * ntiles;
  std::vector<int> cover((size_t)R * ntiles, 0);
  int real = full_tiles_total(a, BM) * ntiles;
  if (real > grid) { printf("real > grid\n"); return 1; }
  for (int h = 0; h < grid; ++h) {
    int g, row0, rows, nt;
    if (h < real) {
      find_tile_2d(a, BM, ntiles, h, real, g, row0, rows, nt);
      // without extended tiles (the persistent kernel) a group's last full
      // tile may report the rows up to the group's end; its body computes BM
      // rows and the tail tile takes the rest
      if (ext == 0 && rows > BM) rows = BM;
      if (rows <= 0 || rows > BM + ext) { printf("bad rows %d h=%d\n", rows, h); return 1; }
    } else if (find_tail(a, BM, ntiles, h - real, g, row0, rows, nt)) {
      if (rows <= 0 || rows > tail) { printf("bad tail rows %d\n", rows); return 1; }
    } else continue;
    if (nt < 0 || nt >= ntiles) { printf("bad nt\n"); return 1; }
    int gs = single ? 0 : off[g], ge = single ? R : off[g + 1];
    if (row0 < gs || row0 + rows > ge) { printf("tile outside group g=%d row0=%d rows=%d [%d,%d)\n", g, row0, rows, gs, ge); return 1; }
    for (int r = row0; r < row0 + rows; ++r) cover[(size_t)r * ntiles + nt]++;
  }
  for (size_t i = 0; i < cover.size(); ++i) if (cover[i] != 1) { printf("row %zu covered %d times\n", i / ntiles, cover[i]); return 1; }
  return 0;
}
// The persistent launch's work queues: blocks on 8 XCDs claim positions in
// random interleavings (own run first, then the other runs, then queue 8,
// with positions reserved one claim ahead as the kernel does); every tile
// slot of [0, total) must be handed out exactly once.
static int check_queues(const std::vector<int>& sizes, int ntiles, int blocks, std::mt19937& rng) {
  int G = (int)sizes.size();
  std::vector<int32_t> off(G + 1, 0), tiles(G + 2, 0), tails(G + 2, 0);
  for (int g = 0; g < G; ++g) off[g + 1] = off[g] + sizes[g];
  for (int g = 0; g < G; ++g) {
    int f, t;
    split_rows(sizes[g], 256, 64, 64, f, t);
    tiles[g + 1] = tiles[g] + f;
    tails[g + 1] = tails[g] + t;
  }
  GemmArgs a{};
  a.offsets = off.data(); a.tiles = tiles.data(); a.tails = tails.data();
  a.tail_rows = 64; a.ext_rows = 64; a.G = G;
  const int real = full_tiles_total(a, 256) * ntiles;
  const int total = real + tail_tiles_total(a, 256) * ntiles;
  const int full = real - real % 8, q = full / 8, rest = total - full;
  std::vector<int> counter(9, 0), cur(blocks, 0), spec(blocks, -1), seen(total, 0);
  std::vector<int> live;
  for (int b = 0; b < blocks; ++b) live.push_back(b);
  while (!live.empty()) {
    const size_t k = rng() % live.size();
    const int b = live[k], xcd = b & 7;
    int h = -1;
    while (cur[b] < 9) {
      const int y = cur[b] < 8 ? (xcd + cur[b]) & 7 : 8;
      const int t = (cur[b] == 0 && spec[b] >= 0) ? spec[b] : counter[y]++;
      spec[b] = -1;
      h = queue_slot(y, t, q, full, rest);
      if (h >= 0) break;
      ++cur[b];
    }
    spec[b] = cur[b] == 0 ? counter[xcd]++ : -1;
    if (h < 0) { live.erase(live.begin() + k); continue; }
    if (h >= total) { printf("slot %d past %d\n", h, total); return 1; }
    seen[h]++;
  }
  for (int h = 0; h < total; ++h) if (seen[h] != 1) { printf("slot %d claimed %d times\n", h, seen[h]); return 1; }
  return 0;
}

// The persistent plan with the tail tiles folded in (find_tile_fold_p): the
// slots [0, span) cover every row of every group once per column tile, full
// tiles computing 256 rows and tail tiles at most kTailRows, each inside its
// group.
static int check_fold(const std::vector<int>& sizes, int ntiles, int chunk) {
  int G = (int)sizes.size();
  std::vector<int32_t> off(G + 1, 0), tiles(G + 2, 0), tails(G + 2, 0);
  for (int g = 0; g < G; ++g) off[g + 1] = off[g] + sizes[g];
  for (int g = 0; g < G; ++g) {
    int f, t;
    split_rows(sizes[g], 256, kTailRows, 0, f, t);
    tiles[g + 1] = tiles[g] + f;
    tails[g + 1] = tails[g] + t;
  }
  GemmArgs a{};
  a.offsets = off.data(); a.tiles = tiles.data(); a.tails = tails.data();
  a.tail_rows = kTailRows; a.ext_rows = 0; a.G = G; a.xcd_chunk = chunk; a.fold_tails = 1;
  const PtrPlan pl = ptr_plan(a);
  const int R = off[G];
  const int span = fold_span(pl, G, ntiles);
  // padding: the tail part of each run is kFoldRun slots, the last run's
  // beyond its width empty
  const int tailed = tails[G], runs = (ntiles + kFoldRun - 1) / kFoldRun;
  const int expect_empty = tailed * (runs * kFoldRun - ntiles);
  int empty = 0;
  std::vector<int> cover((size_t)R * ntiles, 0);
  for (int h = 0; h < span; ++h) {
    int g, row0, rows, nt, bm;
    if (!find_tile_fold_p(a, pl, ntiles, h, span, g, row0, rows, nt, bm)) { ++empty; continue; }
    if (bm == 256 && rows > 256) rows = 256;   // the tile body computes 256 rows
    if (bm != 256 && (bm != kTailRows || rows > kTailRows)) { printf("fold: bm %d rows %d\n", bm, rows); return 1; }
    if (rows <= 0 || nt < 0 || nt >= ntiles) { printf("fold: rows %d nt %d\n", rows, nt); return 1; }
    if (row0 < off[g] || row0 + rows > off[g + 1]) { printf("fold: tile outside group %d\n", g); return 1; }
    for (int r = row0; r < row0 + rows; ++r) cover[(size_t)r * ntiles + nt]++;
  }
  for (size_t i = 0; i < cover.size(); ++i) if (cover[i] != 1) { printf("fold: row %zu covered %d times\n", i / ntiles, cover[i]); return 1; }
  if (empty != expect_empty) { printf("fold: %d empty slots, expected %d\n", empty, expect_empty); return 1; }
  return 0;
}

// The interleaved XCD order: (y, t) for y < 8, t < q maps onto [0, 8q)
// one to one, and P = 0 is the contiguous run.
static int check_xcd_pos(int q, int P) {
  std::vector<int> seen(8 * (size_t)q, 0);
  for (int y = 0; y < 8; ++y)
    for (int t = 0; t < q; ++t) {
      const int L = xcd_pos(y, t, q, P);
      if (L < 0 || L >= 8 * q) { printf("xcd_pos(%d,%d,%d,%d)=%d\n", y, t, q, P, L); return 1; }
      if (P == 0 && L != y * q + t) { printf("xcd_pos contiguous\n"); return 1; }
      seen[L]++;
    }
  for (int L = 0; L < 8 * q; ++L) if (seen[L] != 1) { printf("xcd_pos q=%d P=%d: %d seen %d\n", q, P, L, seen[L]); return 1; }
  return 0;
}

// Split-K of the tail tiles: the piece count stays within the partial-sum
// slots and the blocks, each piece has at least 4 stages, and the pieces of
// a tile cover its stages 0 .. nk-1 exactly once, in order.
static int check_split(int tail_tiles, int blocks, int nk) {
  const int S = split_pieces(tail_tiles, blocks, nk);
  if (S < 1 || S > 4) { printf("S=%d\n", S); return 1; }
  if (S > 1 && (S * tail_tiles > kSplitSlots || S * tail_tiles > blocks)) {
    printf("S=%d tails=%d blocks=%d\n", S, tail_tiles, blocks);
    return 1;
  }
  int next = 0;
  for (int p = 0; p < S; ++p) {
    int kt0, n;
    split_range(p, S, nk, kt0, n);
    if (kt0 != next || n < (S > 1 ? 4 : 1)) { printf("piece %d of %d: %d+%d, nk=%d\n", p, S, kt0, n, nk); return 1; }
    next = kt0 + n;
  }
  if (next != nk) { printf("pieces end at %d, nk=%d\n", next, nk); return 1; }
  return 0;
}

int main() {
  std::mt19937 rng(1);
  int fails = 0, n = 0;
  std::vector<std::vector<int>> fixed = {{257, 320, 321, 300, 0, 255, 1, 600}, {2057, 1968, 2004, 2073, 2088, 2072, 2032, 2090},
                                         {64, 65, 576, 512, 0, 0, 1, 319}, {2048, 2048}, {1}, {0, 0, 5}};
  for (auto& s : fixed)
    for (int nt : {1, 3, 4, 5, 16, 112})
      for (int chunk : {0, 32, 7}) { fails += check(s, nt, false, 256, 64, 64, chunk); ++n; }
  for (auto& s : fixed)
    for (int nt : {1, 3, 4, 5, 16, 31, 32, 33, 40, 112})
      for (int chunk : {0, 32}) { fails += check_fold(s, nt, chunk); ++n; }
  for (int q : {0, 1, 5, 31, 32, 33, 64, 100, 128, 1000})
    for (int P : {0, 1, 7, 32, 64}) { fails += check_xcd_pos(q, P); ++n; }
  for (int M : {1, 26, 64, 65, 255, 256, 257, 320, 321, 1050, 8192, 16384, 16448, 16449})
    for (int nt : {1, 4, 7, 16}) { fails += check({M}, nt, true, 256, 64, 64); ++n; }
  for (int it = 0; it < 3000; ++it) {
    int G = 1 + rng() % 70;
    std::vector<int> s(G);
    for (auto& x : s) { int k = rng() % 4; x = k == 0 ? rng() % 70 : k == 1 ? 256 * (rng() % 9) + rng() % 80 : rng() % 3000; }
    int nt = 1 + rng() % 40;
    fails += check(s, nt, false, 256, 64, 64); ++n;
    fails += check(s, nt, false, 256, 64, 0, 32); ++n;
    fails += check_fold(s, 1 + rng() % 120, rng() % 2 ? 32 : 0); ++n;
    fails += check(s, nt, false, 128, 0, 0); ++n;
    fails += check(s, nt, false, 32, 0, 0); ++n;
  }
  for (int it = 0; it < 400; ++it) {
    int G = 1 + rng() % 64;
    std::vector<int> s(G);
    for (auto& x : s) { int k = rng() % 3; x = k == 0 ? rng() % 70 : k == 1 ? 256 * (rng() % 9) + rng() % 80 : rng() % 3000; }
    fails += check_queues(s, 1 + rng() % 120, 8 * (1 + rng() % 32), rng); ++n;
  }
  for (int tt : {0, 1, 2, 12, 63, 64, 65, 80, 85, 128, 129, 256, 300})
    for (int blocks : {8, 64, 248, 256, 304})
      for (int nk : {1, 3, 4, 7, 8, 16, 22, 224, 225}) {
        if (tt == 0) continue;
        fails += check_split(tt, blocks, nk); ++n;
      }
  for (int it = 0; it < 20000; ++it) {
    fails += check_split(1 + rng() % 400, 8 * (1 + rng() % 40), 1 + rng() % 500); ++n;
  }
  printf("%d cases, %d failures\n", n, fails);
  return fails != 0;
}
