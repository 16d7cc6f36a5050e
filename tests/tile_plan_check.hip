// Host-side check of the grouped-GEMM tile plan: for random and edge-case
// group sizes, the tiles that split_rows, find_tile_2d and find_tail assign
// to the launched grid cover every row of every group exactly once per
// column tile, stay inside their group and within the tile bodies' heights.
// Built with hipcc as a host program (no GPU needed) by tests/test_tile_plan.py.
#include "grouped_gemm.hip"
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <random>
using namespace moe;
static int check(const std::vector<int>& sizes, int ntiles, bool single, int BM, int tail, int ext) {
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
int main() {
  std::mt19937 rng(1);
  int fails = 0, n = 0;
  std::vector<std::vector<int>> fixed = {{257, 320, 321, 300, 0, 255, 1, 600}, {2057, 1968, 2004, 2073, 2088, 2072, 2032, 2090},
                                         {64, 65, 576, 512, 0, 0, 1, 319}, {2048, 2048}, {1}, {0, 0, 5}};
  for (auto& s : fixed) for (int nt : {1, 3, 4, 5, 16, 112}) { fails += check(s, nt, false, 256, 64, 64); ++n; }
  for (int M : {1, 26, 64, 65, 255, 256, 257, 320, 321, 1050, 8192, 16384, 16448, 16449})
    for (int nt : {1, 4, 7, 16}) { fails += check({M}, nt, true, 256, 64, 64); ++n; }
  for (int it = 0; it < 3000; ++it) {
    int G = 1 + rng() % 70;
    std::vector<int> s(G);
    for (auto& x : s) { int k = rng() % 4; x = k == 0 ? rng() % 70 : k == 1 ? 256 * (rng() % 9) + rng() % 80 : rng() % 3000; }
    int nt = 1 + rng() % 40;
    fails += check(s, nt, false, 256, 64, 64); ++n;
    fails += check(s, nt, false, 128, 0, 0); ++n;
    fails += check(s, nt, false, 32, 0, 0); ++n;
  }
  printf("%d cases, %d failures\n", n, fails);
  return fails != 0;
}
