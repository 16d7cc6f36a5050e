// Host-side check of the k-major operand path of the grouped GEMM: the
// direct loads (kmajor_voff) followed by the transposing LDS reads
// (kmajor_read_off) must hand every lane the MFMA operand it needs, 8
// consecutive k of one column, and each half wave's reads must fall on
// distinct 16-byte bank groups.  The transposing read is emulated with the
// lane layout measured on the GPU: in each 16-lane group, lane i receives
// element i % 4 of the 8 bytes that lane 4j + i/4 addressed, as element j.
// Built with hipcc as a host program by tests/test_tile_plan.py.
#include "grouped_gemm.hip"
#include <cstdio>
#include <cstring>
#include <vector>
using namespace moe;
int main() {
  const int ld = 300 * 8;
  std::vector<uint16_t> G(64 * (size_t)ld);
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < ld; ++c) G[(size_t)r * ld + c] = (uint16_t)(r * 256 + c % 256);
  int fails = 0;
  for (int n0 : {0, 256, 512, 1024}) {
    std::vector<uint16_t> lds(64 * 256, 0xffff);
    const uint8_t* gb = (const uint8_t*)(G.data() + n0);
    for (int q = 0; q < 32; ++q)           // instruction q writes 1 KB: lane l at byte 16*l
      for (int lane = 0; lane < 64; ++lane)
        memcpy((uint8_t*)lds.data() + q * 1024 + lane * 16, gb + kmajor_voff(q, lane, ld), 16);
    const uint8_t* tile = (const uint8_t*)lds.data();
    for (int kk = 0; kk < 4; ++kk)
      for (int col0 = 0; col0 < 256; col0 += 32)
        for (int h = 0; h < 2; ++h) {
          int addr[64];
          for (int lane = 0; lane < 64; ++lane) addr[lane] = kmajor_read_off(kk, col0, lane) + h * 2048;
          for (int lane = 0; lane < 64; ++lane) {
            const int g0 = lane & ~15, i = lane & 15;
            for (int j = 0; j < 4; ++j) {
              uint16_t v;
              memcpy(&v, tile + addr[g0 + 4 * j + i / 4] + 2 * (i % 4), 2);
              const int k = 16 * kk + 8 * (lane >> 5) + 4 * h + j;
              const uint16_t want = (uint16_t)(k * 256 + (n0 + col0 + (lane & 31)) % 256);
              if (v != want) ++fails;
            }
          }
          for (int half = 0; half < 2; ++half) {
            int seen[16] = {0};
            for (int lane = 32 * half; lane < 32 * half + 32; lane += 2) seen[(addr[lane] / 16) % 16]++;
            for (int b = 0; b < 16; ++b) fails += seen[b] > 1;
          }
        }
  }
  printf("%d failures\n", fails);
  return fails != 0;
}
