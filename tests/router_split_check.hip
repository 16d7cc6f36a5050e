// Host check of the router's three-part bf16 split of fp32 weights
// (split3 in route.hip): hi + mid + lo must equal w exactly for every
// |w| >= 2^-90, each part must be a bf16 value (low 16 bits zero), and the
// split of a value that is already bf16 must be (w, 0, 0).
#include "route.hip"
#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
using namespace moe;
int main() {
  std::mt19937_64 rng(7);
  long long n = 0, bad = 0;
  auto check = [&](float w) {
    uint16_t hi, mid, lo;
    split3(w, hi, mid, lo);
    const double sum = (double)bf16_bits_to_f32(hi) + (double)bf16_bits_to_f32(mid) + (double)bf16_bits_to_f32(lo);
    ++n;
    if (sum != (double)w) {
      if (bad < 5) printf("inexact: %.9g -> %.9g\n", w, sum);
      ++bad;
    }
  };
  for (int i = 0; i < 4000000; ++i) {
    uint32_t b = (uint32_t)rng();
    float w;
    std::memcpy(&w, &b, 4);
    if (!std::isfinite(w) || std::fabs(w) < std::ldexp(1.0f, -90)) continue;
    check(w);
  }
  std::normal_distribution<float> nd(0.0f, 1.0f);
  for (float sc : {1e-20f, 1e-3f, 0.02f, 1.0f, 1e3f, 1e30f})
    for (int i = 0; i < 500000; ++i) check(nd(rng) * sc);
  for (float w : {0.0f, -0.0f, 1.0f, -1.0f, 2.0f, 0.5f, 3.0e38f, -3.0e38f, 1.0f + 1.0f / 4096.0f, 1.0f / 3.0f}) check(w);
  // values that are bf16 already split into themselves
  for (int i = 0; i < 100000; ++i) {
    uint32_t b = (uint32_t)rng() & 0xffff0000u;
    float w;
    std::memcpy(&w, &b, 4);
    if (!std::isfinite(w)) continue;
    uint16_t hi, mid, lo;
    split3(w, hi, mid, lo);
    ++n;
    if (hi != (b >> 16) || (mid & 0x7fff) != 0 || (lo & 0x7fff) != 0) ++bad;
  }
  printf("%lld cases, %lld failures\n", n, bad);
  return bad != 0;
}
