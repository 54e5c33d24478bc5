// Checks mha::fast_div (csrc/mha_host.h) against plain division: the
// kernels decode block indices as (n + mulhi(n, mul)) >> shift, the same
// expression as below, for indices n in [0, 2^31) and divisors d in
// [1, 2^31).  Build: g++ -std=c++17 -I include -I <csrc> this mha_host.cpp.
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <vector>

#include "mha_host.h"

static uint32_t quotient(uint32_t n, const mha::FastDiv& f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (n + hi) >> f.shift;
}

int main() {
  std::vector<uint32_t> divisors;
  for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
  for (int s = 1; s <= 31; ++s) {
    const uint64_t p = (uint64_t)1 << s;
    for (int64_t e = -3; e <= 3; ++e) {
      const int64_t d = (int64_t)p + e;
      if (d >= 1 && d < ((int64_t)1 << 31)) divisors.push_back((uint32_t)d);
    }
  }
  std::mt19937_64 rng(7);
  for (int i = 0; i < 4000; ++i) divisors.push_back(1 + (uint32_t)(rng() % 0x7fffffffu));

  const uint32_t top = 0x7fffffffu;  // largest index
  long checks = 0, failed = 0;
  for (uint32_t d : divisors) {
    const mha::FastDiv f = mha::fast_div(d);
    if (f.d != d) ++failed;
    std::vector<uint32_t> ns;
    for (uint32_t n = 0; n < 300; ++n) ns.push_back(n);
    for (uint32_t n = top; n > top - 300; --n) ns.push_back(n);
    for (uint64_t k = 1; k * d <= top && k < 300; ++k) {  // around multiples of d
      const uint64_t base = k * d;
      for (int e = -1; e <= 1; ++e)
        if (base + e <= top) ns.push_back((uint32_t)(base + e));
    }
    const uint64_t last = (top / d) * (uint64_t)d;  // the largest multiple and its neighbours
    for (int e = -1; e <= 1; ++e)
      if (last + e <= top) ns.push_back((uint32_t)(last + e));
    for (int i = 0; i < 200; ++i) ns.push_back((uint32_t)(rng() % ((uint64_t)top + 1)));
    for (uint32_t n : ns) {
      ++checks;
      if (quotient(n, f) != n / d) {
        if (failed < 10) printf("d=%u n=%u: got %u, want %u\n", d, n, quotient(n, f), n / d);
        ++failed;
      }
    }
  }
  printf("fast_div: %ld checks, %ld failed\n", checks, failed);
  return failed != 0;
}
