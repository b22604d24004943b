// Host check of the invariant-divisor division used for the kernels' block indices
// (paged_decode_attention_amd/csrc/kvq_fastdiv.h): fast_div(n, make_fast_div(d)) == n / d for
// divisors and numerators at the edges (powers of two and their neighbours, 1, the largest
// 32-bit values) and for pseudo-random pairs. Prints the number of pairs checked, exits 1 on
// the first mismatch.
#include <cstdio>
#include <vector>

#include "kvq_fastdiv.h"

static bool check(uint32_t n, uint32_t d) {
  const kvq::FastDiv f = kvq::make_fast_div(d);
  const uint32_t q = kvq::fast_div(n, f);
  if (q != n / d) {
    std::printf("mismatch: n=%u d=%u got %u want %u\n", n, d, q, n / d);
    return false;
  }
  return true;
}

int main() {
  std::vector<uint32_t> ds, ns;
  for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
  for (int k = 12; k < 32; ++k) {
    const uint32_t p = uint32_t{1} << k;
    ds.push_back(p - 1);
    ds.push_back(p);
    ds.push_back(p + 1);
  }
  ds.push_back(0xFFFFFFFFu);
  ds.push_back(0xFFFFFFFEu);
  for (uint32_t n = 0; n < 4096; ++n) ns.push_back(n);
  for (int k = 12; k < 32; ++k) {
    const uint32_t p = uint32_t{1} << k;
    ns.push_back(p - 1);
    ns.push_back(p);
    ns.push_back(p + 1);
  }
  ns.push_back(0xFFFFFFFFu);
  ns.push_back(0xFFFFFFFEu);
  uint64_t count = 0;
  for (uint32_t d : ds) {
    for (uint32_t n : ns) {
      if (!check(n, d)) return 1;
      ++count;
    }
    // multiples of d and their neighbours (the quotient steps there)
    for (uint64_t q = 1; q * d <= 0xFFFFFFFFull && q < 64; ++q) {
      const uint32_t base = static_cast<uint32_t>(q * d);
      if (!check(base, d) || !check(base - 1, d)) return 1;
      if (base != 0xFFFFFFFFu && !check(base + 1, d)) return 1;
      count += 3;
    }
  }
  uint64_t x = 0x9E3779B97F4A7C15ull;  // xorshift64 stream
  for (int i = 0; i < 2000000; ++i) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const uint32_t n = static_cast<uint32_t>(x);
    uint32_t d = static_cast<uint32_t>(x >> 32) >> (x & 31);
    if (d == 0) d = 1;
    if (!check(n, d)) return 1;
    ++count;
  }
  std::printf("fast_div: %llu pairs equal to integer division\n", static_cast<unsigned long long>(count));
  return 0;
}
