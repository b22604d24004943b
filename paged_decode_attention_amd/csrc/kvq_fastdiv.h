// Division of 32-bit unsigned integers by a divisor that is invariant across a launch
// (Granlund and Montgomery, "Division by Invariant Integers using Multiplication", PLDI 1994,
// the round-up multiplier of their Figure 4.1): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, every n < 2^32 has
//   n / d = (t + ((n - t) >> s1)) >> s2,  t = floor(n m / 2^32),  s1 = min(l, 1),  s2 = max(l - 1, 0).
// The host computes (m, s1, s2) once; the kernels' divisions by it are a multiply-high, a subtract,
// two shifts and an add (scalar instructions when n is uniform across the wave). Plain constexpr C++
// without GPU headers: the kernels and a host test compile the same functions.
#pragma once

#include <stdint.h>

namespace kvq {

struct FastDiv {
  uint32_t d, m;
  int32_t s1, s2;
};

// d = 0 is taken as 1 (no launch divides by an empty extent).
constexpr FastDiv make_fast_div(uint32_t d) {
  if (d == 0) d = 1;
  int l = 0;
  while ((uint64_t{1} << l) < d) ++l;
  FastDiv f{};
  f.d = d;
  f.m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

constexpr uint32_t fast_div(uint32_t n, const FastDiv& f) {
  const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

}  // namespace kvq
