// Division by a divisor fixed for the whole launch as a multiply-high and a
// shift (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, section 4): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (umulhi(m, n) + n) >> l for
// 0 <= n < 2^31 (umulhi(m, n) <= n, so the sum fits in 32 bits).  The host
// computes (m, l); kernels apply it with __umulhi.  Plain C++ (no HIP), so
// that a host-only test can check it.
#pragma once

#include <stdint.h>

namespace attn {

struct FastDiv {
  uint32_t m, l;
};

// d >= 1.
inline FastDiv make_fastdiv(int32_t d) {
  FastDiv f;
  uint32_t l = 0;
  while (l < 31 && (1u << l) < (uint32_t)d) ++l;
  f.l = l;
  f.m = (uint32_t)((((uint64_t)1 << l) - (uint64_t)d) * ((uint64_t)1 << 32) / (uint64_t)d) + 1u;
  return f;
}

// The kernels' arithmetic, on the host.
inline uint32_t fastdiv_apply(uint32_t n, FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)f.m * n) >> 32);
  return (hi + n) >> f.l;
}

}  // namespace attn
