// Division by a runtime-invariant divisor with a multiply-high and shifts
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up method): exact for every 32-bit
// dividend.  The divisor's constants are computed once on the host.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CRU_HD __host__ __device__
#else
#define CRU_HD
#endif

namespace cru {

struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;       // l = ceil(log2 d)
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l > 0 ? 1 : 0;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

CRU_HD inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

}  // namespace cru
