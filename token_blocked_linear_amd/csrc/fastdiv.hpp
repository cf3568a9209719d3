// Division by a run-time invariant divisor with a multiply-high, shift and add (Granlund &
// Montgomery, "Division by invariant integers using multiplication", PLDI 1994):
//   s = ceil(log2 d),  m = floor(2^32 (2^s - d) / d) + 1,  q = (mulhi(n, m) + n) >> s,
// exact for every 0 <= n < 2^31 and 1 <= d < 2^31.  Used for token -> grid-coordinate maps.
// Plain C++ on the host (tested there), HIP on the device.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MHLA_HD __host__ __device__
#else
#define MHLA_HD
#endif

namespace mhla {

struct FastDiv {
  uint32_t d, m, s;
};

MHLA_HD inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}

MHLA_HD inline uint32_t fdiv(uint32_t n, FastDiv f) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t hi = __umulhi(n, f.m);
#else
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
  return (uint32_t)(((uint64_t)hi + n) >> f.s);
}

}  // namespace mhla
