// fastdiv.h -- division of non-negative 32-bit integers by a runtime-invariant
// divisor with one multiply-high, one add and one shift (Granlund & Montgomery,
// "Division by invariant integers using multiplication", round-up variant).
// Valid for dividends n < 2^31 and divisors 1 <= d < 2^31.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define DATTN_HD __host__ __device__ __forceinline__
#else
#define DATTN_HD inline
#endif

namespace dattn {

struct FastDiv {
  uint32_t d;    // divisor
  uint32_t mul;  // magic multiplier
  uint32_t shr;  // ceil(log2(d))
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

DATTN_HD uint32_t fdiv(uint32_t n, FastDiv f) {
  uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (hi + n) >> f.shr;
}

DATTN_HD uint32_t fmod_(uint32_t n, FastDiv f) { return n - fdiv(n, f) * f.d; }

}  // namespace dattn
