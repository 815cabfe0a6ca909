// Index decompositions in the streaming kernels (compose and its backward).

#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace yoco {

// Unsigned division by a runtime-invariant divisor d >= 1 with one high
// multiply (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1,
// q = (t + ((x - t) >> 1)) >> (s - 1) with t = mulhi(x, m); s = 0 means d = 1.
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return {d, (uint32_t)m, s};
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
  if (f.s == 0) return x;
  const uint32_t t = (uint32_t)(((uint64_t)x * f.m) >> 32);   // high word of the product (v_mul_hi_u32)
  return (t + ((x - t) >> 1)) >> (f.s - 1);
}

}  // namespace yoco
