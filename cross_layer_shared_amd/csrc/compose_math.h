// Element arithmetic of the KV composition (YOCO++ technical summary, section
// 2, KV composition equations), shared by the compose kernel and the decode
// that composes on read, so that both produce the same bits.
//
//   X' = c1 * X_1 + c2 * X_i,  c1 = fl32(lambda * a1), c2 = fl32(lambda * a2),
//
// evaluated as fma(c2, X_i, c1 * X_1) in fp32 and rounded once to the storage
// type (round to nearest even for bf16). A zero coefficient drops its term, so
// the initialisation a1 = 0, a2 = 1/lambda returns X_i bit for bit (signed
// zeros included).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace yoco {

__device__ __forceinline__ float compose_value(float x1, float xi, float c1, float c2, int terms) {
  switch (terms) {
    case 3: return __builtin_fmaf(c2, xi, c1 * x1);
    case 2: return c2 * xi;
    case 1: return c1 * x1;
    default: return 0.f;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t bf16_pack(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// One dword of stored values: two bf16 or one fp32.
template <bool BF16>
__device__ __forceinline__ uint32_t compose_dword(uint32_t x1, uint32_t xi, float c1, float c2, int terms) {
  if constexpr (BF16) {
    return bf16_pack(compose_value(bf16_lo(x1), bf16_lo(xi), c1, c2, terms),
                     compose_value(bf16_hi(x1), bf16_hi(xi), c1, c2, terms));
  } else {
    return __float_as_uint(compose_value(__uint_as_float(x1), __uint_as_float(xi), c1, c2, terms));
  }
}

}  // namespace yoco
