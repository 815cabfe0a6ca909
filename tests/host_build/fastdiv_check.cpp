// Host check of the division by invariant integers (fastdiv.h) that the
// streaming kernels use to split a linear thread index into (batch, token,
// head, chunk): fdiv(x, make_fastdiv(d)) must equal x / d for every 32-bit x.
// Checked exhaustively for x < 2^24 with every divisor up to 64, and at the
// edges (0, multiples of d and their neighbours, the top of the 32-bit range)
// plus 10^6 seeded random x for divisors up to 2^20 and at powers of two and
// their neighbours up to 2^31. Prints "ok" and exits 0 on success.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "fastdiv.h"

static int failures = 0;

static void check(uint32_t x, uint32_t d, const yoco::FastDiv& f) {
  const uint32_t got = yoco::fdiv(x, f);
  if (got != x / d && failures++ < 10) fprintf(stderr, "FAIL fdiv(%u, %u) = %u, expected %u\n", x, d, got, x / d);
}

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}

int main() {
  for (uint32_t d = 1; d <= 64; ++d) {
    const yoco::FastDiv f = yoco::make_fastdiv(d);
    for (uint32_t x = 0; x < (1u << 24); ++x) check(x, d, f);
  }
  std::vector<uint32_t> divisors;
  for (uint32_t d = 1; d <= (1u << 20); d = d < 4096 ? d + 1 : d + 997) divisors.push_back(d);
  for (int k = 1; k <= 31; ++k) {
    divisors.push_back((1u << k) - 1);
    divisors.push_back(1u << k);
    divisors.push_back((1u << k) + 1);
  }
  for (uint32_t d : divisors) {
    const yoco::FastDiv f = yoco::make_fastdiv(d);
    const uint32_t top = 0xFFFFFFFFu;
    for (uint32_t x : {0u, 1u, d - 1, d, d + 1, top, top - 1, top - top % d, top - top % d - 1, 0x7FFFFFFFu,
                       0x80000000u})
      check(x, d, f);
    for (uint32_t m = 1; m < 64; ++m) {
      const uint64_t x = (uint64_t)d * (rnd() % ((uint64_t)top / d + 1));
      if (x <= top) {
        check((uint32_t)x, d, f);
        if (x > 0) check((uint32_t)x - 1, d, f);
        if (x < top) check((uint32_t)x + 1, d, f);
      }
    }
    for (int r = 0; r < (d <= 4096 ? 200 : 1000); ++r) check(rnd(), d, f);
  }
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
