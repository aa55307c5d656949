// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11), device side, and the Gumbel noise built on it.
#pragma once
#include "common.h"

namespace eagle {

EDEV uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Odd multiple of 2^-24 in (0, 1), exact in fp32.
EDEV float word_to_uniform(uint32_t x) { return (float)(2u * (x >> 9) + 1u) * 5.9604644775390625e-8f; }

// Gumbel noise -ln(-ln u) in fp32 (used to preselect candidates).  -ln u is
// taken as -log1p(-(1-u)) above 1/2 so it keeps its relative precision near 1.
EDEV float gumbel_f32(float u) {
  const float e = (u > 0.5f) ? -log1pf(-(1.0f - u)) : -logf(u);
  return -logf(e);
}

// The same noise in fp64 (the value the child order is decided on).
EDEV double gumbel_f64(float uf) {
  const double u = (double)uf;
  const double e = (u > 0.5) ? -log1p(-(1.0 - u)) : -log(u);
  return -log(e);
}

// Uniform of token v in slot row (s, b) of round `round_lo`.
EDEV float token_uniform(int v, int s, int b, uint32_t round_lo, uint32_t k0, uint32_t k1) {
  const uint4 w = philox4x32_10(make_uint4((uint32_t)v >> 2, (uint32_t)s, (uint32_t)b, round_lo), k0, k1);
  const int j = v & 3;
  const uint32_t x = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
  return word_to_uniform(x);
}

}  // namespace eagle
