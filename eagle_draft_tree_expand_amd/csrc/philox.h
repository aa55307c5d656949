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
    // one 32x32 -> 64-bit product per multiplier (both halves at once)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
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

// The same noise straight from a Philox word, cheaper, for the bulk scan:
// u = (2j+1) 2^-24 and 1-u are both exact; -ln u is 5 terms of the series of
// -ln(1-d) in d = 1-u while d < 1/16 (truncation below 2e-7 relative) and
// the hardware log2 otherwise; then -ln of that with the hardware log2.
// Measured over all 2^23 possible words against the fp64 noise: the absolute
// error stays below 2e-6, well inside the candidate key slack (>= 1.9e-5).
EDEV float gumbel_fast(uint32_t x) {
  constexpr float kLn2 = 0.693147180559945309f;
  const uint32_t n = 2u * (x >> 9) + 1u;
  const float u = (float)n * 5.9604644775390625e-8f;
  const float d = (float)((1u << 24) - n) * 5.9604644775390625e-8f;
  const float e_log = -__builtin_amdgcn_logf(u) * kLn2;
  const float e_ser = d * (1.f + d * (0.5f + d * (0.333333333f + d * (0.25f + d * 0.2f))));
  const float e = d < 0.0625f ? e_ser : e_log;
  return -__builtin_amdgcn_logf(e) * kLn2;
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
