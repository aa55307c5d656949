// Device helpers shared by the libeagle kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/eagle.h"

#define EDEV __device__ __forceinline__

namespace eagle {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kIdxNone = 0x7fffffff;  // loses every (key desc, idx asc) tie

EDEV float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
EDEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// s_waitcnt immediate for lgkmcnt(0) (LDS operations done), other counters
// unconstrained.
constexpr int kLgkmWait0 = 0xF | (7 << 4) | (3 << 14);

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its global loads (a __syncthreads also waits for every load in flight, which
// would drain a prefetch pipeline).  Callers wait for the global data they
// publish through LDS themselves (the compiler does, before each LDS write of
// loaded registers).
EDEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkmWait0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DPP moves inside a row of 16 lanes, instead of LDS-routed shuffles: swap
// within pairs, within quads, mirror within halves of 8, mirror within the
// row.  Applied in this order, each step pairs every lane with a distinct
// partner in the other half of its current group of 2, 4, 8, 16 lanes, so a
// reduction over such a group ends with the same result in all its lanes.
template <int CTRL>
EDEV int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
EDEV float dpp_f(float v) { return __int_as_float(dpp_i<CTRL>(__float_as_int(v))); }
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

EDEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

EDEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// fp64 sum over the wave: DPP pair/quad/half/row steps (each lane adds its
// partner's value; addition commutes, so all lanes of a row agree bit for
// bit), then the four row sums read from lanes 0, 16, 32, 48 and added in a
// fixed order.  Every lane returns the same value.
template <int CTRL>
EDEV double dpp_d(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>((int)(x & 0xffffffffll)), hi = dpp_i<CTRL>((int)(x >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
EDEV double lane_d(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(x & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
EDEV double wave_sum_d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

EDEV int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

EDEV int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// (key desc, idx asc) order.
EDEV bool beats(float ka, int ia, float kb, int ib) { return ka > kb || (ka == kb && ia < ib); }
EDEV bool beats_d(double ka, int ia, double kb, int ib) { return ka > kb || (ka == kb && ia < ib); }

// Wave-wide argmax under (key desc, idx asc); every lane ends with the winner.
EDEV void wave_argmax(float& key, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float k2 = __shfl_xor(key, o);
    int i2 = __shfl_xor(idx, o);
    if (beats(k2, i2, key, idx)) { key = k2; idx = i2; }
  }
}

EDEV void wave_argmax_d(double& key, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    double k2 = __shfl_xor(key, o);
    int i2 = __shfl_xor(idx, o);
    if (beats_d(k2, i2, key, idx)) { key = k2; idx = i2; }
  }
}

// Order-preserving unsigned image of an fp32 value (-0 counts as +0), and the
// sampling-warp membership test: token v with scaled logit t is kept by a
// row's warp iff it sorts at or before the row's last kept token (code_b,
// id_b) in the order (t desc, id asc).
EDEV uint32_t tcode(float t) {
  const uint32_t b = __float_as_uint(t + 0.0f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
EDEV bool warp_keeps(float t, int v, uint32_t code_b, uint32_t id_b) {
  const uint32_t c = tcode(t);
  return c > code_b || (c == code_b && (uint32_t)v <= id_b);
}

// Compact target rows: a logit as the fp16 offset from its 128-column block
// maximum m (round to nearest even; -inf for non-finite logits and for blocks
// without a finite one), and the value every use reads, fp32(m + offset).
constexpr int kCmpBlockShift = 7;  // 128 columns per block
EDEV uint16_t cmp_encode(float z, float m) {
  if (z == kNegInf || m == kNegInf) return 0xFC00u;  // fp16 -inf
  const _Float16 h = (_Float16)(z - m);
  return __builtin_bit_cast(uint16_t, h);
}
EDEV float cmp_decode(uint16_t h, float m) {
  const float d = (float)__builtin_bit_cast(_Float16, h);
  return d == kNegInf ? kNegInf : m + d;
}

EDEV void set_status(int32_t* st, int bits) {
  if (st) atomicOr(st, bits);
}

// Index i of an LDS array of n elements.  The debug library (built with
// EAGLE_LDS_CHECK) checks it: an index outside [0, n) is clamped into the
// array and EAGLE_STATUS_LDS_INDEX is set, so tests can assert that no access
// of the tree assembly or the walk left its array.  Release builds return i.
EDEV int lds_index(int i, int n, int32_t* st) {
#ifdef EAGLE_LDS_CHECK
  if ((unsigned)i >= (unsigned)n) {
    set_status(st, EAGLE_STATUS_LDS_INDEX);
    return i < 0 ? 0 : n - 1;
  }
#else
  (void)n;
  (void)st;
#endif
  return i;
}

}  // namespace eagle
