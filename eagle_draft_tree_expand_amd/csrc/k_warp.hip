// Sampling warps: top-k and nucleus applied to logits rows (hubwiz section 2:
// with temperature, top-k or nucleus sampling, speculative decoding stays
// exact when both distributions are adjusted the same way before the test).
//
// A row's tokens are ordered by (t desc, id asc), t = fp32(z / T').  top-k
// keeps the first min(k, V); the nucleus then keeps the shortest prefix whose
// mass exp(t - M) reaches top_p of the top-k mass (the crossing token kept);
// at least min_keep tokens are kept.  The kept set is a prefix of the order,
// written as its last token: (code of t_b, id_b), where the code is the
// order-preserving unsigned image of t; token v is kept iff code_v > code_b,
// or code_v == code_b and v <= id_b.  Row stats: M = max t and S = the kept
// mass (fp64 sum, stored fp32), the statistics of the warped softmax.
//
// One workgroup of 1024 threads per row.  Each cut is a radix select on the
// 32-bit key ~code (ascending key = descending t) in four 8-bit passes over
// the row: a 256-bucket histogram of the weight (1 per token for counts,
// the mass for the nucleus) of the tokens that share the key prefix chosen
// so far, then the bucket where the running weight reaches the target; a
// last pass over the tokens equal to the chosen key, in id order, finds the
// token.  Masses are summed as fixed-point integers (2^mshift per unit, at
// most V * 2^mshift < 2^63): integer sums are exact and independent of the
// order of the atomic additions, so every run cuts at the same token.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kWThreads = 1024;
constexpr int kWWaves = kWThreads / 64;

EDEV uint32_t tcode(float t) {
  const uint32_t b = __float_as_uint(t + 0.0f);  // -0 -> +0: equal values tie
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

struct Cut {
  uint32_t key;  // ascending key of the last kept token (~code)
  int32_t id;
};

EDEV bool before_eq(uint32_t key, int v, const Cut& c) { return key < c.key || (key == c.key && v <= c.id); }

struct WarpSmem {
  unsigned long long hist[256];
  unsigned long long part[kWThreads / 64];
  double dred[kWWaves];
  float fred[kWWaves];
  uint32_t prefix;
  unsigned long long below;
  Cut cut;
  int bad;
};

// Block maximum (all threads).
EDEV float block_max(float v, WarpSmem& sm) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sm.fred[wave] = v;
  __syncthreads();
  float m = sm.fred[0];
  for (int w = 1; w < kWWaves; ++w) m = fmaxf(m, sm.fred[w]);
  __syncthreads();
  return m;
}

// Block sums in a fixed order (all threads get the same value).
EDEV double block_sum_d(double v, WarpSmem& sm) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sm.dred[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kWWaves; ++w) s += sm.dred[w];
  __syncthreads();
  return s;
}

EDEV unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

EDEV unsigned long long block_sum_u64(unsigned long long v, WarpSmem& sm) {
  v = wave_sum_u64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sm.part[wave] = v;
  __syncthreads();
  unsigned long long s = 0;
  for (int w = 0; w < kWWaves; ++w) s += sm.part[w];
  __syncthreads();
  return s;
}

struct RowCtx {
  const float* z;
  int V;
  float Tp;
  float M;
  double mscale;  // fixed-point units per unit mass
};

EDEV float t_of(const RowCtx& r, int v, int* bad) {
  const float z = r.z[v];
  if (!isfinite(z)) { *bad = 1; return kNegInf; }
  return z / r.Tp;
}

// Weight of token v in the select: 1 (count) or its fixed-point mass.
EDEV unsigned long long weight(const RowCtx& r, float t, bool mass) {
  if (!mass) return 1ull;
  if (t == kNegInf) return 0ull;
  return __double2ull_rn(exp((double)t - (double)r.M) * r.mscale);
}

// First token of the order (restricted to tokens before_eq `lim`) at which the
// running weight reaches `target` (all threads call; the result is uniform).
EDEV Cut select_cut(const RowCtx& r, const Cut& lim, bool mass, double target, WarpSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  int bad = 0;
  if (tid == 0) { sm.prefix = 0; sm.below = 0; }
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sm.hist[tid] = 0;
    __syncthreads();
    const uint32_t pre = sm.prefix;
    for (int v = tid; v < r.V; v += kWThreads) {
      const float t = t_of(r, v, &bad);
      const uint32_t key = ~tcode(t);
      if (!before_eq(key, v, lim)) continue;
      if (shift < 24 && (key >> (shift + 8)) != (pre >> (shift + 8))) continue;
      const unsigned long long w = weight(r, t, mass);
      if (w) atomicAdd(&sm.hist[(key >> shift) & 255], w);
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: four buckets per lane, prefix over the lanes
      unsigned long long h[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { h[i] = sm.hist[lane * 4 + i]; s += h[i]; }
      unsigned long long inc = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      const unsigned long long below = sm.below;
      const double exc = (double)(below + inc - s);
      const bool hit = (double)(below + inc) >= target && exc < target;
      const uint64_t ball = __ballot(hit);
      // rounding guard: no lane crossing (target above the total) takes the last non-empty bucket
      int l = ball ? __ffsll((long long)ball) - 1 : -1;
      if (l < 0) {
        const uint64_t ne = __ballot(s > 0);
        l = ne ? 63 - __clzll((long long)ne) : 0;
      }
      if (lane == l) {
        unsigned long long c = below + inc - s;
        int d = 3;
        for (int i = 0; i < 4; ++i) {
          if (h[i] > 0 && (double)(c + h[i]) >= target) { d = i; break; }
          c += h[i];
        }
        if (!hit) {  // the last non-empty bucket of this lane
          c = below + inc - s;
          for (int i = 3; i >= 0; --i)
            if (h[i] > 0) { d = i; break; }
          for (int i = 0; i < d; ++i) c += h[i];
        }
        sm.below = c;
        sm.prefix = pre | ((uint32_t)(lane * 4 + d) << shift);
      }
    }
    __syncthreads();
  }
  // tokens equal to the chosen key, in id order: contiguous id ranges per thread
  const uint32_t key = sm.prefix;
  const int C = (r.V + kWThreads - 1) / kWThreads;
  const int v0 = min(r.V, tid * C), v1 = min(r.V, v0 + C);
  unsigned long long mine = 0;
  for (int v = v0; v < v1; ++v) {
    const float t = t_of(r, v, &bad);
    if (~tcode(t) == key && before_eq(key, v, lim)) mine += weight(r, t, mass);
  }
  // exclusive prefix over threads (per wave, then wave totals)
  unsigned long long inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sm.part[tid >> 6] = inc;
  __syncthreads();
  unsigned long long wpre = 0;
  for (int w = 0; w < (tid >> 6); ++w) wpre += sm.part[w];
  const unsigned long long below = sm.below;
  const unsigned long long exc = below + wpre + inc - mine;
  if (tid == 0) sm.cut = Cut{key, -1};
  __syncthreads();
  if (mine > 0 && (double)exc < target && (double)(exc + mine) >= target) {
    unsigned long long c = exc;
    for (int v = v0; v < v1; ++v) {
      const float t = t_of(r, v, &bad);
      if (~tcode(t) != key || !before_eq(key, v, lim)) continue;
      c += weight(r, t, mass);
      if ((double)c >= target) { sm.cut = Cut{key, v}; break; }
    }
  }
  __syncthreads();
  if (sm.cut.id < 0) {  // rounding guard: the last token with this key
    if (tid == 0) {
      int last = -1;
      for (int v = r.V - 1; v >= 0 && last < 0; --v) {
        int b2 = 0;
        const float t = t_of(r, v, &b2);
        if (~tcode(t) == key && before_eq(key, v, lim)) last = v;
      }
      sm.cut.id = last < 0 ? 0 : last;
    }
    __syncthreads();
  }
  if (bad) sm.bad = 1;
  const Cut out = sm.cut;
  __syncthreads();
  return out;
}

__global__ __launch_bounds__(kWThreads) void warp_kernel(int V, int top_k, float top_p, int min_keep, float Tp,
                                                         int mshift, const float* __restrict__ z,
                                                         float* __restrict__ stats, uint32_t* __restrict__ bound,
                                                         int32_t* status) {
  __shared__ WarpSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x;
  RowCtx r;
  r.z = z + (size_t)row * V;
  r.V = V;
  r.Tp = Tp;
  r.mscale = ldexp(1.0, mshift);
  if (tid == 0) sm.bad = 0;
  int bad = 0;
  float lm = kNegInf;
  for (int v = tid; v < V; v += kWThreads) lm = fmaxf(lm, t_of(r, v, &bad));
  if (bad) sm.bad = 1;
  r.M = block_max(lm, sm);
  const Cut all{0xffffffffu, 0x7fffffff};
  Cut cut = all;
  int nA = V;
  if (top_k > 0 && top_k < V) {
    cut = select_cut(r, all, false, (double)top_k, sm);
    nA = top_k;
  }
  if (top_p < 1.0f) {
    unsigned long long sa = 0;
    for (int v = tid; v < V; v += kWThreads) {
      const float t = t_of(r, v, &bad);
      if (before_eq(~tcode(t), v, cut)) sa += weight(r, t, true);
    }
    sa = block_sum_u64(sa, sm);
    Cut c = select_cut(r, cut, true, (double)top_p * (double)sa, sm);
    if (min_keep > 1) {
      const Cut cm = select_cut(r, cut, false, (double)min(min_keep, nA), sm);
      if (cm.key > c.key || (cm.key == c.key && cm.id > c.id)) c = cm;
    }
    cut = c;
  }
  double s = 0.0;
  if (r.M != kNegInf)
    for (int v = tid; v < V; v += kWThreads) {
      const float t = t_of(r, v, &bad);
      if (t != kNegInf && before_eq(~tcode(t), v, cut)) s += exp((double)t - (double)r.M);
    }
  s = block_sum_d(s, sm);
  if (tid == 0) {
    stats[(size_t)row * 2] = r.M;
    stats[(size_t)row * 2 + 1] = (float)s;
    bound[(size_t)row * 2] = ~cut.key;
    bound[(size_t)row * 2 + 1] = (uint32_t)cut.id;
    if (sm.bad) set_status(status, EAGLE_STATUS_NONFINITE);
  }
}

}  // namespace

int warp_mass_shift(int V) {
  int lg = 0;
  while ((1 << lg) < V) ++lg;
  return 62 - lg;
}

hipError_t launch_warp(int rows, int V, int top_k, float top_p, int min_keep, float T, const float* z, float* stats,
                       uint32_t* bound, int32_t* status, hipStream_t st) {
  const float Tp = T > 0.f ? T : 1.0f;
  warp_kernel<<<rows, kWThreads, 0, st>>>(V, top_k, top_p, min_keep, Tp, warp_mass_shift(V), z, stats, bound, status);
  return hipGetLastError();
}

}  // namespace eagle
