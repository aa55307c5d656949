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
// mass (stored fp32), the statistics of the warped softmax.
//
// One workgroup of 1024 threads per row.  Masses are fixed-point integers
// (2^mshift per unit, at most V * 2^mshift < 2^63): integer sums are exact and
// independent of the order of the atomic additions, so every run cuts at the
// same token.
//
// A top-k cut of at most 1024 tokens takes one pass: a bound estimated from
// the first batch lists the tokens at or above it in LDS, where they are
// ranked (onepass_topk); the nucleus, min_keep, M and S then come from the
// list.  Otherwise each cut is a radix select on the 32-bit key ~code
// (ascending key = descending t), digits of 12, 10 and 10 bits: a 4096- or
// 1024-bucket histogram of the weight (1 per token for counts, the mass for
// the nucleus) of the tokens sharing the key prefix chosen so far, then the
// bucket where the running weight reaches the target; the tokens equal to
// the chosen key, in id order, give the token.  A wave whose lanes share a
// bucket adds their summed weight with one atomic instead of 64.  For a
// nucleus the first digit comes from the row and the rest from an LDS list
// of the crossing bucket's tokens (select_nucleus), and S is the fixed-point
// mass through the cut.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kWThreads = 1024;
constexpr int kWWaves = kWThreads / 64;

struct Cut {
  uint32_t key;  // ascending key of the last kept token (~code)
  int32_t id;
};

EDEV bool before_eq(uint32_t key, int v, const Cut& c) { return key < c.key || (key == c.key && v <= c.id); }

constexpr int kWBuckets = 4096;
constexpr int kWList = 64;  // tokens tied at a cut key handled in wave 0
constexpr int kWL2 = 4096;  // tokens of a nucleus's first-digit bucket listed in LDS

// A top-k cut of at most this many tokens finishes in LDS: the kept tokens
// are listed once, sorted, and the nucleus, min_keep cut, M and S are taken
// from the list instead of further passes over the row.
constexpr int kWFast = 1024;
static_assert(kWFast == kWThreads, "one rank counter per thread");

struct FastList {
  uint32_t key[kWFast];  // gathered, unordered
  int id[kWFast];
  float t[kWFast];
  uint32_t skey[kWFast];  // sorted by (key asc, id asc) = the order
  int sid[kWFast];
  float st[kWFast];
  int n;
  int ci;
};

struct WarpSmem {
  FastList fl;
  union {
    unsigned long long hist[kWBuckets];  // radix passes
    unsigned long long pk[kWFast];       // one-pass list: (key << 32) | id
  };
  uint32_t est[kWWaves];
  uint32_t lzc;
  double e2[256];            // 2^(j/256), the mass table
  unsigned long long lk[kWL2];  // nucleus bucket list: (key << 32) | id
  float lt[kWL2];               // and t
  int n2;
  double tgt;                // a select's target (set by its first pass when taken as a fraction)
  unsigned long long cum;    // fixed-point mass through a select's cut token
  int cum_ok;
  unsigned long long part[kWThreads / 64];
  double dred[kWWaves];
  float fred[kWWaves];
  int list_id[kWList], sort_id[kWList];
  unsigned long long list_w[kWList], sort_w[kWList];
  int nlist;
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
  bool vec;  // row 16-byte aligned and V % 4 == 0: 16-byte loads
  int V;
  float Tp;
  float M;
  int mshift;        // fixed-point units per unit mass: 2^mshift
  const double* e2;  // 2^(j/256), j < 256 (LDS)
};

EDEV float t_from(const RowCtx& r, float z, int* bad) {
  if (!isfinite(z)) { *bad = 1; return kNegInf; }
  return r.Tp == 1.0f ? z : z / r.Tp;
}
EDEV float t_of(const RowCtx& r, int v, int* bad) { return t_from(r, r.z[v], bad); }

// The row is walked in batches of kWE = 16 tokens per thread, all of a
// batch's loads issued before the first is used (one memory latency per
// batch): four 16-byte loads (token v0 + 4 (j * 1024 + tid) + e) when the
// row allows, else 16 scalar loads (token v0 + (4 j + e) * 1024 + tid).
constexpr int kWU = 4;
constexpr int kWE = 4 * kWU;
constexpr int kWBatch = kWThreads * kWE;
EDEV int tok_of(const RowCtx& r, int v0, int i) {  // token of batch element i = 4 j + e
  return r.vec ? v0 + ((i >> 2) * kWThreads + (int)threadIdx.x) * 4 + (i & 3) : v0 + i * kWThreads + (int)threadIdx.x;
}
EDEV void load_batch(const RowCtx& r, int v0, float (&zz)[kWE]) {
  if (r.vec) {
#pragma unroll
    for (int j = 0; j < kWU; ++j) {
      const int base = v0 + (j * kWThreads + (int)threadIdx.x) * 4;
      float4 q = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
      if (base < r.V) q = *reinterpret_cast<const float4*>(r.z + base);  // V % 4 == 0: all 4 in range
      zz[4 * j] = q.x; zz[4 * j + 1] = q.y; zz[4 * j + 2] = q.z; zz[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kWE; ++i) {
      const int v = tok_of(r, v0, i);
      zz[i] = v < r.V ? r.z[v] : kNegInf;
    }
  }
}

// One pass over the row, batch by batch in order, two batches' loads in
// flight while f(zz, b) takes batch b (all threads call f for every batch).
// The loads are branch-free, so the compiler's wait for one batch does not
// also wait for the batches behind it: lanes past the row read its last
// element (f masks them by index, rowscan_tok(...) < V) and batch indices
// past the end read the last batch again.
template <bool VEC>
EDEV int rowscan_tok(int v0, int i) {
  return VEC ? v0 + ((i >> 2) * kWThreads + (int)threadIdx.x) * 4 + (i & 3) : v0 + i * kWThreads + (int)threadIdx.x;
}
template <bool VEC>
EDEV void rowscan_load(const RowCtx& r, int nb, int b, float (&zz)[kWE]) {
  const int v0 = min(b, nb - 1) * kWBatch, tid = threadIdx.x;
  if (VEC) {
#pragma unroll
    for (int j = 0; j < kWU; ++j) {
      const float4 q = *reinterpret_cast<const float4*>(r.z + min(v0 + (j * kWThreads + tid) * 4, r.V - 4));
      zz[4 * j] = q.x; zz[4 * j + 1] = q.y; zz[4 * j + 2] = q.z; zz[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kWE; ++i) zz[i] = r.z[min(v0 + i * kWThreads + tid, r.V - 1)];
  }
}
template <bool VEC, class F>
EDEV void scan_row(const RowCtx& r, F&& f) {
  const int nb = (r.V + kWBatch - 1) / kWBatch;
  float za[kWE], zb[kWE], zc[kWE];
  rowscan_load<VEC>(r, nb, 0, za);
  rowscan_load<VEC>(r, nb, 1, zb);
  rowscan_load<VEC>(r, nb, 2, zc);
  f(za, 0);
  for (int b = 1; b < nb; b += 3) {  // batch b sits in za, zb, zc by b % 3
    rowscan_load<VEC>(r, nb, b + 2, za);
    f(zb, b);
    rowscan_load<VEC>(r, nb, b + 3, zb);
    if (b + 1 < nb) f(zc, b + 1);
    rowscan_load<VEC>(r, nb, b + 4, zc);
    if (b + 2 < nb) f(za, b + 2);
  }
}

// Fixed-point mass round(2^mshift exp(x)) of x = t - M <= 0 (exact in fp64:
// t and M are fp32).  Tang's table method (ACM TOMS 15(2), 1989): x =
// (256 e + j) ln2/256 + r with |r| <= ln2/512, exp(x) = 2^e 2^(j/256) e^r, e^r
// by its Taylor series to r^5 (truncation below 1e-20).  Relative error a few
// 1e-16, against 2^-mshift for the rounding to an integer.
EDEV unsigned long long mass_fixed(double x, const RowCtx& r) {
  if (!(x > -44.0)) return 0ull;  // below 2^mshift e^-44 < 1/2 (mshift <= 62); also -inf
  constexpr double kInvL = 369.3299304675746;       // 256 / ln 2
  constexpr double kL1 = 0x1.62e42fefa0000p-9;      // ln 2 / 256, leading 38 bits
  constexpr double kL2 = 0x1.cf79abc9e3b3ap-48;     // the rest
  const double kd = rint(x * kInvL);
  const int k = (int)kd;
  const double rr = fma(-kd, kL2, fma(-kd, kL1, x));  // kd * kL1 is exact (|k| < 2^15)
  const double q = rr * fma(rr, fma(rr, fma(rr, fma(rr, 1.0 / 120, 1.0 / 24), 1.0 / 6), 0.5), 1.0);  // e^r - 1
  const double tj = r.e2[k & 255];
  const double v = ldexp(fma(tj, q, tj), r.mshift + (k >> 8));  // <= 2^mshift
  return __double2ull_rn(v);
}

// Weight of token v in the select: 1 (count) or its fixed-point mass.
EDEV unsigned long long weight(const RowCtx& r, float t, bool mass) {
  if (!mass) return 1ull;
  if (t == kNegInf) return 0ull;
  return mass_fixed((double)t - (double)r.M, r);
}

// First token of the order (restricted to tokens before_eq `lim`) at which the
// running weight reaches `target` (all threads call; the result is uniform).
// key_only: stop after the first npass digit passes and return {key prefix
// of the crossing token, -1} (sm.below = weight of the tokens with smaller
// key prefixes; after one pass sm.hist still holds the first digit's counts).
//
// frac > 0: the target is frac times the total weight of the tokens before
// `lim`, taken from the first pass's histogram (the same integer sum a
// separate pass would give).  On return sm.cum holds the weight through the
// cut token when sm.cum_ok (a crossing was found, not the rounding guard).
// pass0 > 0 resumes a select whose earlier digits (sm.prefix, sm.below) are
// settled; n2 >= 0 then takes the tokens from the LDS list sm.lk/sm.lt (every
// token sharing those digits, n2 of them) instead of the row.
EDEV Cut select_cut(const RowCtx& r, const Cut& lim, bool mass, double target, WarpSmem& sm, bool key_only = false,
                    int npass = 3, double frac = 0.0, int pass0 = 0, int n2 = -1) {
  const int tid = threadIdx.x, lane = tid & 63;
  int bad = 0;
  if (tid == 0) {
    if (pass0 == 0) { sm.prefix = 0; sm.below = 0; }
    sm.cum_ok = 0;
  }
  // digits: key bits [31:20], [19:10], [9:0]
  for (int pass = pass0; pass < (key_only ? npass : 3); ++pass) {
    const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
    const int nb = pass == 0 ? 4096 : 1024;
    for (int x = tid; x < kWBuckets; x += kWThreads) sm.hist[x] = 0;
    __syncthreads();
    const uint32_t pre = sm.prefix;
    const int hshift = pass == 0 ? 32 : pass == 1 ? 20 : 10;  // bits above this digit must match
    auto add = [&](bool valid, uint32_t key, int v, float t) {
      int d = -1;
      unsigned long long w = 0;
      if (valid && before_eq(key, v, lim) && (hshift == 32 || (key >> hshift) == (pre >> hshift))) {
        w = weight(r, t, mass);
        if (w) d = (int)((key >> shift) & (uint32_t)(nb - 1));
      }
      // one atomic per wave when every contributing lane shares the bucket
      const uint64_t act = __ballot(d >= 0);
      if (act == 0ull) return;
      const int d0 = __builtin_amdgcn_readlane(d, __ffsll((long long)act) - 1);
      if (__ballot(d >= 0 && d != d0) == 0ull) {
        // counts: the ballot's population; masses: an integer sum over the
        // wave (64-bit shuffles), exact for every vocabulary size
        const unsigned long long tot = mass ? wave_sum_u64(w) : (unsigned long long)__popcll(act);
        if (lane == __ffsll((long long)act) - 1) atomicAdd(&sm.hist[d0], tot);
      } else if (d >= 0) {
        atomicAdd(&sm.hist[d], w);
      }
    };
    if (n2 >= 0) {
      for (int i0 = 0; i0 < n2; i0 += kWThreads) {
        const int i = i0 + tid;
        const bool ok = i < n2;
        const unsigned long long e = ok ? sm.lk[i] : 0ull;
        add(ok, (uint32_t)(e >> 32), (int)(uint32_t)e, ok ? sm.lt[i] : kNegInf);
      }
    } else {  // one batch in flight: a mass pass is bound by its arithmetic
      for (int v0 = 0; v0 < r.V; v0 += kWBatch) {
        float zz[kWE];
        load_batch(r, v0, zz);
#pragma unroll
        for (int j = 0; j < kWE; ++j) {
          const int v = tok_of(r, v0, j);
          const bool ok = v < r.V;
          const float t = ok ? t_from(r, zz[j], &bad) : kNegInf;
          add(ok, ~tcode(t), v, t);
        }
      }
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: nb / 64 buckets per lane, prefix over the lanes
      const int per = nb / 64;
      unsigned long long s = 0;
      for (int i = 0; i < per; ++i) s += sm.hist[lane * per + i];
      unsigned long long inc = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      if (pass == 0 && frac > 0.0) {
        target = frac * (double)__shfl(inc, 63);
        if (lane == 0) sm.tgt = target;
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
        int dd = per - 1;
        if (hit) {
          for (int i = 0; i < per; ++i) {
            const unsigned long long h = sm.hist[lane * per + i];
            if (h > 0 && (double)(c + h) >= target) { dd = i; break; }
            c += h;
          }
        } else {  // the last non-empty bucket of this lane
          for (int i = per - 1; i >= 0; --i)
            if (sm.hist[lane * per + i] > 0) { dd = i; break; }
          for (int i = 0; i < dd; ++i) c += sm.hist[lane * per + i];
        }
        sm.below = c;
        sm.prefix = pre | ((uint32_t)(lane * per + dd) << shift);
      }
    }
    __syncthreads();
    if (pass == 0 && frac > 0.0) target = sm.tgt;
  }
  if (key_only) {
    if (bad) sm.bad = 1;
    const Cut kc{sm.prefix, -1};
    __syncthreads();
    return kc;
  }
  // Tokens equal to the chosen key, in id order.  Usually a handful: they
  // are listed in LDS and ranked by id in wave 0.  Past kWList of them (near
  // flat rows), each thread scans a contiguous id range instead.
  const uint32_t key = sm.prefix;
  if (tid == 0) { sm.nlist = 0; sm.cut = Cut{key, -1}; }
  __syncthreads();
  auto tie = [&](uint32_t tk, int v, float t) {
    if (tk != key || !before_eq(key, v, lim)) return;
    const unsigned long long w = weight(r, t, mass);
    if (!w) return;
    const int i = atomicAdd(&sm.nlist, 1);
    if (i < kWList) { sm.list_id[i] = v; sm.list_w[i] = w; }
  };
  if (n2 >= 0) {
    for (int i = tid; i < n2; i += kWThreads) {
      const unsigned long long e = sm.lk[i];
      tie((uint32_t)(e >> 32), (int)(uint32_t)e, sm.lt[i]);
    }
  } else {
    for (int v0 = 0; v0 < r.V; v0 += kWBatch) {
      float zz[kWE];
      load_batch(r, v0, zz);
#pragma unroll
      for (int j = 0; j < kWE; ++j) {
        const int v = tok_of(r, v0, j);
        if (v >= r.V) continue;
        const float t = t_from(r, zz[j], &bad);
        tie(~tcode(t), v, t);
      }
    }
  }
  __syncthreads();
  const int nl = sm.nlist;
  if (nl <= kWList) {
    if (tid < 64) {  // wave 0: lane i ranks entry i by id (ids are distinct), then a prefix in id order
      const int myid = lane < nl ? sm.list_id[lane] : 0x7fffffff;
      const unsigned long long myw = lane < nl ? sm.list_w[lane] : 0ull;
      int rank = 0;
      for (int q = 0; q < nl; ++q) rank += __builtin_amdgcn_readlane(myid, q) < myid ? 1 : 0;
      if (lane < nl) { sm.sort_id[rank] = myid; sm.sort_w[rank] = myw; }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const unsigned long long w = lane < nl ? sm.sort_w[lane] : 0ull;
      unsigned long long inc = w;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      const unsigned long long below = sm.below;
      const bool hit = lane < nl && (double)(below + inc) >= target && (double)(below + inc - w) < target;
      const uint64_t ball = __ballot(hit);
      if (ball) {
        const int l = __ffsll((long long)ball) - 1;
        const unsigned long long cum = below + __shfl(inc, l);
        if (lane == 0) { sm.cum = cum; sm.cum_ok = 1; }
      }
      if (lane == 0)
        sm.cut = Cut{key, ball ? sm.sort_id[__ffsll((long long)ball) - 1] : (nl > 0 ? sm.sort_id[nl - 1] : -1)};
    }
    __syncthreads();
  } else {
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
    const unsigned long long exc = sm.below + wpre + inc - mine;
    if (mine > 0 && (double)exc < target && (double)(exc + mine) >= target) {
      unsigned long long c = exc;
      for (int v = v0; v < v1; ++v) {
        const float t = t_of(r, v, &bad);
        if (~tcode(t) != key || !before_eq(key, v, lim)) continue;
        c += weight(r, t, mass);
        if ((double)c >= target) { sm.cut = Cut{key, v}; sm.cum = c; sm.cum_ok = 1; break; }
      }
    }
    __syncthreads();
  }
  // rounding guard: the last token with this key.  The id is read into a
  // register and the barrier passed before tid 0 may rewrite it, so every wave
  // takes the same branch.
  const int cut_id = sm.cut.id;
  __syncthreads();
  if (cut_id < 0) {
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

// Every token of the row (before `lim`, t finite) whose key shares the first
// digit of `pre` goes to the LDS list sm.lk/sm.lt (sm.n2 counts them, also
// past kWL2).
template <bool VEC>
EDEV void list_bucket(const RowCtx& r, const Cut& lim, uint32_t pre, WarpSmem& sm, int* bad) {
  const int lane = threadIdx.x & 63;
  scan_row<VEC>(r, [&](const float (&zz)[kWE], int b) {
#pragma unroll
    for (int j = 0; j < kWE; ++j) {
      const int v = rowscan_tok<VEC>(b * kWBatch, j);
      const bool ok = v < r.V;
      const float t = ok ? t_from(r, zz[j], bad) : kNegInf;
      const uint32_t key = ~tcode(t);
      const bool take = ok && t != kNegInf && (key >> 20) == (pre >> 20) && before_eq(key, v, lim);
      const uint64_t mask = __ballot(take);
      if (mask == 0ull) continue;
      const int leader = __ffsll((long long)mask) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&sm.n2, __popcll(mask));
      base = __builtin_amdgcn_readlane(base, leader);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (take && pos < kWL2) {
        sm.lk[pos] = ((unsigned long long)key << 32) | (uint32_t)v;
        sm.lt[pos] = t;
      }
    }
  });
}

// The nucleus cut: the first token of the order (before `lim`) at which the
// running mass reaches frac of the total.  The first digit pass over the row
// gives the total, the target and the crossing 12-bit bucket; one more pass
// lists that bucket's tokens in LDS (a bucket is an eighth of an octave of t:
// a few thousand tokens at most on these rows), and the other two digits and
// the tied ids are settled from the list with the same arithmetic.  A bucket
// of more than kWL2 tokens goes on with the row passes.
EDEV Cut select_nucleus(const RowCtx& r, const Cut& lim, double frac, WarpSmem& sm) {
  const int tid = threadIdx.x;
  select_cut(r, lim, true, 0.0, sm, true, 1, frac);  // sets sm.prefix (first digit), sm.below, sm.tgt
  const uint32_t pre = sm.prefix;
  const double target = sm.tgt;
  if (tid == 0) sm.n2 = 0;
  __syncthreads();
  int bad = 0;
  if (r.vec)
    list_bucket<true>(r, lim, pre, sm, &bad);
  else
    list_bucket<false>(r, lim, pre, sm, &bad);
  if (bad) sm.bad = 1;
  __syncthreads();
  const int n2 = sm.n2;
  return select_cut(r, lim, true, target, sm, false, 3, 0.0, 1, n2 <= kWL2 ? n2 : -1);
}

// One pass for a top-k cut of at most kWFast tokens.  The first batch of the
// row (one load per thread, kept in registers) estimates a logit bound lz
// that about sqrt(k * kWFast) tokens of the row reach: each wave takes an
// order statistic of its lanes' maxima, scaled to the whole row, and the
// bound is the median of the 16 waves' values.  The row is then read once,
// two batches' loads in flight while one is filtered, and every token with
// z >= lz (or z NaN) is listed in LDS and ranked by (key, id).  The list
// holds the top k exactly when its k-th token has t > t(lz): t = z / T' does
// not decrease with z, so every token left out (z < lz) has t <= t(lz) and
// ranks after it.  With V <= kWFast every token is listed.  Returns k with
// fl.skey/sid/st holding the first k tokens of the order, or 0 when the bound
// missed (too few tokens reach it, or more than kWFast): the radix passes
// then decide.
template <bool VEC>
EDEV int onepass_topk(const RowCtx& r, int top_k, WarpSmem& sm, int* bad) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  FastList& fl = sm.fl;
  if (tid == 0) fl.n = 0;
  fl.key[tid] = 0u;  // rank counters of the list (kWFast == kWThreads)
  const int V = r.V;
  float lz = kNegInf;
  // the bound, from the first batch (its loads and the next two in flight)
  auto estimate = [&](const float (&za)[kWE]) {
    if (V > kWFast) {
      float m = kNegInf;
#pragma unroll
      for (int i = 0; i < kWE; ++i)
        if (rowscan_tok<VEC>(0, i) < V) m = fmaxf(m, za[i]);
      const uint32_t c = tcode(m);
      // a wave sees about min(V, batch) / 16 tokens of the first batch
      const float target = sqrtf((float)top_k * (float)kWFast);
      const float share = (float)min(V, kWBatch) / (16.0f * (float)V);
      const int jw = max(1, min(64, (int)(target * share + 0.5f)));
      uint32_t thr = 0;  // the jw-th largest lane code of this wave
#pragma unroll
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        if (__popcll(__ballot(c >= cand)) >= (unsigned)jw) thr = cand;
      }
      if (lane == 0) sm.est[wave] = thr;
      __syncthreads();
      if (tid < 64) {  // median of the 16 wave values: the 8th largest (ties by wave)
        const uint32_t e = lane < kWWaves ? sm.est[lane] : 0u;
        int rank = 0;
#pragma unroll
        for (int q = 0; q < kWWaves; ++q) {
          const uint32_t eq = __builtin_amdgcn_readlane(e, q);
          rank += (eq > e || (eq == e && q < lane)) ? 1 : 0;
        }
        if (lane < kWWaves && rank == kWWaves / 2 - 1) sm.lzc = e;
      }
      __syncthreads();
      const uint32_t lc = max(sm.lzc, tcode(kNegInf));
      lz = __uint_as_float((lc & 0x80000000u) ? (lc & 0x7fffffffu) : ~lc);
    } else {
      __syncthreads();  // fl.n = 0 is seen before the first listing
    }
  };
  uint64_t badm = 0;
  auto filter = [&](const float (&zz)[kWE], int b) {
    if (b == 0) estimate(zz);
    const int v0 = b * kWBatch;
    uint64_t anym = 0;
    if (v0 + kWBatch <= V) {
#pragma unroll
      for (int i = 0; i < kWE; ++i) {
        badm |= __ballot(!__builtin_isfinite(zz[i]));
        anym |= __ballot(!(zz[i] < lz));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kWE; ++i) {
        const bool ok = rowscan_tok<VEC>(v0, i) < V;
        badm |= __ballot(ok && !__builtin_isfinite(zz[i]));
        anym |= __ballot(ok && !(zz[i] < lz));
      }
    }
    if (anym == 0ull) return;
#pragma unroll
    for (int i = 0; i < kWE; ++i) {
      const int v = rowscan_tok<VEC>(v0, i);
      const bool take = v < V && !(zz[i] < lz);
      const uint64_t mask = __ballot(take);
      if (mask == 0ull) continue;
      const int leader = __ffsll((long long)mask) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&fl.n, __popcll(mask));
      base = __builtin_amdgcn_readlane(base, leader);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (take && pos < kWFast) {
        int b2 = 0;
        const float t = t_from(r, zz[i], &b2);
        sm.pk[pos] = ((unsigned long long)~tcode(t) << 32) | (uint32_t)v;
        fl.t[pos] = t;
      }
    }
  };
  scan_row<VEC>(r, filter);
  if (badm) *bad = 1;
  __syncthreads();
  const int nl = fl.n;
  if (nl < top_k || nl > kWFast) {
    __syncthreads();  // every thread has read fl.n before it is reused
    return 0;
  }
  // Rank by (key asc, id asc) = the packed value: entry e counts the entries
  // below it, its comparisons split over `parts` threads (as many as the
  // workgroup allows, at most 16) whose counts meet in fl.key[e].
  int parts = 1;
  while (parts < 16 && nl * parts * 2 <= kWThreads) parts *= 2;
  {
    const int e = tid / parts, p = tid - e * parts;
    if (e < nl) {
      const unsigned long long my = sm.pk[e];
      const int q0 = p * nl / parts, q1 = (p + 1) * nl / parts;
      int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
      int q = q0;
      for (; q + 4 <= q1; q += 4) {
        r0 += sm.pk[q] < my ? 1 : 0;
        r1 += sm.pk[q + 1] < my ? 1 : 0;
        r2 += sm.pk[q + 2] < my ? 1 : 0;
        r3 += sm.pk[q + 3] < my ? 1 : 0;
      }
      for (; q < q1; ++q) r0 += sm.pk[q] < my ? 1 : 0;
      const int cnt = (r0 + r1) + (r2 + r3);
      if (cnt) atomicAdd(&fl.key[e], (uint32_t)cnt);
    }
  }
  __syncthreads();
  if (tid < nl) {
    const int rank = (int)fl.key[tid];
    if (rank < top_k) {
      const unsigned long long my = sm.pk[tid];
      fl.skey[rank] = (uint32_t)(my >> 32);
      fl.sid[rank] = (int)(uint32_t)my;
      fl.st[rank] = fl.t[tid];
    }
  }
  __syncthreads();
  int b3 = 0;
  const bool ok = lz == kNegInf || fl.st[top_k - 1] > t_from(r, lz, &b3);
  __syncthreads();  // fl.n, pk and the sorted list are read before any reuse
  return ok ? top_k : 0;
}

// grid: one workgroup per warped row; workgroup i warps row map_row(i, rm)
// of z (and writes that row of stats and bound).
__global__ __launch_bounds__(kWThreads) void warp_kernel(int V, int top_k, float top_p, int min_keep, float Tp,
                                                         int mshift, const float* __restrict__ z,
                                                         float* __restrict__ stats, uint32_t* __restrict__ bound,
                                                         int32_t* status, RowMap rm) {
  __shared__ WarpSmem sm;
  const int row = map_row((int)blockIdx.x, rm), tid = threadIdx.x;
  RowCtx r;
  r.z = z + (size_t)row * V;
  r.vec = (V & 3) == 0 && ((uintptr_t)z & 15) == 0;
  r.V = V;
  r.Tp = Tp;
  r.mshift = mshift;
  r.e2 = sm.e2;
  if (tid < 256) sm.e2[tid] = exp2((double)tid * (1.0 / 256));  // published by the first barrier below
  if (tid == 0) sm.bad = 0;
  int bad = 0;
  const Cut all{0xffffffffu, 0x7fffffff};
  Cut cut = all;
  int nA = V;
  if (top_k > 0 && top_k < V && top_k <= kWFast) {
    FastList& fl = sm.fl;
    int n = r.vec ? onepass_topk<true>(r, top_k, sm, &bad) : onepass_topk<false>(r, top_k, sm, &bad);
    if (n == 0) {
    // The top-k cut's key needs no M (counts only).  One pass then lists
    // every token at or before that key (prefix) in LDS, where they are
    // ordered by (key, id): the list's first top_k tokens are the kept ones.
    // Usually the first digit suffices: the tokens whose first digit is at or
    // before the crossing one number below + hist[digit], often a few hundred.
    Cut kc = select_cut(r, all, false, (double)top_k, sm, true, 1);
    const unsigned long long coarse_n = sm.below + sm.hist[kc.key >> 20];
    // every wave has read sm.below and sm.hist before a second select resets them
    __syncthreads();
    uint32_t lim_key = kc.key | 0xFFFFFu;
    if (coarse_n > (unsigned long long)kWFast) {
      kc = select_cut(r, all, false, (double)top_k, sm, true, 3);
      lim_key = kc.key;
    }
    if (tid == 0) fl.n = 0;
    __syncthreads();
    for (int v0 = 0; v0 < V; v0 += kWBatch) {
      float zz[kWE];
      load_batch(r, v0, zz);
#pragma unroll
      for (int j = 0; j < kWE; ++j) {
        const int v = tok_of(r, v0, j);
        if (v >= V) continue;
        const float t = t_from(r, zz[j], &bad);
        const uint32_t key = ~tcode(t);
        if (key > lim_key) continue;
        const int i = atomicAdd(&fl.n, 1);
        if (i < kWFast) { fl.key[i] = key; fl.id[i] = v; fl.t[i] = t; }
      }
    }
    __syncthreads();
    const int nall = fl.n;
    if (nall <= kWFast) {  // else too many ties at the cut key: the passes below decide
      if (tid < nall) {  // rank by (key asc, id asc); keys and ids are read from LDS
        const uint32_t mk = fl.key[tid];
        const int mi = fl.id[tid];
        int rank = 0;
        for (int q = 0; q < nall; ++q) {
          const uint32_t kq = fl.key[q];
          rank += (kq < mk || (kq == mk && fl.id[q] < mi)) ? 1 : 0;
        }
        fl.skey[rank] = mk;
        fl.sid[rank] = mi;
        fl.st[rank] = fl.t[tid];
      }
      __syncthreads();
      n = min(top_k, nall);  // the cut keeps exactly top_k tokens
    }
    }
    if (n > 0) {
      if (tid == 0) fl.ci = 0x7fffffff;
      __syncthreads();
      cut = Cut{fl.skey[n - 1], fl.sid[n - 1]};
      nA = top_k;
      r.M = n > 0 ? fl.st[0] : kNegInf;  // the first of the order holds max t
      if (r.M != kNegInf && n <= 64) {
        // the kept list fits one wave: wave 0 takes the nucleus and the sum
        // alone, with the arithmetic of the workgroup version below (the
        // other waves only ever add zeros)
        if (bad) sm.bad = 1;
        __syncthreads();
        if (tid < 64) {
          int last = n - 1;
          if (top_p < 1.0f) {
            const unsigned long long w = tid < n ? weight(r, fl.st[tid], true) : 0ull;
            unsigned long long inc = w;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const unsigned long long y = __shfl_up(inc, o);
              if (tid >= o) inc += y;
            }
            const unsigned long long sa = __shfl(inc, 63);
            const double target = (double)top_p * (double)sa;
            const uint64_t hit = __ballot(tid < n && (double)inc >= target && (double)(inc - w) < target);
            int ci = hit ? __ffsll((long long)hit) - 1 : n - 1;
            if (min_keep > 1) ci = max(ci, min(min_keep, nA) - 1);
            last = ci;
            cut = Cut{fl.skey[ci], fl.sid[ci]};
          }
          const double sp = (tid <= last && fl.st[tid] != kNegInf) ? exp((double)fl.st[tid] - (double)r.M) : 0.0;
          const double sfin = wave_sum_d(sp);
          if (tid == 0) {
            stats[(size_t)row * 2] = r.M;
            stats[(size_t)row * 2 + 1] = (float)sfin;
            bound[(size_t)row * 2] = ~cut.key;
            bound[(size_t)row * 2 + 1] = (uint32_t)cut.id;
            if (sm.bad) set_status(status, EAGLE_STATUS_NONFINITE);
          }
        }
        return;
      }
      if (r.M != kNegInf) {
        int last = n - 1;  // index of the last kept token in the order
        if (top_p < 1.0f) {
          // fixed-point masses (as the row passes weigh them), inclusive prefix in order
          const unsigned long long w = tid < n ? weight(r, fl.st[tid], true) : 0ull;
          unsigned long long inc = w;
  #pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(inc, o);
            if ((tid & 63) >= o) inc += y;
          }
          if ((tid & 63) == 63) sm.part[tid >> 6] = inc;
          __syncthreads();
          unsigned long long wpre = 0, sa = 0;
          for (int q = 0; q < kWWaves; ++q) {
            if (q < (tid >> 6)) wpre += sm.part[q];
            sa += sm.part[q];
          }
          inc += wpre;
          // the first token at which the running mass reaches top_p of the top-k mass
          const double target = (double)top_p * (double)sa;
          if (tid < n && (double)inc >= target && (double)(inc - w) < target) atomicMin(&fl.ci, tid);
          __syncthreads();
          int ci = fl.ci == 0x7fffffff ? n - 1 : fl.ci;
          if (min_keep > 1) ci = max(ci, min(min_keep, nA) - 1);
          last = ci;
          cut = Cut{fl.skey[ci], fl.sid[ci]};
        }
        double sp = (tid <= last && fl.st[tid] != kNegInf) ? exp((double)fl.st[tid] - (double)r.M) : 0.0;
        const double sfin = block_sum_d(sp, sm);
        if (bad) sm.bad = 1;
        __syncthreads();
        if (tid == 0) {
          stats[(size_t)row * 2] = r.M;
          stats[(size_t)row * 2 + 1] = (float)sfin;
          bound[(size_t)row * 2] = ~cut.key;
          bound[(size_t)row * 2 + 1] = (uint32_t)cut.id;
          if (sm.bad) set_status(status, EAGLE_STATUS_NONFINITE);
        }
        return;
      }
      // an all -inf row: the passes below handle it as before
    }
  }
  // The top-k cut by counts, when the list above did not decide it (no M needed).
  if (top_k > 0 && top_k < V && nA == V) {
    cut = select_cut(r, all, false, (double)top_k, sm);
    nA = top_k;
  }
  // Before a nucleus, one listing pass gives M (the first token of the order)
  // and the min_keep cut (its kk-th token); else a max pass gives M.
  const int kk = max(1, min(min_keep, nA));
  bool listed = false;
  if (top_p < 1.0f && kk <= kWFast) {
    const int n1 = r.vec ? onepass_topk<true>(r, kk, sm, &bad) : onepass_topk<false>(r, kk, sm, &bad);
    listed = n1 > 0 && sm.fl.st[0] != kNegInf;
    if (listed) r.M = sm.fl.st[0];
    if (bad) sm.bad = 1;
  }
  if (!listed) {
    float lm = kNegInf;
    for (int v0 = 0; v0 < V; v0 += kWBatch) {
      float zz[kWE];
      load_batch(r, v0, zz);
#pragma unroll
      for (int j = 0; j < kWE; ++j)
        if (tok_of(r, v0, j) < V) lm = fmaxf(lm, t_from(r, zz[j], &bad));
    }
    if (bad) sm.bad = 1;
    r.M = block_max(lm, sm);
  }
  if (top_p < 1.0f) {
    // the target is top_p of the top-k mass, summed by the select's first pass
    Cut c = select_nucleus(r, cut, (double)top_p, sm);
    bool have_cum = sm.cum_ok != 0;
    const unsigned long long cum = sm.cum;
    __syncthreads();  // read before a later select resets them
    bool list_sum = false;
    if (min_keep > 1) {
      const Cut cm = listed ? Cut{sm.fl.skey[kk - 1], sm.fl.sid[kk - 1]}
                            : select_cut(r, cut, false, (double)min(min_keep, nA), sm);
      if (cm.key > c.key || (cm.key == c.key && cm.id > c.id)) {
        c = cm;
        have_cum = false;
        list_sum = listed;  // the kept set is the list's first kk tokens
      }
    }
    cut = c;
    // S without another pass: the select's fixed-point mass through the cut
    // (within V 2^-(mshift+1) of the fp64 sum, S >= 1), or the list's sum
    if (have_cum || list_sum) {
      double sfin;
      if (have_cum) {
        sfin = ldexp((double)cum, -r.mshift);
      } else {
        const double sp = (tid < kk && sm.fl.st[tid] != kNegInf) ? exp((double)sm.fl.st[tid] - (double)r.M) : 0.0;
        sfin = block_sum_d(sp, sm);
      }
      if (tid == 0) {
        stats[(size_t)row * 2] = r.M;
        stats[(size_t)row * 2 + 1] = (float)sfin;
        bound[(size_t)row * 2] = ~cut.key;
        bound[(size_t)row * 2 + 1] = (uint32_t)cut.id;
        if (sm.bad) set_status(status, EAGLE_STATUS_NONFINITE);
      }
      return;
    }
  }
  double s = 0.0;
  if (r.M != kNegInf)
    for (int v0 = 0; v0 < V; v0 += kWBatch) {
      float zz[kWE];
      load_batch(r, v0, zz);
#pragma unroll
      for (int j = 0; j < kWE; ++j) {
        const int v = tok_of(r, v0, j);
        if (v >= V) continue;
        const float t = t_from(r, zz[j], &bad);
        if (t != kNegInf && before_eq(~tcode(t), v, cut)) s += exp((double)t - (double)r.M);
      }
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

hipError_t launch_warp_map(int rows, int V, int top_k, float top_p, int min_keep, float T, const float* z,
                           float* stats, uint32_t* bound, int32_t* status, RowMap rm, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const float Tp = T > 0.f ? T : 1.0f;
  warp_kernel<<<rows, kWThreads, 0, st>>>(V, top_k, top_p, min_keep, Tp, warp_mass_shift(V), z, stats, bound, status,
                                          rm);
  return hipGetLastError();
}

hipError_t launch_warp(int rows, int V, int top_k, float top_p, int min_keep, float T, const float* z, float* stats,
                       uint32_t* bound, int32_t* status, hipStream_t st) {
  return launch_warp_map(rows, V, top_k, top_p, min_keep, T, z, stats, bound, status, RowMap{1 << 30, 0, 0}, st);
}

}  // namespace eagle
