// Acceptance walk: recursive speculative sampling down each request's tree.
//
// Method: EAGLE-1 notes ("EAGLE: Speculative Sampling Requires Rethinking
// Feature Uncertainty"), background A3 (accept x with probability
// min(1, p(x)/q(x)), else resample from norm(max(0, p - q))), section 3.3 and
// appendix A.2 (multi-round: after a rejection try the next of the node's k
// candidates against the adjusted distribution; sample it only when all k
// fail); hubwiz "LLM 推测性解码原理解读", section 1 (bonus token; between one
// and accepted + 1 committed tokens).  Greedy: follow the child equal to the
// target argmax (EAGLE-1 notes, A.1).
//
// The adjusted distributions are never materialised: after rejecting
// x_0..x_{j-1} (drawn without replacement from q) the unnormalised residual is
// max(0, p(y) - s_j q(y)) for untried y and a frozen value f_i for each tried
// x_i, with s_0 = 0, Z_0 = R_0 = 1,
//   s_{j+1} = s_j + Z_j / R_j,  R_{j+1} = R_j - q(x_j),
//   f_j = max(0, p(x_j) - s_{j+1} q(x_j)),  Z_{j+1} = sum of the residual
// (induction on P <- norm(max(0, P - Q)), Q <- Q without x_j, renormalised).
// Each rejection therefore costs one vocabulary reduction
// G(s) = sum_y max(0, p(y) - s q(y)); the acceptance ratio of trial j is
// max(0, p(x_j) - s_j q(x_j)) R_j / (Z_j q(x_j)) with p(x_j), q(x_j) in fp64.
//
// Parallel layout: a group of G workgroups per request, in one grid no
// larger than the device's resident capacity for this kernel (occupancy times
// compute units), so that in-stream order (the previous kernel has finished)
// leaves every workgroup resident at once.  A plain launch is used: a
// cooperative launch costs ~16 us more per call on this GPU.  If other work
// shares the GPU and keeps part of the grid from starting, the bounded waits
// time out and set EAGLE_STATUS_SYNC_TIMEOUT instead of hanging.  Every
// workgroup runs the same walk (same
// inputs, same code: identical decisions) and owns a contiguous vocabulary
// slice; a reduction is one pass over the slice plus an exchange of the G
// partial sums through per-request mailbox words.  A word carries its own
// validity tag, [1 | epoch 13 | step 10 | value 40], written and read with relaxed
// agent-scope atomics, so no memory fence (which would write back a whole L2)
// is needed.  Two banks alternate by step parity, so a workgroup can publish
// step t+1 while slower ones still read step t.  The partial's value is the
// top 40 bits of its fp64 (28-bit mantissa); every workgroup sums the G
// decoded values in index order, so all agree bit for bit.  Each workgroup
// (1024 threads) first copies the request's tree metadata (slots, pool tokens
// and flat indices, row statistics, uniforms) to LDS, so the walk's serial
// steps read LDS rather than global memory.  Spins are bounded:
// a timeout sets EAGLE_STATUS_SYNC_TIMEOUT and the walk continues.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr double kTie = 1e-6;
constexpr int kSpinMax = 1 << 18;  // polls per wait (a fraction of a second)
constexpr int kAccGroupCap = 32;   // largest group used (exchange cost grows with the group)

constexpr int kCacheMax = 8192;  // slice tokens whose exponential terms fit the LDS token cache (64 KB)

struct Rows {
  const float* zp;  // target logits row of the node (null with a compact row)
  const uint16_t* hp;  // compact target row of the node: fp16 offsets, and
  const float* bp;     // its 128-column block maxima (null: fp32 row zp)
  const float* zq;  // draft logits row of the node's slot (unused when s == 0)
  float Mp, Mq, Tp;
  double invSp, invSq;
  // sampling warps of the two rows (kept prefix: code and id of its last token)
  bool wp, wq;
  uint32_t pc, pi, qc, qi;
};

// Target logit of token v (a compact row decoded), and of tokens base..base+3
// (base a multiple of 4, all inside the row) with one vector load.
EDEV float zp_at(const Rows& R, int v) {
  return R.hp ? cmp_decode(R.hp[v], R.bp[v >> kCmpBlockShift]) : R.zp[v];
}
EDEV float4 zp_at4(const Rows& R, int base) {
  if (R.hp) {
    const uint2 u = *reinterpret_cast<const uint2*>(R.hp + base);
    const float m = R.bp[base >> kCmpBlockShift];  // four tokens from one block
    return make_float4(cmp_decode((uint16_t)(u.x & 0xFFFFu), m), cmp_decode((uint16_t)(u.x >> 16), m),
                       cmp_decode((uint16_t)(u.y & 0xFFFFu), m), cmp_decode((uint16_t)(u.y >> 16), m));
  }
  return *reinterpret_cast<const float4*>(R.zp + base);
}
// Alignment bits that forbid the vector loads of the target row.
EDEV uintptr_t p_misalign(const Rows& R) { return R.hp ? ((uintptr_t)R.hp & 7) : ((uintptr_t)R.zp & 15); }

// fp32 exponential term of token v's logit: exp(z/T' - M), 0 for a
// non-finite z or a token the row's warp drops.
EDEV float eterm(float z, int v, float M, float Tp, bool w, uint32_t wc, uint32_t wi) {
  if (!isfinite(z)) return 0.f;
  const float t = z / Tp;
  if (w && !warp_keeps(t, v, wc, wi)) return 0.f;
  return expf(t - M);
}
EDEV float eterm_p(float z, int v, const Rows& R) { return eterm(z, v, R.Mp, R.Tp, R.wp, R.pc, R.pi); }
EDEV float eterm_q(float z, int v, const Rows& R) { return eterm(z, v, R.Mq, R.Tp, R.wq, R.qc, R.qi); }

// Residual of one token at s from its two terms (s == 0: p alone), in fp64.
EDEV double resid_e(float ep, float eq, const Rows& R, double s) {
  const double p = (double)ep * R.invSp;
  if (s == 0.0) return p;
  const double d = p - s * ((double)eq * R.invSq);
  return d > 0.0 ? d : 0.0;
}

// fp64 probability of token v (acceptance ratios and R); 0 if the warp drops it.
EDEV double prob64(float z, int v, float M, double invS, float Tp, bool w, uint32_t wc, uint32_t wi) {
  if (!isfinite(z)) return 0.0;
  const float t = z / Tp;
  if (w && !warp_keeps(t, v, wc, wi)) return 0.0;
  return exp((double)t - (double)M) * invS;
}

// Tags always carry the top bit, so zero-filled words never match.
EDEV uint64_t tag_of(uint32_t epoch, int step) {
  return (1ull << 63) | ((uint64_t)(epoch & 0x1FFFu) << 50) | ((uint64_t)(step & 1023) << 40);
}
constexpr uint64_t kTagMask = ~((1ull << 40) - 1);
EDEV uint64_t encode_val(double v) { return (uint64_t)__double_as_longlong(v) >> 24; }
EDEV double decode_val(uint64_t w) { return __longlong_as_double((long long)((w & ((1ull << 40) - 1)) << 24)); }

struct Smem {
  double red[kWaves];
  double vals[kAccMaxGroup];   // decoded partials of the last reduction, by workgroup
  double scan[kWaves];
  double bc_d[4];
  int bc_i[4];
  // the current node's k children (sampling order): fp32 terms
  float cep[EAGLE_MAX_TOPK], ceq[EAGLE_MAX_TOPK];
  int tried_x[EAGLE_MAX_TOPK];  // tried token i is child i
  double tried_f[EAGLE_MAX_TOPK];
  int ov_x[EAGLE_MAX_TOPK];     // tried tokens in this workgroup's slice, and their frozen values
  double ov_f[EAGLE_MAX_TOPK];
  int nov;
};

EDEV void publish(uint64_t* w, uint64_t v) { __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
EDEV uint64_t peek(uint64_t* w) { return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Spin until *w carries `tag`; returns the word (bounded).
EDEV uint64_t await_tag(uint64_t* w, uint64_t tag, int* timed_out) {
  if (*timed_out) return tag;  // after one timeout the group no longer waits
  uint64_t v = peek(w);
  int it = 0;
  while ((v & kTagMask) != tag) {
    if (++it > kSpinMax) { *timed_out = 1; return tag; }
    __builtin_amdgcn_s_sleep(1);
    v = peek(w);
  }
  return v;
}

struct Group {
  int G, g, lo, hi;  // group size, own index, own vocabulary slice [lo, hi)
  int span;          // slice length (workgroup j owns [j*span, (j+1)*span))
  Mailbox* mb;
  uint32_t epoch;
  int step;
  float2* cache;     // LDS terms (ep, eq) of the slice's tokens for the current node, or null
  int cstate;        // 0 empty, 1 ep filled, 2 ep and eq filled
};

// The two exponential terms of the 4 tokens base..base+3 of this thread's
// slice position ci: from the LDS cache when it holds the current node, else
// from the logits (and kept in the cache).  Tokens past the slice give 0.
EDEV void slice_terms(const Rows& R, bool need_q, bool from_cache, const Group& gr, int base, int ci, bool vec,
                      float ep[4], float eq[4]) {
  if (from_cache) {
    const float4 c0 = *reinterpret_cast<const float4*>(&gr.cache[ci]);
    const float4 c1 = *reinterpret_cast<const float4*>(&gr.cache[ci + 2]);
    ep[0] = c0.x; eq[0] = c0.y; ep[1] = c0.z; eq[1] = c0.w;
    ep[2] = c1.x; eq[2] = c1.y; ep[3] = c1.z; eq[3] = c1.w;
    return;
  }
  float zp[4], zq[4];
  if (vec && base + 3 < gr.hi) {
    const float4 p4 = zp_at4(R, base);
    zp[0] = p4.x; zp[1] = p4.y; zp[2] = p4.z; zp[3] = p4.w;
    if (need_q) {
      const float4 q4 = *reinterpret_cast<const float4*>(R.zq + base);
      zq[0] = q4.x; zq[1] = q4.y; zq[2] = q4.z; zq[3] = q4.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zp[e] = base + e < gr.hi ? zp_at(R, base + e) : kNegInf;
      if (need_q) zq[e] = base + e < gr.hi ? R.zq[base + e] : kNegInf;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ep[e] = base + e < gr.hi ? eterm_p(zp[e], base + e, R) : 0.f;
    eq[e] = (need_q && base + e < gr.hi) ? eterm_q(zq[e], base + e, R) : 0.f;
  }
  if (gr.cache) {
    *reinterpret_cast<float4*>(&gr.cache[ci]) = make_float4(ep[0], eq[0], ep[1], eq[1]);
    *reinterpret_cast<float4*>(&gr.cache[ci + 2]) = make_float4(ep[2], eq[2], ep[3], eq[3]);
  }
}

EDEV bool cache_ready(const Group& gr, bool need_q) {
  return gr.cache && (gr.cstate == 2 || (gr.cstate == 1 && !need_q));
}

// All threads: this workgroup's part of G(s) over its slice (tried tokens not
// corrected), one partial per wave left in sm.red (no barrier).
EDEV void local_partial(const Rows& R, double s, Group& gr, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool need_q = s != 0.0;
  const bool from_cache = cache_ready(gr, need_q);
  const bool vec = (p_misalign(R) | (need_q ? ((uintptr_t)R.zq & 15) : 0)) == 0;
  double a = 0.0;
  for (int base = gr.lo + tid * 4, ci = tid * 4; base < gr.hi; base += kThreads * 4, ci += kThreads * 4) {
    float ep[4], eq[4];
    slice_terms(R, need_q, from_cache, gr, base, ci, vec, ep, eq);
    a += (resid_e(ep[0], eq[0], R, s) + resid_e(ep[1], eq[1], R, s)) +
         (resid_e(ep[2], eq[2], R, s) + resid_e(ep[3], eq[3], R, s));
  }
  if (gr.cache && !from_cache) gr.cstate = need_q ? 2 : 1;
  a = wave_sum_d(a);
  if (lane == 0) sm.red[wave] = a;
}

// Wave 0 only, after the wave partials are in sm.red: publishes this
// workgroup's partial, collects the G partials (kept in sm.vals) and sums
// them with a butterfly, so every lane of every workgroup of the group holds
// the same total bit for bit.  The caller advances gr.step in all threads.
EDEV double wave0_exchange(Group& gr, Smem& sm, int* timed_out) {
  const int lane = threadIdx.x & 63;
  const double part = wave_sum_d(lane < kWaves ? sm.red[lane] : 0.0);
  const uint64_t tag = tag_of(gr.epoch, gr.step);
  uint64_t* bank = gr.mb->bank[gr.step & 1];
  if (lane == 0) publish(bank + gr.g, tag | encode_val(part));
  double v = 0.0;
  if (lane < gr.G) {
    v = decode_val(await_tag(bank + lane, tag, timed_out));
    sm.vals[lane] = v;
  }
  return wave_sum_d(v);
}

// All threads of every workgroup of the group: Z = G(s) over the vocabulary
// (tried tokens not corrected); per-workgroup partials left in sm.vals.
EDEV double group_reduce(const Rows& R, double s, Group& gr, Smem& sm, int* timed_out) {
  local_partial(R, s, gr, sm);
  lds_barrier();
  if (threadIdx.x < 64) {
    const double v = wave0_exchange(gr, sm, timed_out);
    if (threadIdx.x == 0) sm.bc_d[0] = v;
  }
  __syncthreads();
  ++gr.step;
  return sm.bc_d[0];
}

// Fill the LDS token cache with the terms of rows R over the slice (q terms
// too when need_q).
EDEV void fill_cache(const Rows& R, bool need_q, Group& gr) {
  const int tid = threadIdx.x;
  const bool vec = (p_misalign(R) | (need_q ? ((uintptr_t)R.zq & 15) : 0)) == 0;
  for (int base = gr.lo + tid * 4, ci = tid * 4; base < gr.hi; base += kThreads * 4, ci += kThreads * 4) {
    float ep[4], eq[4];
    slice_terms(R, need_q, false, gr, base, ci, vec, ep, eq);
  }
  gr.cstate = need_q ? 2 : 1;
}

// Inclusive fp64 prefix sum over the wave in lane order: DPP row shifts by
// 1, 2, 4, 8 inside each row of 16 lanes (lanes shifted in from outside the
// row read 0), then the totals of the preceding rows added in order.
EDEV double wave_scan_d(double v) {
  v += dpp_d<0x111>(v);
  v += dpp_d<0x112>(v);
  v += dpp_d<0x114>(v);
  v += dpp_d<0x118>(v);
  const double r0 = lane_d(v, 15), r1 = lane_d(v, 31), r2 = lane_d(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const double pre = row == 0 ? 0.0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  return v + pre;
}

// Inverse-CDF draw from the residual at s (partials from the last exchange at
// the same s, in sm.vals), tried tokens replaced by their frozen values.
// Wave 0 corrects the partials, finds the owning workgroup and the mass left
// before it; that workgroup locates the token in its slice and posts it to
// the mailbox.  Returns the token in workgroup 0 (others: -1).
EDEV int group_draw(const Rows& R, double s, int ntried, double uval, Group& gr, Smem& sm, int V, int* ties,
                    int* timed_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    // lane i < ntried: tried token i's owner and the change from its current
    // term to its frozen value; those in this workgroup's slice are listed
    int own = -1, inslice = 0, x = 0;
    double dlt = 0.0;
    if (lane < ntried) {
      x = sm.tried_x[lane];
      own = min(x / gr.span, gr.G - 1);
      dlt = sm.tried_f[lane] - resid_e(sm.cep[lane], sm.ceq[lane], R, s);
      inslice = x >= gr.lo && x < gr.hi;
    }
    const uint64_t ball = __ballot(inslice);
    if (inslice) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0u));
      sm.ov_x[pos] = x;
      sm.ov_f[pos] = sm.tried_f[lane];
    }
    // corrected partial of workgroup `lane` (corrections in tried order), clamped at 0
    double c = lane < gr.G ? sm.vals[lane] : 0.0;
    for (int i = 0; i < ntried; ++i) {
      const int oi = __builtin_amdgcn_readlane(own, i);
      const double di = lane_d(dlt, i);
      if (lane == oi) c += di;
    }
    c = c > 0.0 ? c : 0.0;
    // total, then the first workgroup whose cumulative mass passes u * total
    double tot = 0.0;
    for (int j = 0; j < gr.G; ++j) tot += lane_d(c, j);
    const double target = uval * tot;
    double cum = 0.0;
    int gstar = -1;
    for (int j = 0; j < gr.G; ++j) {
      const double cj = lane_d(c, j);
      if (cj > 0.0 && cum + cj > target) { gstar = j; break; }
      cum += cj;
    }
    if (gstar < 0) {  // rounding: the last workgroup with mass
      for (int j = gr.G - 1; j >= 0; --j)
        if (lane_d(c, j) > 0.0) { gstar = j; break; }
      cum = 0.0;
      for (int j = 0; j < gstar; ++j) cum += lane_d(c, j);
    }
    if (lane == 0) {
      sm.bc_i[0] = gstar < 0 ? 0 : gstar;
      sm.bc_d[1] = target - cum;
      sm.bc_d[2] = tot;
      sm.nov = __popcll(ball);
    }
  }
  __syncthreads();
  const int gstar = sm.bc_i[0];
  const double off0 = sm.bc_d[1], tot = sm.bc_d[2];
  const int nov = sm.nov;
  const uint64_t rtag = tag_of(gr.epoch, gr.step);
  int token = -1;
  if (gr.g == gstar) {
    // scan the own slice in id order, 4096 tokens (4 per thread) per pass
    const bool need_q = s != 0.0;
    const bool from_cache = cache_ready(gr, need_q);
    const bool vec = (p_misalign(R) | (need_q ? ((uintptr_t)R.zq & 15) : 0)) == 0;
    double off = off0;
    int found = -1, tie = 0, last_pos = -1;
    for (int base0 = gr.lo, ci0 = 0; base0 < gr.hi && found < 0; base0 += kThreads * 4, ci0 += kThreads * 4) {
      const int base = base0 + tid * 4, ci = ci0 + tid * 4;
      double val[4], mine = 0.0;
      float ep[4] = {0.f, 0.f, 0.f, 0.f}, eq[4] = {0.f, 0.f, 0.f, 0.f};
      if (base < gr.hi) slice_terms(R, need_q, from_cache, gr, base, ci, vec, ep, eq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = base + e;
        double xv = 0.0;
        if (v < gr.hi) {
          xv = resid_e(ep[e], eq[e], R, s);
          if (nov > 0)
            for (int i = 0; i < nov; ++i)
              if (sm.ov_x[i] == v) xv = sm.ov_f[i];
        }
        val[e] = xv;
        mine += xv;
      }
      double inc = wave_scan_d(mine);
      if (lane == 63) sm.scan[wave] = inc;
      if (tid == 0) { sm.bc_i[1] = -1; sm.bc_i[2] = 0; sm.bc_i[3] = -1; }
      lds_barrier();
      double pre = 0.0, ptot = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const double t = sm.scan[w];
        pre += w < wave ? t : 0.0;
        ptot += t;
      }
      inc += pre;
      const double exc = inc - mine;
      if (mine > 0.0 && exc <= off && off < inc) {
        double c = exc;
        int pick = -1, t2 = 0;
        for (int e = 0; e < 4; ++e) {
          if (val[e] > 0.0 && c + val[e] > off) {
            pick = e;
            if ((off - c) < kTie * tot || (c + val[e] - off) < kTie * tot) t2 = 1;
            break;
          }
          c += val[e];
        }
        if (pick < 0)
          for (int e = 3; e >= 0; --e)
            if (val[e] > 0.0) { pick = e; break; }
        atomicMax(&sm.bc_i[1], base + pick);
        if (t2) atomicOr(&sm.bc_i[2], 1);
      }
      // remember the last positive token of the slice (rounding fallback):
      // the highest lane holding one has the wave's largest, one atomic per wave
      int lp = -1;
      for (int e = 3; e >= 0; --e)
        if (val[e] > 0.0) { lp = base + e; break; }
      const uint64_t pb = __ballot(lp >= 0);
      if (pb != 0ull) {
        const int top = 63 - __clzll((long long)pb);
        const int wlp = __builtin_amdgcn_readlane(lp, top);
        if (lane == 0) atomicMax(&sm.bc_i[3], wlp);
      }
      lds_barrier();
      found = sm.bc_i[1];
      tie |= sm.bc_i[2];
      if (sm.bc_i[3] >= 0) last_pos = sm.bc_i[3];
      off -= ptot;
      lds_barrier();
    }
    if (found < 0) found = last_pos >= 0 ? last_pos : gr.lo;
    token = found;
    if (tid == 0) {
      if (tie) atomicAdd(ties, 1);
      if (gr.g != 0) publish(&gr.mb->result, rtag | (uint64_t)(uint32_t)token);
    }
  }
  if (gr.g == 0 && gstar != 0) {
    if (tid == 0) {
      const uint64_t w = await_tag(&gr.mb->result, rtag, timed_out);
      sm.bc_i[0] = (int)(uint32_t)(w & 0xFFFFFFFFu);
    }
    __syncthreads();
    token = sm.bc_i[0];
  }
  ++gr.step;
  return gr.g == 0 ? token : -1;
}

__global__ __launch_bounds__(kThreads) void accept_kernel(
    int b0, int nb, int G, int N, int V, int D, int k, int S, float T, int cache_tokens,
    const int32_t* __restrict__ node_tok,
    const int32_t* __restrict__ node_parent, const int32_t* __restrict__ node_slot, const int32_t* __restrict__ pool_tok,
    const int32_t* __restrict__ pool_flat, const float* __restrict__ tlog, const float* __restrict__ tstats,
    const int32_t* __restrict__ targmax, const float* __restrict__ dlog, const float* __restrict__ sstats,
    const uint32_t* __restrict__ tbound, const uint32_t* __restrict__ dbound,
    const uint16_t* __restrict__ thp, const float* __restrict__ tbm,
    const float* __restrict__ uniforms, Mailbox* __restrict__ mail, int32_t* accept_len, int32_t* accept_path,
    int32_t* committed, int32_t* n_committed, int32_t* near_tie, int32_t* status) {
  // dynamic LDS: [cache_tokens] token cache, then the request's tree metadata
  extern __shared__ __attribute__((aligned(16))) float2 tcache[];
  __shared__ Smem sm;
  __shared__ int ties, timed_out;
  __shared__ int path[EAGLE_MAX_DEPTH + 1];
  __shared__ int comm[EAGLE_MAX_DEPTH + 2];
  __shared__ int npath, ncomm;
  __shared__ int cur_u, cur_j, acc_j, zero_resid, follow, stale;
  __shared__ double st_s;

  // Workgroups go round-robin over the XCDs, so a request's group is taken
  // from the blocks of one residue mod 8: its exchanges then stay among the
  // compute units of one XCD (~1.4 instead of ~2 us per exchange).  Placement
  // only affects speed: the exchange protocol is correct on any placement.
  const int xr = (int)blockIdx.x & 7, xj = (int)blockIdx.x >> 3;
  const int r = xr + 8 * (xj / G), g = xj % G, tid = threadIdx.x;
  if (r >= nb) return;  // padding block of the last XCD column
  const int b = b0 + r;
  const bool greedy = !(T > 0.f);
  const float Tp = greedy ? 1.f : T;
  const int32_t* ntok = node_tok + (size_t)b * N;
  const int32_t* npar = node_parent + (size_t)b * N;
  if (tid == 0) { ties = 0; timed_out = 0; npath = 0; ncomm = 0; cur_u = 0; zero_resid = 0; }
  __syncthreads();

  if (greedy) {
    if (g == 0 && tid == 0) {
      int u = 0;
      for (int step = 0; step <= D; ++step) {
        const int y = targmax[(size_t)b * N + u];
        comm[ncomm++] = y;
        int nxt = -1;
        for (int c = u + 1; c < N; ++c)
          if (npar[c] == u && ntok[c] == y) { nxt = c; break; }
        if (nxt < 0 || npath >= D) break;
        path[npath++] = nxt;
        u = nxt;
      }
    }
  } else {
    Group gr;
    gr.G = G;
    gr.g = g;
    const int span = ((V + G - 1) / G + 3) / 4 * 4;
    gr.lo = min(V, g * span);
    gr.hi = min(V, gr.lo + span);
    gr.span = span;
    gr.mb = mail - 1 - b;  // `mail` is the end of the mailbox area: request b's is b + 1 back
    gr.epoch = __hip_atomic_load(&gr.mb->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    gr.step = 0;
    gr.cache = cache_tokens >= span ? tcache : nullptr;
    gr.cstate = 0;
    // The request's tree metadata, copied to LDS once (after the token cache):
    // node slots, pool tokens and flat indices, row statistics, uniforms.
    const int nmeta = N + 2 * S * k + 2 * N + 2 * S + N * (k + 1);
    int* m_slot = reinterpret_cast<int*>(tcache + cache_tokens);
    int* m_ptok = m_slot + N;
    int* m_pflat = m_ptok + S * k;
    float* m_tst = reinterpret_cast<float*>(m_pflat + S * k);
    float* m_sst = m_tst + 2 * N;
    float* m_U = m_sst + 2 * S;
    // four entries per thread in flight at a time (one address each, by range)
    auto meta_src = [&](int i) -> const int32_t* {
      if (i < N) return node_slot + (size_t)b * N + i;
      if (i < N + S * k) return pool_tok + (size_t)b * S * k + (i - N);
      if (i < N + 2 * S * k) return pool_flat + (size_t)b * S * k + (i - N - S * k);
      if (i < 3 * N + 2 * S * k) return reinterpret_cast<const int32_t*>(tstats) + (size_t)b * N * 2 + (i - N - 2 * S * k);
      if (i < 3 * N + 2 * S * k + 2 * S)
        return reinterpret_cast<const int32_t*>(sstats) + (size_t)b * S * 2 + (i - 3 * N - 2 * S * k);
      return reinterpret_cast<const int32_t*>(uniforms) + (size_t)b * N * (k + 1) + (i - 3 * N - 2 * S * k - 2 * S);
    };
    for (int i0 = tid; i0 < nmeta; i0 += 4 * kThreads) {
      int v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r * kThreads;
        v[r] = i < nmeta ? *meta_src(i) : 0;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i0 + r * kThreads < nmeta) m_slot[i0 + r * kThreads] = v[r];
    }
    int cnode = -1;  // node whose terms the token cache holds
    if (tid == 0) {  // retire this workgroup's stale words from earlier calls
      const uint64_t reset = tag_of(gr.epoch, 1023);
      publish(&gr.mb->bank[0][g], reset);
      publish(&gr.mb->bank[1][g], reset);
    }
    __syncthreads();

    // Walk state.  Wave 0 holds the current node's k candidates in its lanes
    // (lane i: candidate i) and runs every serial decision; the other waves
    // take part in the vocabulary passes only.  Loop control goes through LDS.
    const int lane = tid & 63;
    double c_p = 0.0, c_q = 0.0, c_f = 0.0;  // candidate's fp64 p and q, frozen residual
    float c_ep = 0.f, c_eq = 0.f;             // its fp32 terms
    double w_s = 0.0, w_Z = 1.0, w_R = 1.0;   // s_j, Z_j, R_j (wave 0, uniform)
    for (int step = 0; step <= D; ++step) {
      const int u = lds_index(cur_u, N, status);
      const int slot = m_slot[u];
      Rows R;
      if (thp) {  // compact target rows
        R.zp = nullptr;
        R.hp = thp + ((size_t)b * N + u) * V;
        R.bp = tbm + ((size_t)b * N + u) * (((size_t)V + 127) >> kCmpBlockShift);
      } else {
        R.zp = tlog + ((size_t)b * N + u) * V;
        R.hp = nullptr;
        R.bp = nullptr;
      }
      R.wp = tbound != nullptr;
      R.pc = R.wp ? tbound[((size_t)b * N + u) * 2] : 0u;
      R.pi = R.wp ? tbound[((size_t)b * N + u) * 2 + 1] : 0u;
      R.wq = false;
      R.qc = R.qi = 0u;
      R.Tp = Tp;
      R.Mp = m_tst[2 * u];
      R.invSp = 1.0 / (double)m_tst[2 * u + 1];
      R.zq = nullptr;
      R.Mq = 0.f;
      R.invSq = 0.0;
      const float* Uu = m_U + u * (k + 1);
      // The slot's candidates: its pool row up to the first -1 (a static
      // tree's slot may have fewer than k draws; a dynamic tree's has k).
      int kk = k;
      if (slot >= 0 && slot < S) {
        uint32_t none = 0;
#pragma unroll
        for (int j = 0; j < EAGLE_MAX_TOPK; ++j)
          if (j < k && m_ptok[slot * k + j] < 0) none |= 1u << j;
        kk = none ? __builtin_ctz(none) : k;
      }
      if (slot < 0 || slot >= S || kk == 0) {
        // never expanded: bonus token from the target
        gr.cstate = 0;
        group_reduce(R, 0.0, gr, sm, &timed_out);
        const int y = group_draw(R, 0.0, 0, (double)Uu[k], gr, sm, V, &ties, &timed_out);
        if (g == 0 && tid == 0) comm[ncomm++] = y;
        break;
      }
      R.zq = dlog + ((size_t)b * S + slot) * V;
      R.wq = dbound != nullptr;
      R.qc = R.wq ? dbound[((size_t)b * S + slot) * 2] : 0u;
      R.qi = R.wq ? dbound[((size_t)b * S + slot) * 2 + 1] : 0u;
      R.Mq = m_sst[2 * slot];
      R.invSq = 1.0 / (double)m_sst[2 * slot + 1];
      // The node's k children (wave 0, lane i: child i): their loads go out
      // first, then the token cache is filled with the node's rows while
      // they are in flight.  An id out of range is flagged and scored as
      // token 0.
      int c_ok = 0, c_x = 0;
      float zpx = 0.f, zqx = 0.f;
      if (tid < k) {
        const int x = m_ptok[slot * k + tid];
        c_ok = x >= 0 && x < V;
        c_x = c_ok ? x : 0;
        zpx = zp_at(R, c_x);
        zqx = R.zq[c_x];
      }
      // The node's rows for the token cache: the loads go out now, behind the
      // children's, and the terms are stored only when a reduction needs them
      // (a node whose first candidate is accepted never waits for them).
      const bool fill = gr.cache != nullptr && cnode != u;
      const bool vecr = (V & 3) == 0 && (p_misalign(R) | ((uintptr_t)R.zq & 15)) == 0;
      float4 rp[2], rq[2];
      if (fill) {
        gr.cstate = 0;
        if (vecr) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int base = gr.lo + tid * 4 + t * kThreads * 4;
            if (base < gr.hi) {
              rp[t] = zp_at4(R, base);
              rq[t] = *reinterpret_cast<const float4*>(R.zq + base);
            }
          }
        } else {
          fill_cache(R, true, gr);
          cnode = u;
        }
      }
      auto store_rows = [&]() {
        if (!(fill && vecr)) return;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int v = gr.lo + tid * 4 + t * kThreads * 4;
          if (v < gr.hi) {
            const int ci = lds_index(tid * 4 + t * kThreads * 4 + 3, cache_tokens, status) - 3;
            *reinterpret_cast<float4*>(&gr.cache[ci]) =
                make_float4(eterm_p(rp[t].x, v, R), eterm_q(rq[t].x, v, R), eterm_p(rp[t].y, v + 1, R),
                            eterm_q(rq[t].y, v + 1, R));
            *reinterpret_cast<float4*>(&gr.cache[ci + 2]) =
                make_float4(eterm_p(rp[t].z, v + 2, R), eterm_q(rq[t].z, v + 2, R), eterm_p(rp[t].w, v + 3, R),
                            eterm_q(rq[t].w, v + 3, R));
          }
        }
        gr.cstate = 2;
        cnode = u;
      };
      if (tid < k) {
        c_p = prob64(zpx, c_x, R.Mp, R.invSp, Tp, R.wp, R.pc, R.pi);
        c_q = prob64(zqx, c_x, R.Mq, R.invSq, Tp, R.wq, R.qc, R.qi);
        c_ep = eterm_p(zpx, c_x, R);
        c_eq = eterm_q(zqx, c_x, R);
        c_f = 0.0;
        sm.tried_x[tid] = c_x;
        sm.cep[tid] = c_ep;
        sm.ceq[tid] = c_eq;
      }
      // Trial j of the node, by wave 0 with (w_s, w_Z, w_R) = (s_j, Z_j, R_j):
      // accepted, or rejected with s_{j+1}, R_{j+1} computed.
      auto trial = [&](int j, double* s_next) -> bool {
        const double px = lane_d(c_p, j), qx = lane_d(c_q, j);
        bool acc = false;
        if (!__builtin_amdgcn_readlane(c_ok, j)) {
          if (lane == 0) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
        } else {
          const double num = w_s == 0.0 ? px : fmax(0.0, px - w_s * qx);
          double ratio;
          if (qx > 0.0 && w_R > 0.0) ratio = num * w_R / (w_Z * qx);
          else ratio = num > 0.0 ? __builtin_huge_val() : 0.0;
          const double a = ratio < 1.0 ? ratio : 1.0;
          const double uu = (double)Uu[j];
          if (lane == 0 && fabs(uu - a) < kTie) ++ties;
          acc = uu < a;
        }
        if (!acc) {
          *s_next = w_s + w_Z / w_R;
          w_R = w_R - qx;
        }
        return acc;
      };
      if (tid < 64) {
        w_s = 0.0; w_Z = 1.0; w_R = 1.0;
        double sn = 0.0;
        const bool a0 = trial(0, &sn);
        if (lane == 0) { acc_j = a0 ? 0 : -1; st_s = sn; cur_j = 0; stale = 0; }
      }
      lds_barrier();
      if (acc_j < 0) store_rows();
      // Rejections: one vocabulary reduction each.  After rejecting trial j
      // at s_{j+1}: Z_{j+1} = G(s_{j+1}) corrected for the tokens tried before
      // j, f_j frozen, then trial j + 1 is decided in the same wave-0 pass.
      while (acc_j < 0 && cur_j < kk - 1) {
        const int j = cur_j;
        const double snew = st_s;
        local_partial(R, snew, gr, sm);
        lds_barrier();
        if (tid < 64) {
          const double Gs = wave0_exchange(gr, sm, &timed_out);
          const double corr = wave_sum_d(lane < j ? c_f - resid_e(c_ep, c_eq, R, snew) : 0.0);
          const double Z = Gs + corr;
          if (Z > 0.0) {
            if (lane == j) c_f = resid_e(c_ep, c_eq, R, snew);
            w_s = snew;
            w_Z = Z;
          } else {  // zero residual mass: keep P
            if (lane == j) c_f = resid_e(c_ep, c_eq, R, w_s);
            if (lane == 0) zero_resid = 1;
          }
          if (lane == j) sm.tried_f[j] = c_f;
          double sn = 0.0;
          const bool a = trial(j + 1, &sn);
          if (lane == 0) { acc_j = a ? j + 1 : -1; st_s = sn; cur_j = j + 1; stale = Z > 0.0 ? 0 : 1; }
        }
        lds_barrier();
        ++gr.step;
      }
      if (acc_j >= 0) {
        if (tid == 0) {
          const int x = m_ptok[slot * k + acc_j];
          comm[ncomm++] = x;
          const int f = m_pflat[slot * k + acc_j];
          if (f > 0 && f < N && npath < D) {
            path[npath++] = f;
            cur_u = f;
            follow = 1;
          } else {
            follow = 0;
          }
        }
        lds_barrier();
        if (!follow) break;
        continue;
      }
      // all kk rejected: the last rejection (trial kk - 1) still needs its
      // reduction, then the draw from the residual at s_kk (redone at the
      // kept s when that reduction found no residual mass)
      {
        const int j = kk - 1;
        const double snew = st_s;
        local_partial(R, snew, gr, sm);
        lds_barrier();
        if (tid < 64) {
          const double Gs = wave0_exchange(gr, sm, &timed_out);
          const double corr = wave_sum_d(lane < j ? c_f - resid_e(c_ep, c_eq, R, snew) : 0.0);
          const double Z = Gs + corr;
          if (Z > 0.0) {
            if (lane == j) c_f = resid_e(c_ep, c_eq, R, snew);
            w_s = snew;
          } else {
            if (lane == j) c_f = resid_e(c_ep, c_eq, R, w_s);
            if (lane == 0) zero_resid = 1;
          }
          if (lane == j) sm.tried_f[j] = c_f;
          if (lane == 0) { st_s = w_s; stale = Z > 0.0 ? 0 : 1; }
        }
        lds_barrier();
        ++gr.step;
      }
      const double s_fin = st_s;
      if (stale) group_reduce(R, s_fin, gr, sm, &timed_out);
      const int y = group_draw(R, s_fin, kk, (double)Uu[k], gr, sm, V, &ties, &timed_out);
      if (g == 0 && tid == 0) comm[ncomm++] = y;
      break;
    }
    __syncthreads();
    if (g == 0 && tid == 0) __hip_atomic_store(&gr.mb->epoch, gr.epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid == 0 && timed_out) set_status(status, EAGLE_STATUS_SYNC_TIMEOUT);
  if (g != 0) return;
  if (tid == 0 && zero_resid) set_status(status, EAGLE_STATUS_ZERO_RESIDUAL);
  if (tid <= D) {
    if (tid < D) accept_path[(size_t)b * D + tid] = tid < npath ? path[tid] : -1;
    committed[(size_t)b * (D + 1) + tid] = tid < ncomm ? comm[tid] : -1;
  }
  if (tid == 0) {
    accept_len[b] = npath;
    n_committed[b] = ncomm;
    near_tie[b] = ties;
  }
}

// Largest dynamic LDS of one workgroup: a full token cache plus the metadata
// of the largest tree (N = 256 nodes, pool 4096, at most 256 slots, k = 16).
size_t accept_lds_max() {
  return (size_t)kCacheMax * sizeof(float2) +
         (size_t)(3 * EAGLE_MAX_NODES + 2 * EAGLE_MAX_POOL + 2 * EAGLE_MAX_NODES +
                  EAGLE_MAX_NODES * (EAGLE_MAX_TOPK + 1)) * 4;
}

}  // namespace

hipError_t launch_accept(int B, int N, int V, int D, int k, int S, float T, const int32_t* node_tok,
                         const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                         const int32_t* pool_flat, const float* tlog, const float* tstats, const int32_t* targmax,
                         const float* dlog, const float* sstats, const uint32_t* tbound, const uint32_t* dbound,
                         const uint16_t* thp, const float* tbm, const float* uniforms, void* mail,
                         int32_t* accept_len, int32_t* accept_path, int32_t* committed, int32_t* n_committed,
                         int32_t* near_tie, int32_t* status, hipStream_t st) {
  const bool greedy = !(T > 0.f);
  // Group size: as many workgroups per request as stay co-resident; requests
  // beyond the resident capacity go in further launches.
  // The capacity is a property of the device and this kernel: computed once
  // per device and cached in an atomic (concurrent first calls compute the
  // same value; either store wins).
  static std::atomic<int> capacity[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) dev = 0;
  int cap = capacity[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_kernel, kThreads, accept_lds_max());
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cap = per_cu * cus > 0 ? per_cu * cus : 1;
    capacity[dev].store(cap, std::memory_order_relaxed);
  }
  // A launch covers 8 x ceil(nb / 8) x G blocks (request r on residue r mod 8),
  // at most the resident capacity; requests beyond it go in further launches.
  const int cap_x = cap / 8 > 0 ? cap / 8 : 1;  // resident blocks per residue class
  const int cols = (B + 7) / 8;
  int G = 1;
  if (!greedy)
    while (G * 2 <= kAccGroupCap && (size_t)cols * G * 2 <= (size_t)cap_x && G * 2 * 1024 <= V) G *= 2;
  const int per_launch = 8 * (cap_x / G > 0 ? cap_x / G : 1);
  // token cache: the slice's exponential terms stay in LDS across the passes at a node
  const int span = ((V + G - 1) / G + 3) / 4 * 4;
  int cache_tokens = (!greedy && span <= kCacheMax) ? span : 0;
  const size_t meta = greedy ? 0 : (size_t)(3 * N + 2 * S * k + 2 * S + N * (k + 1)) * 4;
  const size_t lds = (size_t)cache_tokens * sizeof(float2) + meta;
  Mailbox* mb = static_cast<Mailbox*>(mail);
  for (int b0 = 0; b0 < B; b0 += per_launch) {
    const int nb = B - b0 < per_launch ? B - b0 : per_launch;
    accept_kernel<<<dim3(8 * ((nb + 7) / 8) * G), dim3(kThreads), lds, st>>>(b0, nb, G, N, V, D, k, S, T, cache_tokens,
        node_tok, node_parent,
        node_slot, pool_tok, pool_flat, tlog, tstats, targmax, dlog, sstats, tbound, dbound, thp, tbm, uniforms, mb,
        accept_len,
        accept_path,
        committed, n_committed, near_tie, status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace eagle
