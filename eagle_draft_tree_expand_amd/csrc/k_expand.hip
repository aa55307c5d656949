// Draft-tree expansion: per-slot softmax statistics and child selection over
// the vocabulary, then tree assembly (values, frontier, rerank, flatten).
//
// Method: EAGLE-2 notes ("EAGLE-2: Faster Inference of Language Models with
// Dynamic Draft Trees"), sections "Expanding the Draft Tree" (value equation:
// product of draft confidences along the root path; expand the k best of the
// current layer), "Rerank draft tokens" (top-m by value, shallower first on
// ties, connected result) and "Tree Attention Mask" (flatten); EAGLE-1 notes
// ("EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"),
// appendix A.1 (greedy: top-k children; non-greedy: k sampled children).
//
// Kernels:
//   expand_scan   grid (ceil(V/4096), B*S), 256 threads.  One pass over 4096
//                 logits of one slot row: per-wave (max, sum exp) of t = z/T'
//                 and the wave's k+2 best candidates by an fp32 key (greedy:
//                 z; sampling: t + Gumbel noise from Philox).  Bound by its
//                 VALU work (Philox, two logarithms and an exponential per
//                 logit when sampling), not by the row reads.
//   expand_merge  grid B*S, 256 threads.  Merges the wave records of a row:
//                 M, S (fp64 sum), exact fp64 keys of the candidates, the k
//                 best in sampling order, their confidences q.  Proves that
//                 the candidate set holds the exact top-k (else re-scans the
//                 row: rare).
//   tree_assemble grid B, 1024 threads, all state in LDS.  Values, frontier
//                 ranks per layer, rerank of the pool by merging per-layer
//                 sorted lists, BFS flattening.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace eagle {

namespace {

constexpr int kPer = 16;  // logits per thread in the scan

// The slots a launch covers: slots s0 .. s0 + n - 1 of every request.
struct SlotRange {
  int s0, n;
};

// Record of one wave's slice: [m, s, key[KP], idx[KP]] as floats (idx bit-cast).
struct UnitView {
  float* p;
  int KP;
  EDEV float& m() { return p[0]; }
  EDEV float& s() { return p[1]; }
  EDEV float& key(int r) { return p[2 + r]; }
  EDEV int idx(int r) const { return __float_as_int(p[2 + KP + r]); }
  EDEV void set_idx(int r, int v) { p[2 + KP + r] = __int_as_float(v); }
};

// MODE: kGreedy (key z), kSampleT1 (key z + g, T = 1), kSampleT (key z/T + g).
constexpr int kGreedy = 0, kSampleT1 = 1, kSampleT = 2;

template <int MODE>
__global__ __launch_bounds__(kExpThreads) void expand_scan_kernel(
    const float* __restrict__ rows, int S, int V, float Tp, uint32_t k0, uint32_t k1,
    uint32_t round_lo, int KP, const uint32_t* __restrict__ bound, float* __restrict__ units, int32_t* status,
    SlotRange sr) {
  // grid row y: slot sr.s0 + y % sr.n of request y / sr.n (all slots: s0 = 0, n = S)
  const int b = (int)blockIdx.y / sr.n, s = sr.s0 + ((int)blockIdx.y - b * sr.n);
  const int row = b * S + s;
  const int chunk = blockIdx.x;
  // sampling warp of this row (null: none): tokens it drops leave the
  // statistics and the keys alike (t = -inf)
  const bool warped = MODE != kGreedy && bound != nullptr;
  const uint32_t wcode = warped ? bound[(size_t)row * 2] : 0u, wid = warped ? bound[(size_t)row * 2 + 1] : 0u;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = rows + (size_t)row * V;

  float key[kPer], t[kPer];
  bool bad = false;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int base = chunk * kExpChunk + it * (kExpThreads * 4) + tid * 4;
    float zz[4];
    if ((V & 3) == 0 && base + 3 < V) {
      const float4 v4 = *reinterpret_cast<const float4*>(z + base);
      zz[0] = v4.x; zz[1] = v4.y; zz[2] = v4.z; zz[3] = v4.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[e] = (base + e < V) ? z[base + e] : kNegInf;
    }
    bool kept = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = it * 4 + e;
      const bool valid = base + e < V;
      float x = zz[e];
      if (valid && !isfinite(x)) { bad = true; x = kNegInf; }
      if (!valid) x = kNegInf;
      t[j] = MODE == kSampleT ? x / Tp : x;
      if (warped && !warp_keeps(t[j], base + e, wcode, wid)) t[j] = kNegInf;
      kept |= t[j] != kNegInf;
      if (MODE == kGreedy) key[j] = x;
    }
    if (MODE != kGreedy) {
      // A warp drops most of a row: a wave none of whose lanes keeps a token
      // of these four skips their noise (every key is -inf either way).
      if (!warped || __any(kept)) {
        const uint4 w4 = philox4x32_10(make_uint4((uint32_t)base >> 2, (uint32_t)s, (uint32_t)b, round_lo), k0, k1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wd = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
          key[it * 4 + e] = t[it * 4 + e] + gumbel_fast(wd);  // -inf stays -inf
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[it * 4 + e] = kNegInf;
      }
    }
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);

  // (max, sum exp) of this wave's slice.
  float lm = kNegInf;
#pragma unroll
  for (int j = 0; j < kPer; ++j) lm = fmaxf(lm, t[j]);
  const float wm = wave_max(lm);
  float ls = 0.f;
  if (wm != kNegInf) {
    constexpr float kLog2e = 1.44269504088896341f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ls += __builtin_amdgcn_exp2f((t[j] - wm) * kLog2e);  // exp2(-inf) = 0
  }
  const float wsum = wave_sum(ls);

  // The wave's KP best (key desc, idx asc).  Keys become order-preserving
  // unsigned codes (0 = past the end of the vocabulary).  The KP-th largest
  // of the 64 lane maxima, found bit by bit with ballots, bounds the wave's
  // KP-th best key from below, so only elements at or above it can be in the
  // top KP; they are compacted into LDS (usually ~KP of them) and each finds
  // its rank by counting.  If more than 64 qualify (heavy ties, or a sparse
  // tail) the wave falls back to KP rounds of wave argmax.
  UnitView u{units + ((size_t)row * gridDim.x * kExpUnitsPerChunk + (size_t)chunk * kExpUnitsPerChunk + wave) * (2 + 2 * KP), KP};
  auto idx_of = [&](int j) { return chunk * kExpChunk + (j >> 2) * (kExpThreads * 4) + tid * 4 + (j & 3); };
  // A warped row keeps few tokens (top-k 50 of 128256: most waves hold none),
  // so its -inf keys would tie at the bound and send the wave to the slow
  // path below.  There the search and the candidates take the finite keys
  // only; a wave with fewer than KP of them lists them, then its -inf tokens
  // in index order (key desc, idx asc: every -inf key ranks after every
  // finite one).  Unwarped rows rank -inf keys like any other.
  uint32_t uk[kPer];
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t bits = __float_as_uint(key[j] + 0.0f);  // -0 -> +0: they tie like equal keys
    const uint32_t code = bits ^ ((uint32_t)((int32_t)bits >> 31) | 0x80000000u);
    uk[j] = idx_of(j) < V && (!warped || key[j] != kNegInf) ? code : 0u;
    lmax = max(lmax, uk[j]);
  }
  int nfin = KP;  // finite keys of the wave (counted for warped rows only)
  if (warped) {
    nfin = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) nfin += __popcll(__ballot(uk[j] != 0u));
  }
  // The bound is searched on the top 16 bits of the lane maxima (a 16-bit
  // bucket holding the KP-th largest; a lower bound all the same, at a cost of
  // a few more candidates), and the candidates take their LDS positions from a
  // per-wave counter, so a group of 64 elements with none at or above the
  // bound costs one compare.
  uint32_t thr = 0;
  if (nfin >= KP) {
    const uint32_t lm16 = lmax >> 16;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = thr | (1u << bit);
      if (__popcll(__ballot(lm16 >= c)) >= (unsigned)KP) thr = c;
    }
    thr <<= 16;
  }
  thr = max(thr, 1u);
  __shared__ uint64_t cand[4][64];
  __shared__ int ccount[4];
  if (lane == 0) ccount[wave] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (uk[j] >= thr) {
      const int pos = atomicAdd(&ccount[wave], 1);
      if (pos < 64) cand[wave][pos] = ((uint64_t)uk[j] << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx_of(j));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int total = ccount[wave];
  if (total <= 64) {
    const uint64_t mine = lane < total ? cand[wave][lane] : 0ull;
    int r = 0;
    for (int c = 0; c < total; ++c) r += cand[wave][c] > mine ? 1 : 0;
    if (lane < total && r < KP) {
      const uint32_t code = (uint32_t)(mine >> 32);
      const uint32_t bits = (code & 0x80000000u) ? (code & 0x7fffffffu) : ~code;
      u.key(r) = __uint_as_float(bits);
      u.set_idx(r, (int)(0xffffffffu - (uint32_t)mine));
    }
    int listed = total;
    if (nfin < KP) {
      // entries nfin .. KP-1: the wave's -inf tokens with the smallest ids.
      // Ids ascend with (group j / 4, lane, j % 4); per group, a lane's
      // count of such tokens is prefix-summed over the lanes from its bits.
      const int need = KP - nfin;
      int before = 0;  // such tokens in earlier groups
      for (int g = 0; g < 4 && before < need; ++g) {
        uint32_t mk = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = g * 4 + e;
          if (idx_of(j) < V && key[j] == kNegInf) mk |= 1u << e;
        }
        const int c = __popc(mk);
        const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
        auto below = [&](uint64_t m) {
          return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        };
        int r2 = before + below(b0) + 2 * below(b1) + 4 * below(b2);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((mk >> e) & 1u) {
            if (r2 < need) { u.key(nfin + r2) = kNegInf; u.set_idx(nfin + r2, idx_of(g * 4 + e)); }
            ++r2;
          }
        before += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
      }
      listed = nfin + min(before, need);
    }
    if (lane >= listed && lane < KP) { u.key(lane) = kNegInf; u.set_idx(lane, kIdxNone); }
  } else {
    float bk = kNegInf;
    int bi = kIdxNone;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int id = idx_of(j);
      if (id < V && beats(key[j], id, bk, bi)) { bk = key[j]; bi = id; }
    }
    uint32_t taken = 0;
    for (int r = 0; r < KP; ++r) {
      float wk = bk;
      int wi = bi;
      wave_argmax(wk, wi);
      if (lane == 0) { u.key(r) = wk; u.set_idx(r, wi); }
      if (wi != kIdxNone && bi == wi) {  // owner lane: drop the winner, find its next best
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (idx_of(j) == wi) taken |= 1u << j;
        bk = kNegInf;
        bi = kIdxNone;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int id = idx_of(j);
          if (id < V && !((taken >> j) & 1u) && beats(key[j], id, bk, bi)) { bk = key[j]; bi = id; }
        }
      }
    }
  }
  if (lane == 0) { u.m() = wm; u.s() = wsum; }
}

// Block-wide helpers for 256 threads (4 waves).
__device__ float block_max_256(float v, float* sh) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  return v;
}

__device__ double block_sum_256(double v, double* sh) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__device__ int block_or_256(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = __any(v) ? 1 : 0;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return sh[0] | sh[1] | sh[2] | sh[3];
}

// Block argmax over per-thread (key, idx) under (key desc, idx asc).
__device__ void block_argmax_256(double& key, int& idx, double* shk, int* shi) {
  wave_argmax_d(key, idx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) { shk[wave] = key; shi[wave] = idx; }
  __syncthreads();
  key = shk[0];
  idx = shi[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (beats_d(shk[w], shi[w], key, idx)) { key = shk[w]; idx = shi[w]; }
}

template <bool GREEDY>
__device__ double exact_key(const float* z, int idx, int s, int b, float Tp, uint32_t k0, uint32_t k1,
                            uint32_t round_lo, bool warped, uint32_t wcode, uint32_t wid) {
  const float zz = z[idx];
  if (!isfinite(zz)) return -__builtin_huge_val();
  if (GREEDY) return (double)zz;
  const float t = zz / Tp;
  if (warped && !warp_keeps(t, idx, wcode, wid)) return -__builtin_huge_val();
  return (double)t + gumbel_f64(token_uniform(idx, s, b, round_lo, k0, k1));
}

// Bound on |fp32 candidate key - fp64 key| (fp32 rounding of t + g, and of g).
EDEV double key_slack(double key) { return 8e-7 * (fabs(key) + 24.0); }

// The k best of nc (key, idx) candidates in LDS under (key desc, idx asc)
// into sel_key/sel_idx (kIdxNone past the end).  Up to one candidate per
// thread: each counts the candidates that beat it, which is its rank; more
// (rare): k rounds of block argmax.  The caller syncs afterwards.
__device__ void block_topk(double* xkey, int* xidx, int nc, int k, double* sel_key, int* sel_idx,
                           double* shd, int* shi) {
  const int tid = threadIdx.x;
  if (nc <= kExpThreads) {
    if (tid < k && tid >= nc) { sel_key[tid] = -__builtin_huge_val(); sel_idx[tid] = kIdxNone; }
    if (tid < nc) {
      const double v = xkey[tid];
      const int vi = xidx[tid];
      int r = 0;
      for (int c = 0; c < nc; ++c) r += beats_d(xkey[c], xidx[c], v, vi) ? 1 : 0;
      if (r < k) { sel_key[r] = v; sel_idx[r] = vi; }
    }
    return;
  }
  double bk = -__builtin_huge_val();
  int bi = kIdxNone, bc = -1;
  for (int c = tid; c < nc; c += kExpThreads)
    if (beats_d(xkey[c], xidx[c], bk, bi)) { bk = xkey[c]; bi = xidx[c]; bc = c; }
  for (int r = 0; r < k; ++r) {
    double wk = bk;
    int wi = bi;
    block_argmax_256(wk, wi, shd, shi);
    if (tid == 0) { sel_key[r] = wk; sel_idx[r] = wi; }
    if (wi != kIdxNone && bi == wi) {  // owner: hide the winner, find its next best
      xkey[bc] = -__builtin_huge_val();
      xidx[bc] = kIdxNone;
      bk = -__builtin_huge_val();
      bi = kIdxNone;
      bc = -1;
      for (int c = tid; c < nc; c += kExpThreads)
        if (beats_d(xkey[c], xidx[c], bk, bi)) { bk = xkey[c]; bi = xidx[c]; bc = c; }
    }
  }
}

template <bool GREEDY>
__global__ __launch_bounds__(kExpThreads) void expand_merge_kernel(
    const float* __restrict__ rows, int S, int V, float Tp, uint32_t k0, uint32_t k1,
    uint32_t round_lo, int k, int KP, int C, const uint32_t* __restrict__ bound, const float* __restrict__ units,
    int32_t* __restrict__ pool_tok, float* __restrict__ pool_q, float* __restrict__ slot_stats,
    int32_t* status, SlotRange sr) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int b = (int)blockIdx.x / sr.n, s = sr.s0 + ((int)blockIdx.x - b * sr.n);
  const int row = b * S + s;
  const bool warped = !GREEDY && bound != nullptr;
  const uint32_t wcode = warped ? bound[(size_t)row * 2] : 0u, wid = warped ? bound[(size_t)row * 2 + 1] : 0u;
  const int tid = threadIdx.x;
  const int U = C * kExpUnitsPerChunk;
  const int UF = 2 + 2 * KP;
  const float* z = rows + (size_t)row * V;
  const float* ubg = units + (size_t)row * U * UF;
  double* xkey = reinterpret_cast<double*>(smem_raw);          // [kExpRescanCap]
  int* xidx = reinterpret_cast<int*>(xkey + kExpRescanCap);     // [kExpRescanCap]
  float* heads = reinterpret_cast<float*>(xidx + kExpRescanCap);  // [U] best key of each record
  float* ub = heads + U;                                           // [U * UF] the row's records

  __shared__ double shd[4];
  __shared__ float shf[4];
  __shared__ int shi[4];
  __shared__ double sel_key[EAGLE_MAX_TOPK];
  __shared__ int sel_idx[EAGLE_MAX_TOPK];
  __shared__ int n_cand;
  __shared__ float head_k;

  // The row's records go to LDS in one coalesced copy; every later pass
  // reads them there.
  if (tid == 0) { n_cand = 0; head_k = kNegInf; }
  {
    // UF is even, so the records are float2-aligned; eight loads per thread
    // go out before their stores
    const int n2 = U * UF / 2;
    const float2* src = reinterpret_cast<const float2*>(ubg);
    float2* dst = reinterpret_cast<float2*>(ub);
    for (int base = 0; base < n2; base += 8 * kExpThreads) {
      float2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * kExpThreads + tid;
        if (i < n2) v[j] = src[i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * kExpThreads + tid;
        if (i < n2) dst[i] = v[j];
      }
    }
  }
  __syncthreads();

  // Row statistics and record heads.
  float lm = kNegInf;
  for (int x = tid; x < U; x += kExpThreads) {
    lm = fmaxf(lm, ub[(size_t)x * UF]);
    heads[x] = __float_as_int(ub[(size_t)x * UF + 2 + KP]) == kIdxNone ? kNegInf : ub[(size_t)x * UF + 2];
  }
  const float M = block_max_256(lm, shf);  // its barriers also publish heads[]
  double ls = 0.0;
  if (M != kNegInf)
    for (int x = tid; x < U; x += kExpThreads) {
      const float um = ub[(size_t)x * UF], us = ub[(size_t)x * UF + 1];
      if (us > 0.f) ls += (double)us * exp((double)um - (double)M);
    }

  // The k-th best record head bounds the k-th best fp32 key from below (k
  // records each hold a key at least that large).  Fewer than k records: no
  // bound.  Each head's rank (count of better heads) is counted by a group
  // of 2^lt lanes, so every lane has a short loop of independent LDS reads.
  {
    const int lt = U * 16 <= kExpThreads ? 4 : U * 8 <= kExpThreads ? 3 : U * 4 <= kExpThreads ? 2
                 : U * 2 <= kExpThreads ? 1 : 0;
    const int tpe = 1 << lt;
    for (int base = 0; base < U * tpe; base += kExpThreads) {
      const int q = base + tid, x = q >> lt, part = q & (tpe - 1);
      if (x < U) {
        const float h = heads[x];
        int r = 0;
#pragma unroll 16
        for (int y = part; y < U; y += tpe) {
          const float w = heads[y];
          r += (w > h || (w == h && y < x)) ? 1 : 0;
        }
        if (lt >= 1) r += dpp_i<kDppXor1>(r);
        if (lt >= 2) r += dpp_i<kDppXor2>(r);
        if (lt >= 3) r += dpp_i<kDppHalfMirror>(r);
        if (lt >= 4) r += dpp_i<kDppMirror>(r);
        if (part == 0 && r == k - 1) head_k = h;
      }
    }
  }
  const double Sd = block_sum_256(ls, shd);  // its barriers also publish head_k

  // Candidates: every record entry whose fp32 key can still reach the k-th
  // place.  Greedy keys are the logits themselves (exact); sampling keys are
  // within key_slack of the fp64 key, so the bound drops by twice the slack.
  const float Hk = head_k;
  const double thr = GREEDY ? (double)Hk : (double)Hk - 2.0 * key_slack(Hk);
  // A record's keys are sorted (key desc, idx asc), so its candidates are a
  // prefix: one thread per record walks it until a key falls below the bound.
  for (int x = tid; x < U; x += kExpThreads) {
    for (int r = 0; r < KP; ++r) {
      const float ka = ub[(size_t)x * UF + 2 + r];
      if ((double)ka < thr) break;
      const int id = __float_as_int(ub[(size_t)x * UF + 2 + KP + r]);
      if (id != kIdxNone && id >= 0 && id < V) {
        const int slot = atomicAdd(&n_cand, 1);
        if (slot < kExpRescanCap) {
          xidx[slot] = id;
          xkey[slot] = (double)ka;
        }
      }
    }
  }
  __syncthreads();
  if (!GREEDY) {
    const int nc = min(n_cand, kExpRescanCap);
    for (int c = tid; c < nc; c += kExpThreads)
      xkey[c] = exact_key<false>(z, xidx[c], s, b, Tp, k0, k1, round_lo, warped, wcode, wid);
    __syncthreads();
  }

  for (int pass = 0; pass < 2; ++pass) {
    const int nc = min(n_cand, kExpRescanCap);
    if (n_cand > kExpRescanCap && tid == 0) set_status(status, EAGLE_STATUS_CAND_OVERFLOW);
    block_topk(xkey, xidx, nc, k, sel_key, sel_idx, shd, shi);
    __syncthreads();
    // Greedy: every token is in exactly one record and each record holds its
    // slice's KP >= k best in exact order, so the union holds the top k.
    if (GREEDY || pass == 1) break;
    // Sampling: proof that no logit outside the records can reach the k-th
    // exact key: every full record must end strictly below it (minus slack).
    const double Ek = sel_key[k - 1];
    const double delta = key_slack(Ek);
    int need = 0;
    for (int x = tid; x < U; x += kExpThreads) {
      const int last = __float_as_int(ub[(size_t)x * UF + 2 + KP + (KP - 1)]);
      if (last != kIdxNone && (double)ub[(size_t)x * UF + 2 + (KP - 1)] + delta >= Ek) need = 1;
    }
    if (!block_or_256(need, shi)) break;
    // Rare: re-scan the row, keeping every logit whose fp32 key can reach Ek.
    if (tid == 0) { n_cand = 0; set_status(status, EAGLE_STATUS_TOPK_RESCAN); }
    __syncthreads();
    const double thr2 = Ek - delta;
    for (int v = tid; v < V; v += kExpThreads) {
      const float zz = z[v];
      if (!isfinite(zz)) continue;
      const float t = zz / Tp;
      if (warped && !warp_keeps(t, v, wcode, wid)) continue;
      const float ka = t + gumbel_f32(token_uniform(v, s, b, round_lo, k0, k1));
      if ((double)ka >= thr2) {
        const int slot = atomicAdd(&n_cand, 1);
        if (slot < kExpRescanCap) {
          xidx[slot] = v;
          xkey[slot] = exact_key<false>(z, v, s, b, Tp, k0, k1, round_lo, warped, wcode, wid);
        }
      }
    }
    __syncthreads();
  }

  if (tid < k) {
    const int id = sel_idx[tid];
    const size_t o = (size_t)row * k + tid;
    if (id == kIdxNone) {
      pool_tok[o] = 0;
      pool_q[o] = 0.f;
    } else {
      pool_tok[o] = id;
      const double t = (double)(z[id] / Tp);
      pool_q[o] = (float)(exp(t - (double)M) / Sd);
    }
  }
  if (tid == 0) {
    slot_stats[(size_t)row * 2] = M;
    slot_stats[(size_t)row * 2 + 1] = (float)Sd;
  }
}

// ---- tree assembly ------------------------------------------------------
// Pool index e = s*k + j (child j of slot s).  Layer 1 = [0, k); layer d >= 2
// = [k + (d-2)k^2, k + (d-1)k^2).  Pool-index order equals (depth, cidx) order,
// so every tie-break "(depth asc, cidx asc)" is "pool index asc".


EDEV int layer_lo(int d, int k) { return d == 1 ? 0 : k + (d - 2) * k * k; }
EDEV int layer_n(int d, int k) { return d == 1 ? k : k * k; }
EDEV int depth_of(int e, int k) { return e < k ? 1 : 2 + (e - k) / (k * k); }

// Order key of a pool node: value bits (values are >= 0, so their bit
// patterns order like the values) over the complement of the pool index, so
// that "larger key" is exactly (value desc, pool index asc).  All keys are
// distinct; 0 is below every real key.
EDEV uint64_t node_key(float v, int e) {
  return ((uint64_t)__float_as_uint(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}
EDEV float key_value(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }
EDEV int key_node(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }

constexpr int kTreeThreads = 1024;  // one workgroup per request: every layer step has the CU to itself

// One workgroup per request; everything in LDS.
//  1. layers, one block step each: every node of the layer counts the keys
//     of its layer above its own, which is its layer rank; the k best become
//     the next frontier (slots) and give their children the values
//     parent value * q;
//  2. rerank: the m largest keys of the pool.  Only the first min(m, n) of
//     each layer's sorted keys can make it; each of them adds, for every
//     other layer, the count of larger keys there (binary search) to its
//     layer rank;
//  3. flatten: BFS order (depth, parent flat index, sibling rank) is the order
//     of (depth, path of sibling ranks from the root) read as a number, so a
//     selected node's flat index is 1 + the count of selected nodes before it.
__global__ __launch_bounds__(kTreeThreads) void tree_assemble_kernel(
    int S, int k, int D, int m, int V, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ pool_tok_g, const float* __restrict__ pool_q_g,
    int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
    int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_flat_g,
    int32_t* slot_src_g, int32_t* status, int upto, const int32_t* __restrict__ prefix_len,
    uint64_t* __restrict__ mask_out, int32_t* __restrict__ pos_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int P = S * k, N = m + 1;
  const int LS = (k * k + 1) & ~1;                                 // layer stride (keys), even
  // [D][LS] keys in pool order, 0 padded; then 2 zero keys and 32 write sinks
  uint64_t* lay = reinterpret_cast<uint64_t*>(smem_raw);
  uint64_t* skeys = lay + D * LS + 2 + 32;                         // [D][LS] keys sorted desc
  uint64_t* spath = skeys + D * LS;                                // [S + 1] path of the node at each slot; sink
  uint64_t* sel_key = spath + S + 1;                               // [m] (depth, path) of each selected node
  uint64_t* sel_key2 = sel_key + m;                                // [m] path alone (deep trees)
  float* q = reinterpret_cast<float*>(sel_key2 + m);               // [P]
  int* lrank = reinterpret_cast<int*>(q + P);                      // [P] rank inside the layer
  int* flat_of = lrank + P;                                        // [P] flat index or -1
  int* slot_src = flat_of + P;                                     // [S + 1] frontier node of each slot; sink
  int* sel_e = slot_src + S + 1;                                   // [m] pool index of each selected node
  int* sel_dep = sel_e + m;                                        // [m]
  int* ptok = sel_dep + m;                                         // [P] pool tokens, read with q up front
  int* fpar = ptok + P;                                            // [N] flat parent (the mask, when asked for)
  int* fdep = fpar + N;                                            // [N] depth
  __shared__ int n_sel;

  const float* pq = pool_q_g + (size_t)b * P;
  for (int e = tid; e < P; e += nt) {
    const float qe = pq[e];
    ptok[e] = pool_tok_g[(size_t)b * P + e];
    q[e] = qe;
    flat_of[e] = -1;
  }
  for (int x = tid; x < D * LS + 2; x += nt) lay[x] = x < k ? node_key(pq[x], x) : 0ull;  // layer 1: value = 1 * q
  for (int x = tid; x < S; x += nt) slot_src[x] = -1;
  for (int x = tid; x < N; x += nt) { fpar[x] = -1; fdep[x] = 0; }
  if (tid == 0) n_sel = 0;
  __syncthreads();

  // 1. Layers (1..upto; upto < D: only the frontiers up to depth upto are
  // wanted, while the tree is still being drafted depth by depth).  A lane
  // group of 2^lt lanes ranks two nodes of the layer: each key pair it reads
  // is compared with both, and every read of the step (the key pairs and the
  // paths of the two nodes' parents) is issued before the first wait, so a
  // step costs one barrier and two LDS round trips (the keys, then the q of
  // the new frontier's children).  The step is latency-bound: one wave's
  // instruction stream per step is what the loop keeps short.
  // x / k == (x * kdiv) >> 16 for every x < 65536 / k (here x < 4096)
  const uint32_t kdiv = __builtin_amdgcn_readfirstlane(65536u / (uint32_t)k + 1u);
  auto div_k = [&](int x) __attribute__((always_inline)) {
    uint32_t r;
    asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"((uint32_t)x), "s"(kdiv));
    return (int)(r >> 16);
  };
  const uint32_t ku = __builtin_amdgcn_readfirstlane((uint32_t)k);
  auto mul_k = [&](int x) __attribute__((always_inline)) {  // x * k for 0 <= x < 2^24
    uint32_t r;
    asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"((uint32_t)x), "s"(ku));
    return (int)r;
  };
  const ulonglong2* Z2 = reinterpret_cast<const ulonglong2*>(lay + D * LS);  // a pair of zero keys
  uint64_t* sink = lay + D * LS + 2;                                          // 32 keys nobody reads
  // One layer step.  FAST (k <= 11): every layer has at most 61 node pairs,
  // so every step takes 16-lane groups and one chunk of four key pairs, and
  // the writes go without branches (lanes with nothing to write store to
  // the sinks).
  auto step = [&](auto fast_tag, int d) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const int lo = layer_lo(d, k), n = layer_n(d, k), np = (n + 1) >> 1, dl = d - 1;
    const ulonglong2* L2 = reinterpret_cast<const ulonglong2*>(lay + dl * LS);  // pairs; LS is even
    const int lt = FAST ? 4 : np * 16 <= nt ? 4 : np * 8 <= nt ? 3 : np * 4 <= nt ? 2 : np * 2 <= nt ? 1 : 0;
    const int tpe = 1 << lt, p1 = tpe > 1 ? 1 : 0;
    const int g = tid >> lt, part = tid & (tpe - 1);
    if (g >= np) return;
    const int x0 = 2 * g, x1 = x0 + 1;
    const bool has1 = x1 < n;
    // parents' slots and the nodes' sibling ranks (layer 1: the root, slot 0)
    const int q0 = div_k(x0), q1 = div_k(x1);
    const int ps0 = d == 1 ? 0 : 1 + (d - 2) * k + q0, ps1 = d == 1 ? 0 : 1 + (d - 2) * k + q1;
    const uint64_t pp0 = spath[lds_index(ps0, S + 1, status)], pp1 = spath[lds_index(has1 ? ps1 : ps0, S + 1, status)];
    const ulonglong2 own = L2[g];  // nodes x0, x1 (a key of 0 past the layer's end)
    const uint64_t K0 = own.x, K1 = own.y;
    int r0 = 0, r1 = 0;
    const int T = FAST ? 1 : (np + tpe - 1) >> lt;  // chunks of four key pairs per lane (FAST: np <= 64)
    for (int i0 = 0; i0 < (FAST ? 4 : T); i0 += 4) {
      ulonglong2 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int y2 = part + (i0 + u) * tpe;
        w[u] = *(y2 < np ? L2 + y2 : Z2);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        r0 += (w[u].x > K0 ? 1 : 0) + (w[u].y > K0 ? 1 : 0);
        r1 += (w[u].x > K1 ? 1 : 0) + (w[u].y > K1 ? 1 : 0);
      }
    }
    (void)T;
    // the parents' paths were read with the keys: keep their loads up there
    // (left to itself the compiler sinks them below the sums, a second wait)
    asm volatile("" ::"v"(pp0), "v"(pp1));
    // sums over the pair's lane group (aligned, inside one DPP row)
    if (FAST || lt >= 1) { r0 += dpp_i<kDppXor1>(r0); r1 += dpp_i<kDppXor1>(r1); }
    if (FAST || lt >= 2) { r0 += dpp_i<kDppXor2>(r0); r1 += dpp_i<kDppXor2>(r1); }
    if (FAST || lt >= 3) { r0 += dpp_i<kDppHalfMirror>(r0); r1 += dpp_i<kDppHalfMirror>(r1); }
    if (FAST || lt >= 4) { r0 += dpp_i<kDppMirror>(r0); r1 += dpp_i<kDppMirror>(r1); }
    const bool f0 = d < D && r0 < k, f1 = d < D && has1 && r1 < k;
    const int s0 = 1 + dl * k + r0, s1 = 1 + dl * k + r1;
    // lane 0 records node x0, lane p1 node x1: its layer rank, its key in
    // sorted order and, for a frontier node, its slot's source and path
    auto record = [&](int x, int r, uint64_t K, uint64_t pp, int qx, bool f, int sl) __attribute__((always_inline)) {
      lrank[lds_index(lo + x, P, status)] = r;
      skeys[lds_index(dl * LS + r, D * LS, status)] = K;
      const int ss = lds_index(f ? sl : S, S + 1, status);
      slot_src[ss] = lo + x;
      spath[ss] = d == 1 ? (uint64_t)x : ((pp << 4) | (uint64_t)(x - mul_k(qx)));
    };
    if (FAST) {
      if (part < 2 && (part == 0 || has1)) {
        const bool one = part == 1;
        record(one ? x1 : x0, one ? r1 : r0, one ? K1 : K0, one ? pp1 : pp0, one ? q1 : q0, one ? f1 : f0,
               one ? s1 : s0);
      }
      // the frontier's children: lane j writes child j of each frontier node
      const int j = part;
      const bool a0 = f0 && j < k, a1 = f1 && j < k;
      const int rk0 = mul_k(r0) + j, rk1 = mul_k(r1) + j;  // child index inside the next layer
      const int c0 = lo + n + rk0, c1 = lo + n + rk1;        // its pool index: the next layer starts at lo + n
      const float qa = q[lds_index(a0 ? c0 : 0, P, status)], qb = q[lds_index(a1 ? c1 : 0, P, status)];
      uint64_t* Ln = lay + (d < D ? d : 0) * LS;
      *(a0 ? Ln + lds_index(rk0, LS, status) : sink + 2 * part) = node_key(key_value(K0) * qa, c0);
      *(a1 ? Ln + lds_index(rk1, LS, status) : sink + 2 * part + 1) = node_key(key_value(K1) * qb, c1);
    } else {
      if (part == 0) record(x0, r0, K0, pp0, q0, f0, s0);
      if (part == p1 && has1) record(x1, r1, K1, pp1, q1, f1, s1);
      if (f0 || f1) {
        uint64_t* Ln = lay + d * LS;
        const float v0 = key_value(K0), v1 = key_value(K1);
        for (int j = part; j < k; j += tpe) {
          const int c0 = s0 * k + j, c1 = s1 * k + j;
          const float qa = q[lds_index(f0 ? c0 : 0, P, status)], qb = q[lds_index(f1 ? c1 : 0, P, status)];
          if (f0) Ln[lds_index(r0 * k + j, LS, status)] = node_key(v0 * qa, c0);
          if (f1) Ln[lds_index(r1 * k + j, LS, status)] = node_key(v1 * qb, c1);
        }
      }
    }
  };
  if (k <= 11) {
    for (int d = 1; d <= upto; ++d) {
      step(std::true_type{}, d);
      __syncthreads();
    }
  } else {
    for (int d = 1; d <= upto; ++d) {
      step(std::false_type{}, d);
      __syncthreads();
    }
  }

  if (upto < D) {
    for (int x = tid; x < S; x += nt) slot_src_g[(size_t)b * S + x] = slot_src[x];
    return;
  }

  // 2. Rerank.  A candidate's global rank is its layer rank plus, for every
  // other layer, the count of larger keys there (a binary search of that
  // layer's sorted keys).  Two lanes per candidate, each searching every
  // other layer, four searches interleaved.
  const int c1 = min(m, k), cm = min(m, k * k);
  const int ncand = c1 + (D - 1) * cm;
  const int iters = 32 - __clz(cm);  // halvings that cover a prefix of cm keys
  for (int c2 = tid; c2 < 2 * ncand; c2 += nt) {  // nt is even: both lanes of a candidate take the same trip
    const int c = c2 >> 1, h = c2 & 1;
    const int dc = c < c1 ? 0 : 1 + (c - c1) / cm;
    const int r = c < c1 ? c : (c - c1) - (dc - 1) * cm;
    const uint64_t K = skeys[dc * LS + r];
    int above = 0;
    for (int d0 = h; d0 < D; d0 += 8) {
      int lo_[4], hi_[4];
      const uint64_t* A_[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = d0 + 2 * u;
        lo_[u] = 0;
        hi_[u] = (d >= D || d == dc) ? 0 : (d == 0 ? c1 : cm);
        A_[u] = skeys + (d < D ? d : 0) * LS;
      }
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int mid = (lo_[u] + hi_[u]) >> 1;
          const bool act = lo_[u] < hi_[u];
          const bool gt = A_[u][act ? mid : 0] > K;
          lo_[u] = (act && gt) ? mid + 1 : lo_[u];
          hi_[u] = (act && !gt) ? mid : hi_[u];
        }
      }
      above += lo_[0] + lo_[1] + lo_[2] + lo_[3];
    }
    above += dpp_i<kDppXor1>(above);
    const int grank = r + above;
    if (h == 0 && grank < m) {
      const int i = atomicAdd(&n_sel, 1);
      if (i < m) {
        const int e = lds_index(key_node(K), P, status);
        const int de = dc + 1;
        const int ps = div_k(e);
        const uint64_t path = de == 1 ? (uint64_t)e : ((spath[lds_index(ps, S + 1, status)] << 4) | (uint64_t)(e - ps * k));
        sel_e[i] = e;
        sel_dep[i] = de;
        sel_key[i] = D < 16 ? (((uint64_t)de << 60) | path) : (uint64_t)de;
        sel_key2[i] = path;
      }
    }
  }
  __syncthreads();

  // 3. Flatten: a node's flat index is 1 + the count of selected keys below
  // its own; 16 lanes per node.
  const int cnt = n_sel < m ? n_sel : m;
  for (int t = tid; t < cnt * 16; t += nt) {
    const int i = t >> 4, part = t & 15;
    const uint64_t key = sel_key[i], key2 = sel_key2[i];
    int r = 0;
    for (int j = part; j < cnt; j += 16) {
      const uint64_t kj = sel_key[j];
      r += (kj < key || (D >= 16 && kj == key && sel_key2[j] < key2)) ? 1 : 0;
    }
    r += dpp_i<kDppXor1>(r);
    r += dpp_i<kDppXor2>(r);
    r += dpp_i<kDppHalfMirror>(r);
    r += dpp_i<kDppMirror>(r);
    if (part == 0) flat_of[lds_index(sel_e[i], P, status)] = 1 + r;
  }
  __syncthreads();
  int bad = (tid == 0 && n_sel != m) ? 1 : 0;  // keys are distinct, so exactly m are selected
  for (int i = tid; i < cnt; i += nt) {
    const int e = lds_index(sel_e[i], P, status), de = sel_dep[i], f = lds_index(flat_of[e], N, status);
    int pf = 0;
    if (de > 1) {
      const int pe = slot_src[lds_index(e / k, S + 1, status)];
      pf = pe >= 0 ? flat_of[lds_index(pe, P, status)] : -1;
      if (pf < 0) bad = 1;  // parent not selected: the tree would not be connected
    }
    const int lr = lrank[e];
    const size_t o = (size_t)b * N + f;
    fpar[f] = pf;
    fdep[f] = de;
    node_tok[o] = ptok[e];
    node_parent[o] = pf;
    node_depth[o] = de;
    node_sib[o] = e % k;
    node_slot[o] = (de < D && lr < k) ? 1 + (de - 1) * k + lr : -1;
    node_value[o] = key_value(skeys[lds_index((de - 1) * LS + lr, D * LS, status)]);
    node_q[o] = q[e];
  }
  if (bad) set_status(status, EAGLE_STATUS_BAD_TREE);
  for (int e = tid; e < P; e += nt) pool_flat_g[(size_t)b * P + e] = flat_of[e] > 0 ? flat_of[e] : -1;
  for (int x = tid; x < S; x += nt) slot_src_g[(size_t)b * S + x] = slot_src[x];
  if (tid == 0) {
    const size_t o = (size_t)b * N;
    int rt = root_token[b];
    if (rt < 0 || rt >= V) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
    node_tok[o] = rt;
    node_parent[o] = -1;
    node_depth[o] = 0;
    node_sib[o] = -1;
    node_slot[o] = 0;
    node_value[o] = 1.f;
    node_q[o] = 1.f;
  }
  if (mask_out == nullptr) return;
  // 4. The ancestor-only mask and positions of the flattened tree (the rows
  // eagle_build_tree_mask writes): bit j of row f is set iff j is f or one of
  // its ancestors; a node the selection left unset sees itself only.
  __syncthreads();
  const int W = (N + 63) >> 6;
  const int L = prefix_len[b];
  for (int f = tid; f < N; f += nt) {
    uint64_t w[(EAGLE_MAX_NODES + 63) / 64] = {0ull, 0ull, 0ull, 0ull};
    int a = f;
    for (int step = 0; a >= 0 && step <= D; ++step) {
      w[a >> 6] |= 1ull << (a & 63);
      a = a == 0 ? -1 : fpar[lds_index(a, N, status)];
    }
    uint64_t* row = mask_out + ((size_t)b * N + f) * W;
    for (int x = 0; x < W; ++x) row[x] = w[x];
    pos_out[(size_t)b * N + f] = L + fdep[f];
  }
}

}  // namespace

namespace {

// Children of the slots in `sr` (scan + merge).
hipError_t launch_children(int B, int S, int V, int k, float T, uint64_t seed, uint64_t round_id, const float* rows,
                           const uint32_t* bound, int32_t* pool_tok, float* pool_q, float* slot_stats,
                           float* ws_units, int32_t* status, SlotRange sr, hipStream_t st) {
  const bool greedy = !(T > 0.f);
  const float Tp = greedy ? 1.0f : T;
  const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
  const uint32_t rlo = (uint32_t)(round_id & 0xffffffffu);
  const int KP = exp_kp(k);
  const int C = exp_chunks(V);
  dim3 g1(C, B * sr.n);
  if (greedy)
    expand_scan_kernel<kGreedy><<<g1, kExpThreads, 0, st>>>(rows, S, V, Tp, k0, k1, rlo, KP, nullptr, ws_units, status, sr);
  else if (Tp == 1.0f)
    expand_scan_kernel<kSampleT1><<<g1, kExpThreads, 0, st>>>(rows, S, V, Tp, k0, k1, rlo, KP, bound, ws_units, status, sr);
  else
    expand_scan_kernel<kSampleT><<<g1, kExpThreads, 0, st>>>(rows, S, V, Tp, k0, k1, rlo, KP, bound, ws_units, status, sr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int U = C * kExpUnitsPerChunk;
  const size_t sm2 = (size_t)kExpRescanCap * (sizeof(double) + sizeof(int)) +
                     (size_t)U * (1 + exp_unit_floats(k)) * sizeof(float);
  if (greedy)
    expand_merge_kernel<true><<<B * sr.n, kExpThreads, sm2, st>>>(rows, S, V, Tp, k0, k1, rlo, k, KP, C, nullptr, ws_units,
                                                                pool_tok, pool_q, slot_stats, status, sr);
  else
    expand_merge_kernel<false><<<B * sr.n, kExpThreads, sm2, st>>>(rows, S, V, Tp, k0, k1, rlo, k, KP, C, bound, ws_units,
                                                                 pool_tok, pool_q, slot_stats, status, sr);
  return hipGetLastError();
}

// Static tree: one workgroup per request, one thread per node of the shape.
// Node c > 0 is child sib[c] of its parent's slot: its token and confidence
// are that pool entry's, its value the fp32 product of the confidences on its
// root path, multiplied from the root down.  Pool entries past a slot's own
// child count are no draws (-1, q 0); pool_flat maps each drawn child to its
// node.
constexpr int kStaticThreads = 256;
__global__ __launch_bounds__(kStaticThreads) void static_assemble_kernel(
    StaticShape sh, int k, int V, const int32_t* __restrict__ root_token, int32_t* __restrict__ pool_tok,
    float* __restrict__ pool_q, int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
    int32_t* node_slot, float* node_value, float* node_q, int32_t* __restrict__ pool_flat,
    int32_t* __restrict__ slot_src, int32_t* status) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = sh.n, S = sh.S;
  const size_t P = (size_t)S * k;
  // entries that are no draws: pool rows past the slot's count (disjoint from
  // the entries the nodes below read and map)
  for (int e = tid; e < S * k; e += kStaticThreads) {
    const int s = e / k, j = e - s * k;
    if (j >= sh.slot_k[s]) {
      pool_tok[b * P + e] = -1;
      pool_q[b * P + e] = 0.f;
      pool_flat[b * P + e] = -1;
    }
  }
  for (int s = tid; s < S; s += kStaticThreads) {
    const int u = sh.slot_node[s];
    slot_src[(size_t)b * S + s] = u == 0 ? -1 : sh.slot[sh.parent[u]] * k + sh.sib[u];
  }
  const int c = tid;
  if (c >= n) return;
  const size_t o = (size_t)b * n + c;
  if (c == 0) {
    const int rt = root_token[b];
    if (rt < 0 || rt >= V) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
    node_tok[o] = rt;
    node_parent[o] = -1;
    node_depth[o] = 0;
    node_sib[o] = -1;
    node_slot[o] = sh.slot[0];
    node_value[o] = 1.f;
    node_q[o] = 1.f;
    return;
  }
  const int par = sh.parent[c];
  const size_t e = (size_t)sh.slot[par] * k + sh.sib[c];
  const int tok = pool_tok[b * P + e];
  if (tok < 0 || tok >= V) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
  // confidences of the path, deepest first, then multiplied from the root down
  float qs[EAGLE_MAX_DEPTH];
  int nq = 0;
  for (int a = c; a > 0 && nq < EAGLE_MAX_DEPTH; a = sh.parent[a])
    qs[nq++] = pool_q[b * P + (size_t)sh.slot[sh.parent[a]] * k + sh.sib[a]];
  float v = 1.f;
  for (int i = nq - 1; i >= 0; --i) v = v * qs[i];
  node_tok[o] = tok;
  node_parent[o] = par;
  node_depth[o] = sh.depth[c];
  node_sib[o] = sh.sib[c];
  node_slot[o] = sh.slot[c];
  node_value[o] = v;
  node_q[o] = qs[0];
  pool_flat[b * P + e] = c;
}

hipError_t launch_assemble(int B, int S, int V, int D, int k, int m, int upto, const int32_t* root,
                           int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
                           int32_t* node_slot, float* node_value, float* node_q, const int32_t* pool_tok,
                           const float* pool_q, int32_t* pool_flat, int32_t* slot_src, int32_t* status,
                           hipStream_t st, const int32_t* prefix_len = nullptr, uint64_t* mask = nullptr,
                           int32_t* pos = nullptr) {
  const int P = S * k;
  const size_t LS = (size_t)((k * k + 1) & ~1);
  const size_t sm3 = (2 * (size_t)D * LS + 2 + 32 + S + 1 + 2 * (size_t)m) * 8 + (size_t)P * 4 * 4 + (size_t)(S + 1) * 4 +
                     (size_t)m * 2 * 4 + 2 * (size_t)(m + 1) * 4;
  tree_assemble_kernel<<<B, kTreeThreads, sm3, st>>>(S, k, D, m, V, root, pool_tok, pool_q, node_tok, node_parent,
                                                     node_depth, node_sib, node_slot, node_value, node_q, pool_flat,
                                                     slot_src, status, upto, prefix_len, mask, pos);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(int B, int S, int V, int D, int k, int m, float T, uint64_t seed,
                         uint64_t round_id, const float* rows, const uint32_t* bound, const int32_t* root,
                         int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                         int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                         int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                         float* slot_stats, float* ws_units, int32_t* status, hipStream_t st,
                         const int32_t* prefix_len, uint64_t* mask, int32_t* pos) {
  hipError_t e = launch_children(B, S, V, k, T, seed, round_id, rows, bound, pool_tok, pool_q, slot_stats, ws_units,
                                 status, SlotRange{0, S}, st);
  if (e != hipSuccess) return e;
  return launch_assemble(B, S, V, D, k, m, D, root, node_tok, node_parent, node_depth, node_sib, node_slot,
                         node_value, node_q, pool_tok, pool_q, pool_flat, slot_src, status, st, prefix_len, mask,
                         pos);
}

hipError_t launch_expand_depth(int B, int S, int V, int D, int k, int m, float T, uint64_t seed, uint64_t round_id,
                               int depth, const float* rows, const uint32_t* bound, int32_t* pool_tok, float* pool_q,
                               int32_t* slot_src, float* slot_stats, float* ws_units, int32_t* status, hipStream_t st) {
  const SlotRange sr = depth == 0 ? SlotRange{0, 1} : SlotRange{1 + (depth - 1) * k, k};
  hipError_t e = launch_children(B, S, V, k, T, seed, round_id, rows, bound, pool_tok, pool_q, slot_stats, ws_units,
                                 status, sr, st);
  if (e != hipSuccess || depth + 1 >= D) return e;
  // the next depth's frontier (slot_src of its slots); no node is written
  return launch_assemble(B, S, V, D, k, m, depth + 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, pool_tok, pool_q, nullptr, slot_src, status, st);
}

hipError_t launch_expand_static(int B, int V, const StaticShape& sh, float T, uint64_t seed, uint64_t round_id,
                                const float* rows, const int32_t* root, int32_t* node_tok, int32_t* node_parent,
                                int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value,
                                float* node_q, int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                                float* slot_stats, float* ws_units, int32_t* status, hipStream_t st) {
  const int S = sh.S, k = sh.kmax;
  hipError_t e = launch_children(B, S, V, k, T, seed, round_id, rows, nullptr, pool_tok, pool_q, slot_stats, ws_units,
                                 status, SlotRange{0, S}, st);
  if (e != hipSuccess) return e;
  static_assemble_kernel<<<B, kStaticThreads, 0, st>>>(sh, k, V, root, pool_tok, pool_q, node_tok, node_parent,
                                                       node_depth, node_sib, node_slot, node_value, node_q, pool_flat,
                                                       slot_src, status);
  return hipGetLastError();
}

hipError_t launch_expand_finish(int B, int S, int V, int D, int k, int m, const int32_t* root, int32_t* node_tok,
                                int32_t* node_parent, int32_t* node_depth, int32_t* node_sib, int32_t* node_slot,
                                float* node_value, float* node_q, const int32_t* pool_tok, const float* pool_q,
                                int32_t* pool_flat, int32_t* slot_src, int32_t* status, hipStream_t st) {
  return launch_assemble(B, S, V, D, k, m, D, root, node_tok, node_parent, node_depth, node_sib, node_slot,
                         node_value, node_q, pool_tok, pool_q, pool_flat, slot_src, status, st);
}

}  // namespace eagle
