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
//                 z; sampling: t + Gumbel noise from Philox).  HBM-bound.
//   expand_merge  grid B*S, 256 threads.  Merges the wave records of a row:
//                 M, S (fp64 sum), exact fp64 keys of the candidates, the k
//                 best in sampling order, their confidences q.  Proves that
//                 the candidate set holds the exact top-k (else re-scans the
//                 row: rare).
//   tree_assemble grid B, 256 threads, all state in LDS.  Values, frontier
//                 ranks per layer, rerank of the pool by merging per-layer
//                 sorted lists, BFS flattening.
#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace eagle {

namespace {

constexpr int kPer = 16;  // logits per thread in the scan

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

template <bool GREEDY>
__global__ __launch_bounds__(kExpThreads) void expand_scan_kernel(
    const float* __restrict__ rows, int S, int V, float Tp, uint32_t k0, uint32_t k1,
    uint32_t round_lo, int KP, float* __restrict__ units, int32_t* status) {
  const int row = blockIdx.y;
  const int b = row / S, s = row - b * S;
  const int chunk = blockIdx.x;
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
    uint4 w4 = make_uint4(0, 0, 0, 0);
    if (!GREEDY) w4 = philox4x32_10(make_uint4((uint32_t)base >> 2, (uint32_t)s, (uint32_t)b, round_lo), k0, k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = it * 4 + e;
      const bool valid = base + e < V;
      float x = zz[e];
      if (valid && !isfinite(x)) { bad = true; x = kNegInf; }
      if (!valid) x = kNegInf;
      t[j] = x / Tp;
      if (GREEDY) {
        key[j] = x;
      } else {
        const uint32_t wd = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
        key[j] = (x == kNegInf) ? kNegInf : t[j] + gumbel_f32(word_to_uniform(wd));
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
#pragma unroll
    for (int j = 0; j < kPer; ++j) ls += (t[j] == kNegInf) ? 0.f : expf(t[j] - wm);
  }
  const float wsum = wave_sum(ls);

  // The wave's KP best (key desc, idx asc), by repeated wave argmax.
  UnitView u{units + ((size_t)row * gridDim.x * kExpUnitsPerChunk + (size_t)chunk * kExpUnitsPerChunk + wave) * (2 + 2 * KP), KP};
  uint32_t taken = 0;
  auto idx_of = [&](int j) { return chunk * kExpChunk + (j >> 2) * (kExpThreads * 4) + tid * 4 + (j & 3); };
  float bk = kNegInf;
  int bi = kIdxNone;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int id = idx_of(j);
    if (id < V && beats(key[j], id, bk, bi)) { bk = key[j]; bi = id; }
  }
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
                            uint32_t round_lo) {
  const float zz = z[idx];
  if (!isfinite(zz)) return -__builtin_huge_val();
  if (GREEDY) return (double)zz;
  const float t = zz / Tp;
  return (double)t + gumbel_f64(token_uniform(idx, s, b, round_lo, k0, k1));
}

template <bool GREEDY>
__global__ __launch_bounds__(kExpThreads) void expand_merge_kernel(
    const float* __restrict__ rows, int S, int V, float Tp, uint32_t k0, uint32_t k1,
    uint32_t round_lo, int k, int KP, int C, const float* __restrict__ units,
    int32_t* __restrict__ pool_tok, float* __restrict__ pool_q, float* __restrict__ slot_stats,
    int32_t* status) {
  extern __shared__ unsigned char smem_raw[];
  const int row = blockIdx.x;
  const int b = row / S, s = row - b * S;
  const int tid = threadIdx.x;
  const int U = C * kExpUnitsPerChunk;
  const int UF = 2 + 2 * KP;
  const float* z = rows + (size_t)row * V;
  const float* ub = units + (size_t)row * U * UF;

  __shared__ double shd[4];
  __shared__ float shf[4];
  __shared__ int shi[4];
  __shared__ double sel_key[EAGLE_MAX_TOPK];
  __shared__ int sel_idx[EAGLE_MAX_TOPK];
  __shared__ int n_cand;

  // Row statistics from the wave records.
  float lm = kNegInf;
  for (int x = tid; x < U; x += kExpThreads) lm = fmaxf(lm, ub[(size_t)x * UF]);
  const float M = block_max_256(lm, shf);
  double ls = 0.0;
  if (M != kNegInf)
    for (int x = tid; x < U; x += kExpThreads) {
      const float um = ub[(size_t)x * UF], us = ub[(size_t)x * UF + 1];
      if (us > 0.f) ls += (double)us * exp((double)um - (double)M);
    }
  const double Sd = block_sum_256(ls, shd);

  // Candidates with exact keys.
  const int ncand0 = U * KP;
  const int cap = ncand0 > kExpRescanCap ? ncand0 : kExpRescanCap;
  double* ckey = reinterpret_cast<double*>(smem_raw);
  int* cidx = reinterpret_cast<int*>(smem_raw + sizeof(double) * cap);
  for (int c = tid; c < ncand0; c += kExpThreads) {
    const int x = c / KP, r = c - x * KP;
    const int id = __float_as_int(ub[(size_t)x * UF + 2 + KP + r]);
    if (id == kIdxNone || id < 0 || id >= V) {
      ckey[c] = -__builtin_huge_val();
      cidx[c] = kIdxNone;
    } else {
      ckey[c] = exact_key<GREEDY>(z, id, s, b, Tp, k0, k1, round_lo);
      cidx[c] = id;
    }
  }
  if (tid == 0) n_cand = ncand0;
  __syncthreads();

  for (int pass = 0; pass < 2; ++pass) {
    const int nc = n_cand;
    // Select the k best by repeated block argmax.
    double bk = -__builtin_huge_val();
    int bi = kIdxNone;
    for (int c = tid; c < nc; c += kExpThreads)
      if (beats_d(ckey[c], cidx[c], bk, bi)) { bk = ckey[c]; bi = cidx[c]; }
    for (int r = 0; r < k; ++r) {
      double wk = bk;
      int wi = bi;
      block_argmax_256(wk, wi, shd, shi);
      if (tid == 0) { sel_key[r] = wk; sel_idx[r] = wi; }
      if (wi != kIdxNone && bi == wi) {
        bk = -__builtin_huge_val();
        bi = kIdxNone;
        for (int c = tid; c < nc; c += kExpThreads) {
          if (cidx[c] == wi) { cidx[c] = kIdxNone; ckey[c] = -__builtin_huge_val(); }
          else if (beats_d(ckey[c], cidx[c], bk, bi)) { bk = ckey[c]; bi = cidx[c]; }
        }
      }
    }
    __syncthreads();
    if (GREEDY || pass == 1) break;

    // Proof that no dropped logit can reach the k-th exact key: every wave
    // record that is full must end strictly below it (minus the fp32 key error).
    const double Ek = sel_key[k - 1];
    const double delta = 8e-7 * (fabs(Ek) + 24.0);
    int need = 0;
    for (int x = tid; x < U; x += kExpThreads) {
      const int last = __float_as_int(ub[(size_t)x * UF + 2 + KP + (KP - 1)]);
      if (last != kIdxNone && (double)ub[(size_t)x * UF + 2 + (KP - 1)] + delta >= Ek) need = 1;
    }
    if (!block_or_256(need, shi)) break;

    // Rare: re-scan the row, keeping every logit whose fp32 key can reach Ek.
    if (tid == 0) { n_cand = 0; set_status(status, EAGLE_STATUS_TOPK_RESCAN); }
    __syncthreads();
    const double thr = Ek - delta;
    for (int v = tid; v < V; v += kExpThreads) {
      const float zz = z[v];
      if (!isfinite(zz)) continue;
      const float t = zz / Tp;
      const float ka = t + gumbel_f32(token_uniform(v, s, b, round_lo, k0, k1));
      if ((double)ka >= thr) {
        const int slot = atomicAdd(&n_cand, 1);
        if (slot < cap) { cidx[slot] = v; ckey[slot] = exact_key<GREEDY>(z, v, s, b, Tp, k0, k1, round_lo); }
      }
    }
    __syncthreads();
    if (n_cand > cap) {
      if (tid == 0) { set_status(status, EAGLE_STATUS_CAND_OVERFLOW); n_cand = cap; }
      __syncthreads();
    }
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

struct TreeSmem {
  float* val;
  float* q;
  int* lrank;
  int* sorted;
  int* slot_of;
  int* flat_of;
  int* gkey;
  int* slot_src;
};

EDEV int layer_lo(int d, int k) { return d == 1 ? 0 : k + (d - 2) * k * k; }
EDEV int layer_n(int d, int k) { return d == 1 ? k : k * k; }
EDEV int depth_of(int e, int k) { return e < k ? 1 : 2 + (e - k) / (k * k); }
EDEV bool vbeats(const float* val, int f, int e) { return val[f] > val[e] || (val[f] == val[e] && f < e); }

__global__ __launch_bounds__(256) void tree_assemble_kernel(
    int S, int k, int D, int m, int V, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ pool_tok_g, const float* __restrict__ pool_q_g,
    int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
    int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_flat_g,
    int32_t* slot_src_g, int32_t* status) {
  extern __shared__ unsigned char smem_raw[];
  const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int P = S * k, N = m + 1;
  TreeSmem sm;
  sm.val = reinterpret_cast<float*>(smem_raw);
  sm.q = sm.val + P;
  sm.lrank = reinterpret_cast<int*>(sm.q + P);
  sm.sorted = sm.lrank + P;
  sm.slot_of = sm.sorted + P;
  sm.flat_of = sm.slot_of + P;
  sm.gkey = sm.flat_of + P;
  sm.slot_src = sm.gkey + P;
  __shared__ int cnt[EAGLE_MAX_DEPTH + 2];
  __shared__ int base[EAGLE_MAX_DEPTH + 2];

  const float* pq = pool_q_g + (size_t)b * P;
  for (int e = tid; e < P; e += nt) {
    sm.q[e] = pq[e];
    sm.val[e] = e < k ? pq[e] : 0.f;  // layer 1: V = 1 * q
    sm.slot_of[e] = -1;
    sm.flat_of[e] = -1;
  }
  for (int x = tid; x < S; x += nt) sm.slot_src[x] = -1;
  if (tid <= D + 1) cnt[tid] = 0;
  __syncthreads();

  // Layer by layer: rank within the layer, frontier -> slots, children values.
  for (int d = 1; d <= D; ++d) {
    const int lo = layer_lo(d, k), n = layer_n(d, k);
    for (int x = tid; x < n; x += nt) {
      const int e = lo + x;
      int r = 0;
      for (int y = 0; y < n; ++y) r += vbeats(sm.val, lo + y, e) ? 1 : 0;
      sm.lrank[e] = r;
      sm.sorted[lo + r] = e;
      if (d < D && r < k) {
        const int slot = 1 + (d - 1) * k + r;
        sm.slot_src[slot] = e;
        sm.slot_of[e] = slot;
      }
    }
    __syncthreads();
    if (d < D) {
      for (int c = tid; c < k * k; c += nt) {
        const int slot = 1 + (d - 1) * k + c / k;
        const int child = slot * k + (c % k);
        const int par = sm.slot_src[slot];
        sm.val[child] = sm.val[par] * sm.q[child];
      }
      __syncthreads();
    }
  }

  // Rerank: global rank = own layer rank + members of other layers that beat e.
  for (int e = tid; e < P; e += nt) {
    int g = sm.lrank[e];
    if (g < m) {
      const int de = depth_of(e, k);
      for (int d = 1; d <= D && g < m; ++d) {
        if (d == de) continue;
        const int lo = layer_lo(d, k), n = layer_n(d, k);
        int a = 0, z = n;  // count of sorted prefix beating e
        while (a < z) {
          const int mid = (a + z) >> 1;
          if (vbeats(sm.val, sm.sorted[lo + mid], e)) a = mid + 1; else z = mid;
        }
        g += a;
      }
    }
    if (g < m) {
      sm.flat_of[e] = 0;  // selected, flat index assigned below
      atomicAdd(&cnt[depth_of(e, k)], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    base[1] = 1;
    for (int d = 1; d <= D; ++d) base[d + 1] = base[d] + cnt[d];
  }
  __syncthreads();

  // Flatten: (depth, parent flat index, sibling rank).
  int bad = 0;
  for (int d = 1; d <= D; ++d) {
    const int lo = layer_lo(d, k), n = layer_n(d, k);
    for (int x = tid; x < n; x += nt) {
      const int e = lo + x;
      if (sm.flat_of[e] < 0) continue;
      int pf = 0;
      if (d > 1) {
        pf = sm.flat_of[sm.slot_src[e / k]];
        if (pf <= 0) bad = 1;
      }
      sm.gkey[e] = pf * k + (e % k);
    }
    __syncthreads();
    for (int x = tid; x < n; x += nt) {
      const int e = lo + x;
      if (sm.flat_of[e] < 0) continue;
      int r = 0;
      for (int y = 0; y < n; ++y) {
        const int f = lo + y;
        r += (sm.flat_of[f] >= 0 && sm.gkey[f] < sm.gkey[e]) ? 1 : 0;
      }
      const int flat = base[d] + r;
      if (flat >= N) { bad = 1; continue; }  // cannot happen for a strict rank order; never write out of range
      const size_t o = (size_t)b * N + flat;
      node_tok[o] = pool_tok_g[(size_t)b * P + e];
      node_parent[o] = d == 1 ? 0 : sm.gkey[e] / k;
      node_depth[o] = d;
      node_sib[o] = e % k;
      node_slot[o] = sm.slot_of[e];
      node_value[o] = sm.val[e];
      node_q[o] = sm.q[e];
      sm.lrank[e] = flat;  // lrank no longer needed: holds the flat index
    }
    __syncthreads();
    for (int x = tid; x < n; x += nt) {
      const int e = lo + x;
      if (sm.flat_of[e] >= 0) sm.flat_of[e] = sm.lrank[e];
    }
    __syncthreads();
  }
  if (bad) set_status(status, EAGLE_STATUS_BAD_TREE);
  for (int e = tid; e < P; e += nt) pool_flat_g[(size_t)b * P + e] = sm.flat_of[e];
  for (int x = tid; x < S; x += nt) slot_src_g[(size_t)b * S + x] = sm.slot_src[x];
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
}

}  // namespace

hipError_t launch_expand(int B, int S, int V, int D, int k, int m, float T, uint64_t seed,
                         uint64_t round_id, const float* rows, const int32_t* root,
                         int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                         int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                         int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                         float* slot_stats, float* ws_units, int32_t* status, hipStream_t st) {
  const bool greedy = !(T > 0.f);
  const float Tp = greedy ? 1.0f : T;
  const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
  const uint32_t rlo = (uint32_t)(round_id & 0xffffffffu);
  const int KP = exp_kp(k);
  const int C = exp_chunks(V);
  dim3 g1(C, B * S);
  if (greedy)
    expand_scan_kernel<true><<<g1, kExpThreads, 0, st>>>(rows, S, V, Tp, k0, k1, rlo, KP, ws_units, status);
  else
    expand_scan_kernel<false><<<g1, kExpThreads, 0, st>>>(rows, S, V, Tp, k0, k1, rlo, KP, ws_units, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ncand = C * kExpUnitsPerChunk * KP;
  const int cap = ncand > kExpRescanCap ? ncand : kExpRescanCap;
  const size_t sm2 = (size_t)cap * (sizeof(double) + sizeof(int));
  if (greedy)
    expand_merge_kernel<true><<<B * S, kExpThreads, sm2, st>>>(rows, S, V, Tp, k0, k1, rlo, k, KP, C, ws_units,
                                                             pool_tok, pool_q, slot_stats, status);
  else
    expand_merge_kernel<false><<<B * S, kExpThreads, sm2, st>>>(rows, S, V, Tp, k0, k1, rlo, k, KP, C, ws_units,
                                                              pool_tok, pool_q, slot_stats, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = S * k;
  const size_t sm3 = (size_t)P * 7 * 4 + (size_t)S * 4;
  tree_assemble_kernel<<<B, 256, sm3, st>>>(S, k, D, m, V, root, pool_tok, pool_q, node_tok, node_parent,
                                            node_depth, node_sib, node_slot, node_value, node_q, pool_flat,
                                            slot_src, status);
  return hipGetLastError();
}

}  // namespace eagle
