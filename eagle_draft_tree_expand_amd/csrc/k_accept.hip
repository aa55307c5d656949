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
// One workgroup of 1024 threads per request.  The adjusted distributions are
// never materialised: after rejecting x_0..x_{j-1} (drawn without replacement
// from q) the unnormalised residual is max(0, p(y) - s_j q(y)) for untried y
// and a frozen value f_i for each tried x_i, with s_0 = 0, Z_0 = R_0 = 1,
//   s_{j+1} = s_j + Z_j / R_j,  R_{j+1} = R_j - q(x_j),
//   f_j = max(0, p(x_j) - s_{j+1} q(x_j)),  Z_{j+1} = sum of the residual,
// (induction on P <- norm(max(0, P - Q)), Q <- Q without x_j, renormalised).
// So each rejection costs one vocabulary reduction G(s) = sum_y max(0, p - s q),
// and the final draw one more pass over a single 4096-token chunk.  The
// acceptance ratio of trial j is max(0, p(x_j) - s_j q(x_j)) R_j / (Z_j q(x_j)),
// with p(x_j), q(x_j) evaluated in fp64.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = kThreads * 4;         // token ids per reduction chunk
constexpr int kMaxChunks = (EAGLE_MAX_VOCAB + kChunk - 1) / kChunk;
constexpr double kTie = 1e-6;

struct Rows {
  const float* zp;  // target logits row of the node
  const float* zq;  // draft logits row of the node's slot (may be null when s == 0)
  float Mp, Mq, Tp;
  double invSp, invSq;
};

// Residual term of one token from fp32 exponentials (the bulk formula).
EDEV double resid_term(float zp, float zq, const Rows& R, double s) {
  const double p = isfinite(zp) ? (double)expf(zp / R.Tp - R.Mp) * R.invSp : 0.0;
  if (s == 0.0) return p;
  const double q = isfinite(zq) ? (double)expf(zq / R.Tp - R.Mq) * R.invSq : 0.0;
  const double d = p - s * q;
  return d > 0.0 ? d : 0.0;
}

// fp64 probabilities of one token (used for acceptance ratios and R).
EDEV double prob64(float z, float M, double invS, float Tp) {
  if (!isfinite(z)) return 0.0;
  return exp((double)(z / Tp) - (double)M) * invS;
}

struct Shared {
  double csum[kMaxChunks];          // chunk sums of the last reduction
  double wpart[kMaxChunks][kWaves]; // per-wave partials
  double scan[kWaves];
  double bc_d[4];
  int bc_i[4];
  int tried_x[EAGLE_MAX_TOPK];
  double tried_f[EAGLE_MAX_TOPK];
};

// All threads: chunk sums and total of the residual at s (tried tokens not
// yet corrected).  Result total broadcast to all threads.
EDEV double reduce_pass(const Rows& R, double s, int V, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (V + kChunk - 1) / kChunk;
  const bool vec = ((V & 3) == 0) && (((uintptr_t)R.zp & 15) == 0) && (R.zq == nullptr || ((uintptr_t)R.zq & 15) == 0);
  for (int c = 0; c < nch; ++c) {
    const int base = c * kChunk + tid * 4;
    double a = 0.0;
    if (vec && base + 3 < V) {
      const float4 p4 = *reinterpret_cast<const float4*>(R.zp + base);
      float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s != 0.0) q4 = *reinterpret_cast<const float4*>(R.zq + base);
      a = resid_term(p4.x, q4.x, R, s) + resid_term(p4.y, q4.y, R, s) + resid_term(p4.z, q4.z, R, s) +
          resid_term(p4.w, q4.w, R, s);
    } else {
      for (int e = 0; e < 4; ++e) {
        const int v = base + e;
        if (v < V) a += resid_term(R.zp[v], s != 0.0 ? R.zq[v] : 0.f, R, s);
      }
    }
    a = wave_sum_d(a);
    if (lane == 0) sh.wpart[c][wave] = a;
  }
  __syncthreads();
  for (int c = tid; c < nch; c += kThreads) {
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) t += sh.wpart[c][w];
    sh.csum[c] = t;
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int c = 0; c < nch; ++c) t += sh.csum[c];
    sh.bc_d[0] = t;
  }
  __syncthreads();
  const double tot = sh.bc_d[0];
  __syncthreads();
  return tot;
}

// All threads: inverse-CDF draw from the residual at s (chunk sums from the
// reduce_pass at the same s), tried tokens replaced by their frozen values.
// Returns the token and counts a near tie into *ties (thread 0).
EDEV int draw_pass(const Rows& R, double s, int V, int ntried, double uval, Shared& sh, int* ties) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (V + kChunk - 1) / kChunk;
  if (tid == 0) {
    // corrected chunk sums and total
    for (int i = 0; i < ntried; ++i) {
      const int x = sh.tried_x[i];
      const double cur = resid_term(R.zp[x], s != 0.0 ? R.zq[x] : 0.f, R, s);
      sh.csum[x / kChunk] += sh.tried_f[i] - cur;
    }
    double tot = 0.0;
    for (int c = 0; c < nch; ++c) tot += sh.csum[c] > 0.0 ? sh.csum[c] : 0.0;
    const double target = uval * tot;
    double cum = 0.0;
    int cstar = -1;
    for (int c = 0; c < nch; ++c) {
      const double cs = sh.csum[c] > 0.0 ? sh.csum[c] : 0.0;
      if (cs > 0.0 && cum + cs > target) { cstar = c; break; }
      cum += cs;
    }
    if (cstar < 0) {  // rounding: take the last chunk with mass
      for (int c = nch - 1; c >= 0; --c)
        if (sh.csum[c] > 0.0) { cstar = c; break; }
      cum = 0.0;
      for (int c = 0; c < cstar; ++c) cum += sh.csum[c] > 0.0 ? sh.csum[c] : 0.0;
    }
    sh.bc_i[0] = cstar;
    sh.bc_d[1] = target - cum;  // offset inside the chunk
    sh.bc_d[2] = tot;
  }
  __syncthreads();
  const int cstar = sh.bc_i[0];
  const double off = sh.bc_d[1], tot = sh.bc_d[2];
  // per-thread values of the chunk (ids cstar*4096 + 4*tid + e)
  double val[4];
  double mine = 0.0;
  for (int e = 0; e < 4; ++e) {
    const int v = (cstar < 0 ? 0 : cstar) * kChunk + tid * 4 + e;
    double x = 0.0;
    if (cstar >= 0 && v < V) {
      x = resid_term(R.zp[v], s != 0.0 ? R.zq[v] : 0.f, R, s);
      for (int i = 0; i < ntried; ++i)
        if (sh.tried_x[i] == v) x = sh.tried_f[i];
    }
    val[e] = x;
    mine += x;
  }
  // inclusive scan over threads (id order)
  double inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh.scan[wave] = inc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) { const double y = sh.scan[w]; sh.scan[w] = t; t += y; }
    sh.bc_i[1] = -1;
  }
  __syncthreads();
  inc += sh.scan[wave];
  const double exc = inc - mine;
  // the thread whose [exc, inc) holds off picks inside its 4 values
  if (mine > 0.0 && exc <= off && off < inc) {
    double c = exc;
    int pick = -1;
    for (int e = 0; e < 4; ++e) {
      if (val[e] > 0.0 && c + val[e] > off) {
        pick = e;
        if ((off - c) < kTie * tot || (c + val[e] - off) < kTie * tot) atomicAdd(ties, 1);
        break;
      }
      c += val[e];
    }
    if (pick < 0) for (int e = 3; e >= 0; --e) if (val[e] > 0.0) { pick = e; break; }
    atomicMax(&sh.bc_i[1], cstar * kChunk + tid * 4 + pick);
  }
  __syncthreads();
  if (tid == 0 && sh.bc_i[1] < 0) {
    // rounding beyond the chunk's last positive value: take the last positive id
    int last = -1;
    for (int e = kChunk - 1; e >= 0 && last < 0 && cstar >= 0; --e) {
      const int v = cstar * kChunk + e;
      if (v >= V) continue;
      double x = resid_term(R.zp[v], s != 0.0 ? R.zq[v] : 0.f, R, s);
      for (int i = 0; i < ntried; ++i)
        if (sh.tried_x[i] == v) x = sh.tried_f[i];
      if (x > 0.0) last = v;
    }
    sh.bc_i[1] = last < 0 ? 0 : last;
  }
  __syncthreads();
  const int y = sh.bc_i[1];
  __syncthreads();
  return y;
}

__global__ __launch_bounds__(kThreads) void accept_kernel(
    int N, int V, int D, int k, float T, const int32_t* __restrict__ node_tok, const int32_t* __restrict__ node_parent,
    const int32_t* __restrict__ node_slot, const int32_t* __restrict__ pool_tok, const int32_t* __restrict__ pool_flat,
    const float* __restrict__ tlog, const float* __restrict__ tstats, const int32_t* __restrict__ targmax,
    const float* __restrict__ dlog, const float* __restrict__ sstats, const float* __restrict__ uniforms,
    int32_t* accept_len, int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
    int32_t* status) {
  __shared__ Shared sh;
  __shared__ int ties;
  __shared__ int path[EAGLE_MAX_DEPTH + 1];
  __shared__ int comm[EAGLE_MAX_DEPTH + 2];
  __shared__ int npath, ncomm;
  __shared__ int cur_u, cur_slot, acc_j, zero_resid;
  __shared__ double st_s, st_Z, st_R;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int S = 1 + (D - 1) * k;
  const bool greedy = !(T > 0.f);
  const float Tp = greedy ? 1.f : T;
  const int32_t* ntok = node_tok + (size_t)b * N;
  const int32_t* npar = node_parent + (size_t)b * N;
  const int32_t* nslot = node_slot + (size_t)b * N;
  const int32_t* ptok = pool_tok + (size_t)b * S * k;
  const int32_t* pflat = pool_flat + (size_t)b * S * k;
  const float* U = uniforms + (size_t)b * N * (k + 1);
  if (tid == 0) { ties = 0; npath = 0; ncomm = 0; cur_u = 0; zero_resid = 0; }
  __syncthreads();

  if (greedy) {
    if (tid == 0) {
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
    for (int step = 0; step <= D; ++step) {
      if (tid == 0) cur_slot = nslot[cur_u];
      __syncthreads();
      const int u = cur_u, slot = cur_slot;
      const float* zp = tlog + ((size_t)b * N + u) * V;
      Rows R;
      R.zp = zp;
      R.Tp = Tp;
      R.Mp = tstats[((size_t)b * N + u) * 2];
      R.invSp = 1.0 / (double)tstats[((size_t)b * N + u) * 2 + 1];
      if (slot < 0 || slot >= S) {
        // never expanded: bonus token from the target
        R.zq = nullptr; R.Mq = 0.f; R.invSq = 0.0;
        reduce_pass(R, 0.0, V, sh);
        const int y = draw_pass(R, 0.0, V, 0, (double)U[(size_t)u * (k + 1) + k], sh, &ties);
        if (tid == 0) comm[ncomm++] = y;
        break;
      }
      R.zq = dlog + ((size_t)b * S + slot) * V;
      R.Mq = sstats[((size_t)b * S + slot) * 2];
      R.invSq = 1.0 / (double)sstats[((size_t)b * S + slot) * 2 + 1];
      if (tid == 0) { st_s = 0.0; st_Z = 1.0; st_R = 1.0; acc_j = -1; }
      __syncthreads();
      int ntried = 0;
      bool stale = false;  // chunk sums do not match st_s
      for (int j = 0; j < k; ++j) {
        if (tid == 0) {
          const int x = ptok[(size_t)slot * k + j];
          if (x < 0 || x >= V) {
            set_status(status, EAGLE_STATUS_TOKEN_RANGE);
          } else {
            const double px = prob64(R.zp[x], R.Mp, R.invSp, Tp);
            const double qx = prob64(R.zq[x], R.Mq, R.invSq, Tp);
            const double num = st_s == 0.0 ? px : fmax(0.0, px - st_s * qx);
            double ratio;
            if (qx > 0.0 && st_R > 0.0) ratio = num * st_R / (st_Z * qx);
            else ratio = num > 0.0 ? __builtin_huge_val() : 0.0;
            const double a = ratio < 1.0 ? ratio : 1.0;
            const double uu = (double)U[(size_t)u * (k + 1) + j];
            if (fabs(uu - a) < kTie) ++ties;
            if (uu < a) acc_j = j;
          }
        }
        __syncthreads();
        if (acc_j >= 0) break;
        // rejected: s_{j+1}, R_{j+1}, frozen f_j, then Z_{j+1} by one reduction
        if (tid == 0) {
          const int x = ptok[(size_t)slot * k + j];
          const int xc = (x < 0 || x >= V) ? 0 : x;
          const double qx = prob64(R.zq[xc], R.Mq, R.invSq, Tp);
          sh.bc_d[3] = st_s + st_Z / st_R;          // candidate s_{j+1}
          sh.tried_x[ntried] = xc;
          st_R = st_R - qx;
        }
        __syncthreads();
        const double snew = sh.bc_d[3];
        const double G = reduce_pass(R, snew, V, sh);
        if (tid == 0) {
          double Z = G;
          for (int i = 0; i < ntried; ++i) {
            const int xi = sh.tried_x[i];
            Z += sh.tried_f[i] - resid_term(R.zp[xi], R.zq[xi], R, snew);
          }
          const int xj = sh.tried_x[ntried];
          if (Z > 0.0) {
            sh.tried_f[ntried] = resid_term(R.zp[xj], R.zq[xj], R, snew);
            st_s = snew;
            st_Z = Z;
            sh.bc_i[2] = 0;
          } else {  // zero residual mass: keep P
            sh.tried_f[ntried] = resid_term(R.zp[xj], R.zq[xj], R, st_s);
            zero_resid = 1;
            sh.bc_i[2] = 1;
          }
        }
        __syncthreads();
        stale = sh.bc_i[2] != 0;
        ++ntried;
      }
      if (acc_j >= 0) {
        if (tid == 0) {
          const int x = ptok[(size_t)slot * k + acc_j];
          comm[ncomm++] = x;
          const int f = pflat[(size_t)slot * k + acc_j];
          if (f > 0 && f < N && npath < D) {
            path[npath++] = f;
            cur_u = f;
            sh.bc_i[3] = 1;
          } else {
            sh.bc_i[3] = 0;
          }
        }
        __syncthreads();
        if (!sh.bc_i[3]) break;
        continue;
      }
      // all k rejected: draw from the residual at st_s
      const double s_fin = st_s;
      if (stale) reduce_pass(R, s_fin, V, sh);
      const int y = draw_pass(R, s_fin, V, ntried, (double)U[(size_t)u * (k + 1) + k], sh, &ties);
      if (tid == 0) comm[ncomm++] = y;
      break;
    }
  }
  __syncthreads();
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

}  // namespace

hipError_t launch_accept(int B, int N, int V, int D, int k, float T, const int32_t* node_tok,
                         const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                         const int32_t* pool_flat, const float* tlog, const float* tstats, const int32_t* targmax,
                         const float* dlog, const float* sstats, const float* uniforms, int32_t* accept_len,
                         int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
                         int32_t* status, hipStream_t st) {
  accept_kernel<<<B, kThreads, 0, st>>>(N, V, D, k, T, node_tok, node_parent, node_slot, pool_tok, pool_flat, tlog,
                                       tstats, targmax, dlog, sstats, uniforms, accept_len, accept_path, committed,
                                       n_committed, near_tie, status);
  return hipGetLastError();
}

}  // namespace eagle
