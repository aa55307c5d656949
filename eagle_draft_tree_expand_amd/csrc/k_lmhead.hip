// LM-head logits at every tree node and the statistics of their softmax.
//
// Method: EAGLE-1 notes ("EAGLE: Speculative Sampling Requires Rethinking
// Feature Uncertainty"), background section A3: the LM head maps the feature
// of position j to the next-token distribution p_{j+1}; temperature adjusts the
// distribution before the acceptance test (hubwiz "LLM 推测性解码原理解读",
// section 2).
//
// bf16 kernel (lmhead_bf16): logits = X W^T on MFMA (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation).  One workgroup = 64 rows x 256 vocab columns; 4 waves,
// each owning 64 columns.  For the skinny shapes of a verify round (one or a
// few 64-row tiles) the kernel streams W exactly once from HBM: each lane loads
// its B-operand fragments (8 consecutive hidden values of one vocab row) straight
// from global memory into registers, one 128-wide hidden chunk ahead of the
// MFMAs, while the small X tile is staged through LDS.  The epilogue writes the
// fp32 logits and a per-(row, tile) record (max z/T', sum exp, max z, argmax);
// the last workgroup of each row block (atomic ticket) merges the records into
// the row statistics, so one launch yields logits + stats + argmax.
// fp32 kernel (lmhead_f32): one thread per vocab column; same records, merged by
// a separate small kernel.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kKC = 128;             // hidden values per pipeline chunk
constexpr int kXPad = kKC + 8;       // LDS row stride of the X chunk (bf16)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

union B8 {
  bf16x8 v;
  uint4 u;
  u32x4 w;
};

// Record per (row, vocab tile): tmax = max z/T', s = sum exp(z/T' - tmax), zmax, argmax.
struct Rec {
  float tmax, s, zmax;
  int arg;
};

EDEV void rec_merge(Rec& a, const Rec& b) {
  if (b.tmax == kNegInf) {
    // nothing to add to the sum; argmax still merges below
  } else if (a.tmax == kNegInf) {
    a.tmax = b.tmax;
    a.s = b.s;
  } else {
    const float m = fmaxf(a.tmax, b.tmax);
    a.s = a.s * expf(a.tmax - m) + b.s * expf(b.tmax - m);
    a.tmax = m;
  }
  if (beats(b.zmax, b.arg, a.zmax, a.arg)) { a.zmax = b.zmax; a.arg = b.arg; }
}

// Merge the records of rows [m0, m0 + nrows) into final stats (fp64 sums).
// Called by a full workgroup; one wave per row at a time.
EDEV void finalize_rows(const float* part, int ntiles, int m0, int nrows, float* row_stats, int32_t* row_argmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int r = wave; r < nrows; r += nw) {
    const int m = m0 + r;
    const float* pr = part + (size_t)m * ntiles * 4;
    float tm = kNegInf, zm = kNegInf;
    int ai = kIdxNone;
    for (int t = lane; t < ntiles; t += 64) {
      tm = fmaxf(tm, pr[t * 4]);
      const float z = pr[t * 4 + 2];
      const int a = __float_as_int(pr[t * 4 + 3]);
      if (beats(z, a, zm, ai)) { zm = z; ai = a; }
    }
    const float M = wave_max(tm);
    wave_argmax(zm, ai);
    double s = 0.0;
    if (M != kNegInf)
      for (int t = lane; t < ntiles; t += 64) {
        const float tt = pr[t * 4], ss = pr[t * 4 + 1];
        if (tt != kNegInf) s += (double)ss * exp((double)tt - (double)M);
      }
    s = wave_sum_d(s);
    if (lane == 0) {
      row_stats[(size_t)m * 2] = M;
      row_stats[(size_t)m * 2 + 1] = (float)s;
      row_argmax[m] = ai == kIdxNone ? 0 : ai;
    }
  }
}

__global__ __launch_bounds__(256) void lmhead_bf16_kernel(int rows, int H, int V, float Tp,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, float* __restrict__ logits,
                                                          float* __restrict__ part, int32_t* __restrict__ tickets,
                                                          float* __restrict__ row_stats,
                                                          int32_t* __restrict__ row_argmax, int32_t* status) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kLmTileM * kXPad];
  __shared__ Rec wrec[4][kLmTileM];
  __shared__ int is_last;

  const int ntiles = gridDim.x;
  const int nt_idx = blockIdx.x, mt_idx = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int m0 = mt_idx * kLmTileM;
  const int n0 = nt_idx * kLmTileN + wave * 64;

  // B-operand source rows of this lane: vocab n0 + nt*16 + col (clamped in range).
  const uint16_t* wrow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    int n = n0 + nt * 16 + col;
    n = n < V ? n : V - 1;
    wrow[nt] = w + (size_t)n * H + grp * 8;
  }
  // X chunk loader: 64 rows x 128 values = 1024 uint4, 4 per thread.
  uint4 xr[4];
  auto load_x = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      const int r = e >> 4, c = (e & 15) * 8;
      int m = m0 + r;
      m = m < rows ? m : rows - 1;
      xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)m * H + k0 + c);
    }
  };
  auto store_x = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      const int r = e >> 4, c = (e & 15) * 8;
      *reinterpret_cast<uint4*>(&Xs[r * kXPad + c]) = xr[i];
    }
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  B8 wcur[kKC / 32][4], wnxt[kKC / 32][4];
#pragma unroll
  for (int ks = 0; ks < kKC / 32; ++ks)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) wcur[ks][nt].w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[nt] + ks * 32));
  load_x(0);
  store_x();
  __syncthreads();

  const int nchunks = H / kKC;
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      const int k1 = (c + 1) * kKC;
#pragma unroll
      for (int ks = 0; ks < kKC / 32; ++ks)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          wnxt[ks][nt].w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[nt] + k1 + ks * 32));
      load_x(k1);
    }
#pragma unroll
    for (int ks = 0; ks < kKC / 32; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        B8 a;
        a.u = *reinterpret_cast<const uint4*>(&Xs[(mt * 16 + col) * kXPad + ks * 32 + grp * 8]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, wcur[ks][nt].v, acc[mt][nt], 0, 0, 0);
      }
    }
    if (more) {
      __syncthreads();
      store_x();
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < kKC / 32; ++ks)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) wcur[ks][nt] = wnxt[ks][nt];
    }
  }

  // Epilogue: logits + per-row record over this wave's 64 columns.
  bool bad = false;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + grp * 4 + i;
      const int m = m0 + r;
      float zm = kNegInf;
      int ai = kIdxNone;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + nt * 16 + col;
        float z = acc[mt][nt][i];
        if (n < V) {
          if (m < rows) logits[(size_t)m * V + n] = z;
          if (!isfinite(z)) { bad = true; z = kNegInf; }
          if (beats(z, n, zm, ai)) { zm = z; ai = n; }
        }
        acc[mt][nt][i] = (n < V) ? z : kNegInf;
      }
      // reduce over the 16 lanes sharing this row (xor 1..8 keeps grp)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float z2 = __shfl_xor(zm, o);
        const int a2 = __shfl_xor(ai, o);
        if (beats(z2, a2, zm, ai)) { zm = z2; ai = a2; }
      }
      const float tmax = zm / Tp;  // division is monotone: max z/T' = fl(max z / T')
      float s = 0.f;
      if (zm != kNegInf) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float z = acc[mt][nt][i];
          s += (z == kNegInf) ? 0.f : expf(z / Tp - tmax);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
      if (col == 0) wrec[wave][r] = Rec{zm == kNegInf ? kNegInf : tmax, s, zm, ai};
    }
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  __syncthreads();
  if (tid < kLmTileM) {
    Rec rc = wrec[0][tid];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) rec_merge(rc, wrec[wv][tid]);
    const int m = m0 + tid;
    if (m < rows) {
      float* pr = part + ((size_t)m * ntiles + nt_idx) * 4;
      *reinterpret_cast<float4*>(pr) = make_float4(rc.tmax, rc.s, rc.zmax, __int_as_float(rc.arg));
    }
  }
  // Last workgroup of this row block merges every tile's record.
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&tickets[mt_idx], 1) == ntiles - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const int nrows = min(kLmTileM, rows - m0);
  finalize_rows(part, ntiles, m0, nrows, row_stats, row_argmax);
  if (tid == 0) atomicExch(&tickets[mt_idx], 0);
}

// fp32: block = 256 vocab columns of one row.  Reference-precision path for
// small fp32 shapes.
__global__ __launch_bounds__(256) void lmhead_f32_kernel(int rows, int H, int V, float Tp, const float* __restrict__ x,
                                                         const float* __restrict__ w, float* __restrict__ logits,
                                                         float* __restrict__ part, int32_t* status) {
  extern __shared__ float xs[];
  const int ntiles = gridDim.x;
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int k = tid; k < H; k += 256) xs[k] = x[(size_t)m * H + k];
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  float z = kNegInf;
  if (n < V) {
    const float* wr = w + (size_t)n * H;
    float a = 0.f;
    for (int k = 0; k < H; ++k) a = fmaf(xs[k], wr[k], a);
    logits[(size_t)m * V + n] = a;
    z = a;
    if (!isfinite(z)) { set_status(status, EAGLE_STATUS_NONFINITE); z = kNegInf; }
  }
  float zm = z;
  int ai = n < V ? n : kIdxNone;
  wave_argmax(zm, ai);
  const float tmax = zm / Tp;
  float s = (z == kNegInf || zm == kNegInf) ? 0.f : expf(z / Tp - tmax);
  s = wave_sum(s);
  __shared__ Rec wr4[4];
  if (lane == 0) wr4[wave] = Rec{zm == kNegInf ? kNegInf : tmax, s, zm, ai};
  __syncthreads();
  if (tid == 0) {
    Rec rc = wr4[0];
    for (int wv = 1; wv < 4; ++wv) rec_merge(rc, wr4[wv]);
    float* pr = part + ((size_t)m * ntiles + blockIdx.x) * 4;
    pr[0] = rc.tmax;
    pr[1] = rc.s;
    pr[2] = rc.zmax;
    pr[3] = __int_as_float(rc.arg);
  }
}

__global__ __launch_bounds__(256) void lm_finalize_kernel(int rows, int ntiles, const float* __restrict__ part,
                                                          float* __restrict__ row_stats, int32_t* __restrict__ row_argmax) {
  const int m0 = blockIdx.x * 4;
  finalize_rows(part, ntiles, m0, min(4, rows - m0), row_stats, row_argmax);
}

__global__ __launch_bounds__(256) void probs_kernel(int rows, int V, float Tp, const float* __restrict__ logits,
                                                    const float* __restrict__ row_stats, float* __restrict__ probs) {
  const size_t total = (size_t)rows * V;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / V);
    const float M = row_stats[(size_t)m * 2], S = row_stats[(size_t)m * 2 + 1];
    const float z = logits[e];
    probs[e] = isfinite(z) ? expf(z / Tp - M) / S : 0.f;
  }
}

}  // namespace

hipError_t launch_lmhead(int rows, int H, int V, int dtype, const void* x, const void* w, float T, float* logits,
                         float* row_stats, int32_t* row_argmax, float* probs, float* ws_part, int32_t* tickets,
                         int32_t* status, hipStream_t st) {
  const float Tp = (T > 0.f) ? T : 1.0f;
  const int ntiles = lm_ntiles(V);
  if (dtype == EAGLE_BF16) {
    dim3 grid(ntiles, lm_mtiles(rows));
    lmhead_bf16_kernel<<<grid, 256, 0, st>>>(rows, H, V, Tp, (const uint16_t*)x, (const uint16_t*)w, logits,
                                             ws_part, tickets, row_stats, row_argmax, status);
  } else {
    dim3 grid(ntiles, rows);
    lmhead_f32_kernel<<<grid, 256, (size_t)H * sizeof(float), st>>>(rows, H, V, Tp, (const float*)x,
                                                                    (const float*)w, logits, ws_part, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lm_finalize_kernel<<<(rows + 3) / 4, 256, 0, st>>>(rows, ntiles, ws_part, row_stats, row_argmax);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || probs == nullptr) return e;
  const size_t total = (size_t)rows * V;
  const int grid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  probs_kernel<<<grid, 256, 0, st>>>(rows, V, Tp, logits, row_stats, probs);
  return hipGetLastError();
}

}  // namespace eagle
