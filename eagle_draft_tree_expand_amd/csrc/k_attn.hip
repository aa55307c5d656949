// Tree-masked verify attention: every tree query attends to all prefix keys of
// its request and to the tree keys its ancestor mask allows.
//
// Method: EAGLE-1 notes ("EAGLE: Speculative Sampling Requires Rethinking
// Feature Uncertainty"), sections 3.1 and 3.3 (tree attention: one target
// forward scores the whole draft tree); hubwiz "LLM 推测性解码原理解读",
// section 5 (each root-to-leaf path is scored as an independent sequence).
//
// Work split (flash-decoding style): one workgroup per (request b, kv head g,
// key split).  Splits 0..nsplit-1 cover the prefix in runs of split_keys keys;
// split nsplit covers the n tree keys under the mask.  All n*(hq/hkv) query
// rows of the kv head live in the workgroup, so each K/V byte is read from HBM
// once per split.  Each split writes unnormalised partials (O, running max,
// running sum); attn_merge combines them with log-sum-exp weights.
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16): scores are computed
// transposed, S^T = K Q^T, so the softmax'ed tile is already in the B-operand
// layout of O^T = V^T P^T (no shuffles); K is staged in LDS row-major and V
// transposed.  fp32 path: plain FMA loop (small fp32 shapes).
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKT = 64;            // keys per LDS tile

union B8 {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
};

// Partial record of one query row: O[DH], m, l.
EDEV float* partial_row(float* ws, int b, int g, int hkv, int nsp1, int split, int rows_pad, int r, int DH) {
  return ws + ((((size_t)b * hkv + g) * nsp1 + split) * rows_pad + r) * (DH + 2);
}

// NTH threads (256: 4 waves, 512: 8 waves), each wave kQT 16-row query
// tiles; a (request, kv head, split) with more query rows than one workgroup
// holds is covered by several row blocks, which read the same K/V tiles.
template <int DH, int NTH, int kQT>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(512 / NTH))) void attn_split_bf16_kernel(
    int n, int hq, int hkv, int Lmax, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const int32_t* __restrict__ plen, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vt, const uint64_t* __restrict__ mask, float scale, float* __restrict__ ws,
    int rows, int rows_pad, int split_keys, int nsplit, int nq, int qoff) {
  constexpr int KPAD = DH + 8;    // K row stride in LDS (bf16 elements)
  constexpr int VPAD = kKT + 4;   // V^T row stride in LDS (+4: 2.6x fewer bank-conflict cycles than +8 or +16)
  constexpr float kLog2e = 1.44269504088896341f, kLn2 = 0.693147180559945309f;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKT * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vts[DH * VPAD];

  constexpr int kRows = NTH / 64 * kQT * 16;  // query rows per workgroup
  const int nrb = (rows + kRows - 1) / kRows;
  const int split = blockIdx.x, g = blockIdx.y / nrb, rb = blockIdx.y - g * nrb, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = hq / hkv;
  const int row0 = rb * kRows + wave * (kQT * 16);  // first query row of this wave
  const int W = (n + 63) >> 6;
  const bool tree = split == nsplit;
  const int L = min(max(plen[b], 0), Lmax);  // prefix lengths beyond the buffer are clamped
  int k_begin, k_end;
  if (tree) { k_begin = 0; k_end = n; }
  else { k_begin = split * split_keys; k_end = min(L, k_begin + split_keys); }
  const float sl2 = scale * kLog2e;  // scores are kept in the log2 domain

  const uint16_t* kbase = tree ? kt + ((size_t)b * n * hkv + g) * DH : kp + (((size_t)b * hkv + g) * Lmax) * DH;
  const uint16_t* vbase = tree ? vt + ((size_t)b * n * hkv + g) * DH : vp + (((size_t)b * hkv + g) * Lmax) * DH;
  const size_t kstride = tree ? (size_t)hkv * DH : (size_t)DH;
  const bool wave_active = row0 < rows;

  // K/V tiles of 64 keys: this thread's share of the next tile is loaded
  // into registers while the current tile is in use, then written to LDS
  // (K row-major, V transposed) between two barriers.  A thread owns two
  // consecutive keys of one 8-wide d chunk, so its V^T writes are 4-byte
  // (key pair) words and the 32 threads of a chunk fill 128 contiguous bytes
  // of each V^T row (no bank conflicts).
  constexpr int kPairs = (kKT / 2) * (DH / 8);                          // key-pair chunks per tile
  constexpr int kChunks = (kPairs + NTH - 1) / NTH;  // per thread
  // Two tiles in flight: register sets A and B alternate tile by tile.
  uint4 kregA[2 * kChunks], vregA[2 * kChunks], kregB[2 * kChunks], vregB[2 * kChunks];
  // K/V loads go through buffer resources whose range ends at the split's
  // last key: keys past it read as zero, so every tile issues the same loads
  // with no branches and the counter waits stay exact.
  const int kbytes = k_end > k_begin ? (int)(((size_t)(k_end - 1) * kstride + DH) * 2) : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, kbytes, 0x00020000);
#define ATTN_LOAD_TILE(T0, kreg, vreg)                                                         \
  _Pragma("unroll") for (int i = 0; i < kChunks; ++i) {                                        \
    const int x = tid + i * NTH, kp = x & 31, dc = (x >> 5) * 8;                      \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                            \
      const uint32_t off = (uint32_t)(((size_t)((T0) + 2 * kp + h) * kstride + dc) * 2);       \
      if (kPairs % NTH == 0 || x < kPairs) {                                          \
        const auto kv = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);                 \
        const auto vv = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);                 \
        kreg[2 * i + h] = make_uint4(kv[0], kv[1], kv[2], kv[3]);                              \
        vreg[2 * i + h] = make_uint4(vv[0], vv[1], vv[2], vv[3]);                              \
      }                                                                                        \
    }                                                                                          \
  }
  // the first two K/V tiles in flight while Q loads
  if (k_begin < k_end) {
    ATTN_LOAD_TILE(k_begin, kregA, vregA)
    ATTN_LOAD_TILE(k_begin + kKT, kregB, vregB)
  }

  // Query tiles of this wave.
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 qreg[kQT][DH / 32];
  const uint64_t* mrow[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    const int r = row0 + t * 16 + col;
    const bool ok = r < rows;
    const int node = ok ? r / G : 0, h = g * G + (ok ? r % G : 0);
    const uint16_t* qp = q + (((size_t)b * nq + node) * hq + h) * DH;
#pragma unroll
    for (int ds = 0; ds < DH / 32; ++ds) {
      B8 x;
      x.u = ok ? *reinterpret_cast<const uint4*>(qp + ds * 32 + grp * 8) : make_uint4(0, 0, 0, 0);
      qreg[t][ds] = x.v;
    }
    mrow[t] = mask + ((size_t)b * n + qoff + node) * W;
  }

  floatx4 o[kQT][DH / 16];
  float mrun[kQT], lrun[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    mrun[t] = kNegInf;
    lrun[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) o[t][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile: its registers go to LDS between two barriers, the tile two
  // ahead is loaded into the freed registers, then the wave's MFMAs.
  auto stage_tile = [&](uint4* kreg, uint4* vreg) __attribute__((always_inline)) {
    lds_barrier();  // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int x = tid + i * NTH, kp = x & 31, dc = (x >> 5) * 8;
      if (x >= kPairs) break;
      *reinterpret_cast<uint4*>(&Ks[(2 * kp) * KPAD + dc]) = kreg[2 * i];
      *reinterpret_cast<uint4*>(&Ks[(2 * kp + 1) * KPAD + dc]) = kreg[2 * i + 1];
      const uint16_t* v0 = reinterpret_cast<const uint16_t*>(&vreg[2 * i]);
      const uint16_t* v1 = reinterpret_cast<const uint16_t*>(&vreg[2 * i + 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(&Vts[(dc + e) * VPAD + 2 * kp]) = (uint32_t)v0[e] | ((uint32_t)v1[e] << 16);
    }
    lds_barrier();  // the tile is in LDS; the next tile's loads stay in flight
  };
  auto compute_tile = [&](int t0) __attribute__((always_inline)) {
    // Masking is needed only in the tree split and in a ragged last tile.
    const bool masked = tree || t0 + kKT > k_end;
    // S^T tiles of both query tiles: 64 keys x 16 queries each, lane holds
    // keys 16*kt4 + 4*grp + i of query col.  Each K fragment read from LDS
    // feeds the MFMAs of both query tiles.
    floatx4 sc[kQT][4];
#pragma unroll
    for (int t = 0; t < kQT; ++t)
#pragma unroll
      for (int kt4 = 0; kt4 < 4; ++kt4) sc[t][kt4] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt4 = 0; kt4 < 4; ++kt4) {
#pragma unroll
      for (int ds = 0; ds < DH / 32; ++ds) {
        B8 a;
        a.u = *reinterpret_cast<const uint4*>(&Ks[(kt4 * 16 + col) * KPAD + ds * 32 + grp * 8]);
#pragma unroll
        for (int t = 0; t < kQT; ++t)
          sc[t][kt4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, qreg[t][ds], sc[t][kt4], 0, 0, 0);
      }
    }
    B8 pb[kQT][2];
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      float mx = kNegInf;
      if (masked) {
        // tiles start at multiples of 64 in the tree split; rows >= n read node 0
        const uint64_t mw = tree ? mrow[t][t0 >> 6] : ~0ull;
#pragma unroll
        for (int kt4 = 0; kt4 < 4; ++kt4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + kt4 * 16 + grp * 4 + i;
            const bool vis = key < k_end && ((mw >> (key & 63)) & 1ull);
            const float v = vis ? sc[t][kt4][i] * sl2 : kNegInf;
            sc[t][kt4][i] = v;
            mx = fmaxf(mx, v);
          }
      } else {
#pragma unroll
        for (int kt4 = 0; kt4 < 4; ++kt4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = sc[t][kt4][i] * sl2;
            sc[t][kt4][i] = v;
            mx = fmaxf(mx, v);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[t], mx);
      const float mref = mnew == kNegInf ? 0.f : mnew;  // keeps exp2(-inf - mref) = 0
      const float alpha = __builtin_amdgcn_exp2f(mrun[t] - mref);
      mrun[t] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt4 = 0; kt4 < 4; ++kt4) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(sc[t][kt4][i] - mref);
          psum += p[i];
        }
        const bf16x2 lo2 = {(__bf16)p[0], (__bf16)p[1]}, hi2 = {(__bf16)p[2], (__bf16)p[3]};
        pb[t][kt4 >> 1].h[kt4 & 1] = make_uint2(__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2));
      }
      lrun[t] = lrun[t] * alpha + psum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) o[t][dt] *= alpha;
      }
    }
    // O^T += V^T P^T for both query tiles; each V^T fragment read once.
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int beta = 0; beta < 2; ++beta) {
        B8 a;
        const uint16_t* vr = &Vts[(dt * 16 + col) * VPAD + beta * 32 + grp * 4];
        a.h[0] = *reinterpret_cast<const uint2*>(vr);
        a.h[1] = *reinterpret_cast<const uint2*>(vr + 16);
#pragma unroll
        for (int t = 0; t < kQT; ++t)
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, pb[t][beta].v, o[t][dt], 0, 0, 0);
      }
    }
  };
  for (int t0 = k_begin; t0 < k_end; t0 += 2 * kKT) {
    stage_tile(kregA, vregA);
    ATTN_LOAD_TILE(t0 + 2 * kKT, kregA, vregA)
    if (wave_active) compute_tile(t0);
    if (t0 + kKT < k_end) {
      stage_tile(kregB, vregB);
      ATTN_LOAD_TILE(t0 + 3 * kKT, kregB, vregB)
      if (wave_active) compute_tile(t0 + kKT);
    }
  }
#undef ATTN_LOAD_TILE
  if (!wave_active) return;

  // Write partials (running max back in the natural-log domain): O^T lane
  // holds d = 16*dt + 4*grp + i of query col.
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    float l = lrun[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = row0 + t * 16 + col;
    if (r >= rows) continue;
    float* pr = partial_row(ws, b, g, hkv, nsplit + 1, split, rows_pad, r, DH);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<float4*>(pr + dt * 16 + grp * 4) = make_float4(o[t][dt][0], o[t][dt][1], o[t][dt][2], o[t][dt][3]);
    if (grp == 0) { pr[DH] = mrun[t] == kNegInf ? kNegInf : mrun[t] * kLn2; pr[DH + 1] = l; }
  }
}

// fp32 path: one thread per query row, keys staged in LDS.
template <int DH>
__global__ __launch_bounds__(256) void attn_split_f32_kernel(
    int n, int hq, int hkv, int Lmax, const float* __restrict__ q, const float* __restrict__ kp,
    const float* __restrict__ vp, const int32_t* __restrict__ plen, const float* __restrict__ kt,
    const float* __restrict__ vt, const uint64_t* __restrict__ mask, float scale, float* __restrict__ ws,
    int rows, int rows_pad, int split_keys, int nsplit, int nq, int qoff) {
  constexpr int TK = 32;
  __shared__ float Ks[TK * DH], Vs[TK * DH];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = hq / hkv;
  const int W = (n + 63) >> 6;
  const bool tree = split == nsplit;
  const int L = min(max(plen[b], 0), Lmax);  // prefix lengths beyond the buffer are clamped
  int k_begin, k_end;
  if (tree) { k_begin = 0; k_end = n; }
  else { k_begin = split * split_keys; k_end = min(L, k_begin + split_keys); }
  const float* kbase = tree ? kt + ((size_t)b * n * hkv + g) * DH : kp + (((size_t)b * hkv + g) * Lmax) * DH;
  const float* vbase = tree ? vt + ((size_t)b * n * hkv + g) * DH : vp + (((size_t)b * hkv + g) * Lmax) * DH;
  const size_t kstride = tree ? (size_t)hkv * DH : (size_t)DH;

  for (int r0 = 0; r0 < rows; r0 += blockDim.x) {
    const int r = r0 + tid;
    const bool ok = r < rows;
    const int node = ok ? r / G : 0, h = g * G + (ok ? r % G : 0);
    float qv[DH], ov[DH];
    const float* qp = q + (((size_t)b * nq + node) * hq + h) * DH;
    for (int d = 0; d < DH; ++d) { qv[d] = ok ? qp[d] : 0.f; ov[d] = 0.f; }
    float m = kNegInf, l = 0.f;
    for (int t0 = k_begin; t0 < k_end; t0 += TK) {
      __syncthreads();
      for (int x = tid; x < TK * DH; x += blockDim.x) {
        const int kk = x / DH, d = x - kk * DH;
        const int key = t0 + kk;
        Ks[x] = key < k_end ? kbase[(size_t)key * kstride + d] : 0.f;
        Vs[x] = key < k_end ? vbase[(size_t)key * kstride + d] : 0.f;
      }
      __syncthreads();
      if (!ok) continue;
      for (int kk = 0; kk < TK; ++kk) {
        const int key = t0 + kk;
        if (key >= k_end) break;
        if (tree && !((mask[((size_t)b * n + qoff + node) * W + (key >> 6)] >> (key & 63)) & 1ull)) continue;
        float sc = 0.f;
        for (int d = 0; d < DH; ++d) sc = fmaf(qv[d], Ks[kk * DH + d], sc);
        sc *= scale;
        const float mn = fmaxf(m, sc);
        const float a = (m == kNegInf) ? 0.f : expf(m - mn);
        const float p = expf(sc - mn);
        l = l * a + p;
        for (int d = 0; d < DH; ++d) ov[d] = ov[d] * a + p * Vs[kk * DH + d];
        m = mn;
      }
    }
    if (ok) {
      float* pr = partial_row(ws, b, g, hkv, nsplit + 1, split, rows_pad, r, DH);
      for (int d = 0; d < DH; ++d) pr[d] = ov[d];
      pr[DH] = m;
      pr[DH + 1] = l;
    }
  }
}

// grid (n, hq, B), block DH threads: combine the splits of one (node, head).
// The split maxima and sums are read once in parallel (one thread per
// split); each output element then sums its splits with the resulting
// weights, eight loads in flight at a time.
template <bool BF16>
__global__ __launch_bounds__(128) void attn_merge_kernel(int nq, int hq, int hkv, int DH, const float* __restrict__ ws,
                                                         int rows_pad, int nsplit, void* __restrict__ out) {
  extern __shared__ float wgt[];  // [nsplit + 1] weights exp(m_s - M)
  __shared__ float red[2][2];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = (blockDim.x + 63) >> 6;
  const int G = hq / hkv, g = h / G, r = i * G + (h - g * G);
  const int nsp1 = nsplit + 1;
  const float* p0 = partial_row(const_cast<float*>(ws), b, g, hkv, nsp1, 0, rows_pad, r, DH);
  const size_t sstride = (size_t)rows_pad * (DH + 2);  // floats between splits of one row
  float mloc = kNegInf;
  for (int s = tid; s < nsp1; s += blockDim.x) {
    const float ms = p0[s * sstride + DH];
    wgt[s] = ms;
    mloc = fmaxf(mloc, ms);
  }
  mloc = wave_max(mloc);
  if (lane == 0) red[0][wave] = mloc;
  __syncthreads();
  const float M = nw > 1 ? fmaxf(red[0][0], red[0][1]) : red[0][0];
  float lloc = 0.f;
  for (int s = tid; s < nsp1; s += blockDim.x) {
    const float ms = wgt[s];
    const float w = ms == kNegInf ? 0.f : expf(ms - M);
    wgt[s] = w;
    lloc += p0[s * sstride + DH + 1] * w;
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[1][wave] = lloc;
  __syncthreads();
  const float L = nw > 1 ? red[1][0] + red[1][1] : red[1][0];
  for (int d = tid; d < DH; d += blockDim.x) {
    float acc = 0.f;
    int s = 0;
    for (; s + 8 <= nsp1; s += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p0[(s + j) * sstride + d];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j] * wgt[s + j];
    }
    for (; s < nsp1; ++s) acc += p0[s * sstride + d] * wgt[s];
    const float v = L > 0.f ? acc / L : 0.f;
    const size_t o = (((size_t)b * nq + i) * hq + h) * DH + d;
    if (BF16) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(v);
    else reinterpret_cast<float*>(out)[o] = v;
  }
}

// grid (ceil(rows / 4), hkv, B), 256 threads: four query rows of one
// (request, kv head), one per wave.  Up to 64 splits: lane s holds split s's
// max and sum; each lane then sums its DH / 64 output elements over the
// splits in split order.
template <bool BF16, int DH>
__global__ __launch_bounds__(256) void attn_merge_rows_kernel(int nq, int hq, int hkv, const float* __restrict__ ws,
                                                              int rows, int rows_pad, int nsplit,
                                                              void* __restrict__ out) {
  constexpr int PER = DH / 64;  // output elements per lane
  const int g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = hq / hkv, nsp1 = nsplit + 1;
  const size_t sstride = (size_t)rows_pad * (DH + 2);
  {
    const int r = blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const float* p0 = partial_row(const_cast<float*>(ws), b, g, hkv, nsp1, 0, rows_pad, r, DH);
    const float ms = lane < nsp1 ? p0[lane * sstride + DH] : kNegInf;
    const float ls = lane < nsp1 ? p0[lane * sstride + DH + 1] : 0.f;
    const float M = wave_max(ms);
    const float w = ms == kNegInf ? 0.f : expf(ms - M);
    const float L = wave_sum(ls * w);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < nsp1; s0 += 8) {
      float v[8][PER];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < PER; ++e) v[j][e] = s0 + j < nsp1 ? p0[(s0 + j) * sstride + lane * PER + e] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float wj = __shfl(w, s0 + j < 64 ? s0 + j : 63);
#pragma unroll
        for (int e = 0; e < PER; ++e)
          if (s0 + j < nsp1) acc[e] += v[j][e] * wj;
      }
    }
    const int node = r / G, h = g * G + (r - node * G);
    const size_t o = (((size_t)b * nq + node) * hq + h) * DH + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float val = L > 0.f ? acc[e] / L : 0.f;
      if (BF16) reinterpret_cast<uint16_t*>(out)[o + e] = f32_to_bf16(val);
      else reinterpret_cast<float*>(out)[o + e] = val;
    }
  }
}

}  // namespace

AttnPlan attn_plan(int B, int n, int hq, int hkv, int head_dim, int max_prefix, int dtype) {
  AttnPlan pl;
  pl.rows = n * (hq / hkv);
  pl.rows_pad = (pl.rows + 15) / 16 * 16;
  // Enough splits to give every CU a workgroup (256 CUs), each at least two
  // 64-key tiles so that the register prefetch has something to overlap.
  const int per = B * hkv;
  const int target = (256 + per - 1) / per;
  int sk = (max_prefix + target - 1) / (target > 0 ? target : 1);
  sk = (sk + kKT - 1) / kKT * kKT;
  if (sk < 128) sk = 128;
  // Many (request, kv head) pairs fill the chip by themselves: longer splits
  // then write fewer partial rows for the merge to read back.
  const int cap = per >= 256 ? 2048 : 1024;
  if (sk > cap) sk = cap;
  // Few (request, kv head) pairs and long prefixes: 384-key splits measured
  // best (13B- and 70B-shaped rounds at batch 1: 49 and 38 us against 69 and
  // 48 us with the rule above); shorter splits write more partial rows, longer
  // ones leave CUs idle.
  if (per <= 64 && max_prefix >= 2048) sk = 384;
  pl.split_keys = sk;
  pl.nsplit = (max_prefix + sk - 1) / sk;
  // Row blocks: 64 rows (4 waves x one 16-row tile), 128 (4 x two) or 256
  // (8 x two).  The smallest block whose grid still fits one pass over the
  // 256 CUs wins (batch-1 8B: 64-row blocks, 20 against 25 us for one 256-row
  // block; 70B: 256-row blocks, 32 against 41 us with 64); grids past one pass
  // take the smallest block that holds all rows of a kv head (13B MHA: 64),
  // else 256 (batch 64: 370 against 520 us with 64-row blocks).
  // Many pairs of few rows (batch-64 drafting: 40 rows, 512 pairs, prefixes
  // of 512-4096): 1024-key splits and 128-row blocks, 185 against 205 us
  // with 2048-key splits and 64-row blocks; the partial rows are small.
  if (per >= 256 && pl.rows <= 64) {
    pl.split_keys = 1024;
    pl.nsplit = (max_prefix + 1023) / 1024;
    pl.threads = 256;
    pl.qt = 2;
    return pl;
  }
  const int pairs = B * hkv * (pl.nsplit + 1);
  const int nb64 = (pl.rows + 63) / 64, nb128 = (pl.rows + 127) / 128;
  if (pairs * nb64 <= 256 || pl.rows <= 64) { pl.threads = 256; pl.qt = 1; }
  else if (pairs * nb128 <= 256 || pl.rows <= 128) { pl.threads = 256; pl.qt = 2; }
  else { pl.threads = 512; pl.qt = 2; }
  (void)head_dim;
  (void)dtype;
  return pl;
}

hipError_t launch_attention(int B, int n, int hq, int hkv, int DH, int Lmax, int dtype, const void* q, const void* kp,
                            const void* vp, const int32_t* plen, const void* kt, const void* vt, const uint64_t* mask,
                            float scale, void* out, float* ws, const AttnPlan& pl, int32_t* status, hipStream_t st) {
  return launch_attention_window(B, n, n, 0, hq, hkv, DH, Lmax, dtype, q, kp, vp, plen, kt, vt, mask, scale, out, ws,
                                 pl, status, st);
}

hipError_t launch_attention_window(int B, int n, int nq, int qoff, int hq, int hkv, int DH, int Lmax, int dtype,
                                   const void* q, const void* kp, const void* vp, const int32_t* plen, const void* kt,
                                   const void* vt, const uint64_t* mask, float scale, void* out, float* ws,
                                   const AttnPlan& pl, int32_t* status, hipStream_t st) {
  (void)status;
  if (dtype == EAGLE_BF16) {
    const int threads = pl.threads == 256 ? 256 : 512, qt = pl.qt == 1 ? 1 : 2;
    const int rows_wg = threads / 64 * qt * 16;
    const int nrb = (pl.rows + rows_wg - 1) / rows_wg;
    dim3 grid(pl.nsplit + 1, hkv * nrb, B);
#define EAGLE_ATTN_BF16(D, T, Q)                                                                                     \
  attn_split_bf16_kernel<D, T, Q><<<grid, T, 0, st>>>(n, hq, hkv, Lmax, (const uint16_t*)q, (const uint16_t*)kp,    \
                                                      (const uint16_t*)vp, plen, (const uint16_t*)kt,               \
                                                      (const uint16_t*)vt, mask, scale, ws, pl.rows, pl.rows_pad,   \
                                                      pl.split_keys, pl.nsplit, nq, qoff)
#define EAGLE_ATTN_BF16_T(D)                    \
  if (threads == 256 && qt == 1) EAGLE_ATTN_BF16(D, 256, 1); \
  else if (threads == 256) EAGLE_ATTN_BF16(D, 256, 2);      \
  else if (qt == 1) EAGLE_ATTN_BF16(D, 512, 1);             \
  else EAGLE_ATTN_BF16(D, 512, 2);
    if (DH == 64) {
      EAGLE_ATTN_BF16_T(64)
    } else {
      EAGLE_ATTN_BF16_T(128)
    }
#undef EAGLE_ATTN_BF16_T
#undef EAGLE_ATTN_BF16
  } else {
    dim3 grid(pl.nsplit + 1, hkv, B);
#define EAGLE_ATTN_F32(D)                                                                                          \
  attn_split_f32_kernel<D><<<grid, 256, 0, st>>>(n, hq, hkv, Lmax, (const float*)q, (const float*)kp,             \
                                                 (const float*)vp, plen, (const float*)kt, (const float*)vt, mask, \
                                                 scale, ws, pl.rows, pl.rows_pad, pl.split_keys, pl.nsplit, nq, \
                                                 qoff)
    if (DH <= 16) EAGLE_ATTN_F32(16);
    else if (DH <= 32) EAGLE_ATTN_F32(32);
    else if (DH <= 64) EAGLE_ATTN_F32(64);
    else EAGLE_ATTN_F32(128);
#undef EAGLE_ATTN_F32
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.nsplit + 1 <= 64 && (DH == 64 || DH == 128)) {
    dim3 rg((pl.rows + 3) / 4, hkv, B);
#define EAGLE_MERGE_ROWS(BF, D) \
  attn_merge_rows_kernel<BF, D><<<rg, 256, 0, st>>>(nq, hq, hkv, ws, pl.rows, pl.rows_pad, pl.nsplit, out)
    if (dtype == EAGLE_BF16) {
      if (DH == 64) EAGLE_MERGE_ROWS(true, 64);
      else EAGLE_MERGE_ROWS(true, 128);
    } else {
      if (DH == 64) EAGLE_MERGE_ROWS(false, 64);
      else EAGLE_MERGE_ROWS(false, 128);
    }
#undef EAGLE_MERGE_ROWS
    return hipGetLastError();
  }
  dim3 mg(nq, hq, B);
  const int mt = DH <= 64 ? 64 : 128;  // whole waves (the merge reduces across lanes)
  const size_t lds = (size_t)(pl.nsplit + 1) * sizeof(float);
  if (dtype == EAGLE_BF16) attn_merge_kernel<true><<<mg, mt, lds, st>>>(nq, hq, hkv, DH, ws, pl.rows_pad, pl.nsplit, out);
  else attn_merge_kernel<false><<<mg, mt, lds, st>>>(nq, hq, hkv, DH, ws, pl.rows_pad, pl.nsplit, out);
  return hipGetLastError();
}

}  // namespace eagle
