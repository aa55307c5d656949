// LM-head logits at every tree node and the statistics of their softmax.
//
// Method: EAGLE-1 notes ("EAGLE: Speculative Sampling Requires Rethinking
// Feature Uncertainty"), background section A3: the LM head maps the feature
// of position j to the next-token distribution p_{j+1}; temperature adjusts the
// distribution before the acceptance test (hubwiz "LLM 推测性解码原理解读",
// section 2).
//
// bf16 kernel (lmhead_bf16): logits = X W^T on MFMA (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation).  One workgroup = 64 rows x 512 vocab columns, 8 waves:
// four column quarters of 128 columns times two halves of the hidden
// dimension.  For the skinny shapes of a verify round (one or a few 64-row
// tiles) the kernel streams W exactly once from HBM: each lane loads its
// B-operand fragments straight from global memory into registers, one 64-wide
// hidden chunk ahead of the MFMAs, and reads the small X tile through L2/L1.
// The two hidden halves are summed through LDS; the epilogue writes the fp32
// logits and a per-(row, tile) record (max z/T', sum exp, max z, argmax); a
// second small launch (one workgroup per row) merges the records into the row
// statistics and the argmax.  fp32 kernel (lmhead_f32): one thread per two
// vocab columns, same records.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kKC = 64;              // hidden values per pipeline chunk (two MFMA k-steps)
constexpr float kLog2e = 1.44269504088896341f;
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

// Reductions over the 16 lanes of a DPP row (the lanes sharing one output row
// of an MFMA tile) with DPP moves instead of LDS-routed shuffles: swap within
// pairs, within quads, mirror within halves, mirror within the row.  Every
// step pairs each lane with a distinct partner of the other half of its
// current group, so all 16 lanes end with the same result.
template <int CTRL>
EDEV int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
EDEV float dpp_f(float v) { return __int_as_float(dpp_i<CTRL>(__float_as_int(v))); }
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
EDEV void argmax_step(float& z, int& a) {
  const float z2 = dpp_f<CTRL>(z);
  const int a2 = dpp_i<CTRL>(a);
  if (beats(z2, a2, z, a)) { z = z2; a = a2; }
}
EDEV void row16_argmax(float& z, int& a) {
  argmax_step<kDppXor1>(z, a);
  argmax_step<kDppXor2>(z, a);
  argmax_step<kDppHalfMirror>(z, a);
  argmax_step<kDppMirror>(z, a);
}
EDEV float row16_sum(float s) {
  s += dpp_f<kDppXor1>(s);
  s += dpp_f<kDppXor2>(s);
  s += dpp_f<kDppHalfMirror>(s);
  s += dpp_f<kDppMirror>(s);
  return s;
}

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

template <bool PACKED>
__global__ __launch_bounds__(kLmThreads) void lmhead_bf16_kernel(int rows, int H, int V, float Tp,
                                                                 const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w,
                                                                 float* __restrict__ logits, float* __restrict__ part,
                                                                 int32_t* status) {
  constexpr int NT = 8;  // 16-column n-tiles per wave: 128 vocab columns
  __shared__ floatx4 xch[4][2][NT][64];  // accumulator exchange between the two hidden halves (64 KB)
  __shared__ Rec wrec[4][kLmTileM];

  const int ntiles = gridDim.x;
  const int nt_idx = blockIdx.x, mt_idx = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 3, kh = wave >> 2;  // column quarter, hidden half
  const int col = lane & 15, grp = lane >> 4;
  const int m0 = mt_idx * kLmTileM;
  const int n0 = nt_idx * kLmTileN + wq * (NT * 16);  // first vocab column of this wave
  const int nch = H / kKC;
  const int c0 = kh * (nch / 2), c1 = kh ? nch : nch / 2;
  const int ngroups = (V + 63) / 64;

  // Operand sources of this lane.  A = X rows m0 + mt*16 + col (clamped), k
  // offset grp*8 within each 32-wide k-step.  B = W: row-major rows
  // n0 + nt*16 + col (clamped), or the packed layout, where each 64-row group
  // is one contiguous stream: chunk c, load j of group g is the 1 KB at
  // ((g*nch + c)*8 + j)*512 elements, lane l reading its 16 bytes at l*8.
  // Packed addresses are a wave-uniform base plus the lane's 16 bytes.
  const uint16_t* wq0 = w + (size_t)min(n0 / 64, ngroups - 1) * nch * 4096;      // this wave's first group
  const uint16_t* wq1 = w + (size_t)min(n0 / 64 + 1, ngroups - 1) * nch * 4096;  // and its second
  size_t wrow[PACKED ? 1 : NT];
#pragma unroll
  for (int t = 0; t < (PACKED ? 1 : NT); ++t) wrow[t] = (size_t)min(n0 + t * 16 + col, V - 1) * H + grp * 8;
  uint32_t xoff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) xoff[t] = (uint32_t)min(m0 + t * 16 + col, rows - 1) * (uint32_t)H + grp * 8;
  floatx4 acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Every wave streams its 128 W rows over one half of the hidden dimension
  // (no LDS, no barrier in the loop) and reads the small X tile through
  // L2/L1, one 64-wide chunk ahead of its MFMAs in two register buffers.
  // Loads are unconditional (chunk indices clamp at the end) so the pipeline
  // counters stay exact.
  u32x4 wa[2 * NT], wb[2 * NT], xa[8], xb[8];
#define LM_LOAD(wbuf, xbuf, c)                                                                                     \
  {                                                                                                               \
    const int k0 = (c) * kKC;                                                                                     \
    _Pragma("unroll") for (int j = 0; j < 2 * NT; ++j) {                                                          \
      const int t = (j >> 3) * 4 + (j & 3), ks = (j >> 2) & 1;                                                    \
      const uint16_t* src = PACKED ? (t < 4 ? wq0 : wq1) + ((size_t)(c) * 8 + ks * 4 + (t & 3)) * 512 + lane * 8  \
                                   : w + wrow[PACKED ? 0 : t] + k0 + ks * 32;                                     \
      wbuf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));                                 \
    }                                                                                                             \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                                 \
      xbuf[j] = *reinterpret_cast<const u32x4*>(x + xoff[j & 3] + k0 + (j >> 2) * 32);                            \
  }
#define LM_COMPUTE(wbuf, xbuf)                                                                    \
  _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                              \
    _Pragma("unroll") for (int mt = 0; mt < 4; ++mt) {                                            \
      B8 a;                                                                                       \
      a.w = xbuf[ks * 4 + mt];                                                                    \
      _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                            \
        B8 bb;                                                                                    \
        bb.w = wbuf[(t >> 2) * 8 + ks * 4 + (t & 3)];                                             \
        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bb.v, acc[mt][t], 0, 0, 0);     \
      }                                                                                           \
    }                                                                                             \
  }
  LM_LOAD(wa, xa, c0)
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    LM_LOAD(wb, xb, c + 1)
    LM_COMPUTE(wa, xa)
    LM_LOAD(wa, xa, min(c + 2, c1 - 1))
    LM_COMPUTE(wb, xb)
  }
  if (c < c1) LM_COMPUTE(wa, xa)  // odd number of chunks in this half
#undef LM_COMPUTE
#undef LM_LOAD

  // Sum the two hidden halves through LDS: rows 0..31 end in the kh = 0
  // waves, rows 32..63 in the kh = 1 waves, which then share the epilogue.
  if (kh == 1) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) xch[wq][mt][t][lane] = acc[mt][t];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[mt][t] += xch[wq][mt][t][lane];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) xch[wq][mt][t][lane] = acc[mt + 2][t];
  }
  __syncthreads();
  if (kh == 1) {  // this wave's rows move to acc[0..1] (constant indices keep acc in registers)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[mt][t] = acc[mt + 2][t] + xch[wq][mt][t][lane];
  }

  // Epilogue: logits + per-row record over this wave's 128 columns, rows
  // kh*32 + [0, 32).
  bool bad = false;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = kh * 32 + mt * 16 + grp * 4 + i;
      const int m = m0 + r;
      float zm = kNegInf;
      int ai = kIdxNone;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = n0 + t * 16 + col;
        float z = acc[mt][t][i];
        if (n < V) {
          if (m < rows) logits[(size_t)m * V + n] = z;
          if (!isfinite(z)) { bad = true; z = kNegInf; }
          if (beats(z, n, zm, ai)) { zm = z; ai = n; }
        }
        acc[mt][t][i] = (n < V) ? z : kNegInf;
      }
      // reduce over the 16 lanes sharing this row (one DPP row)
      row16_argmax(zm, ai);
      const float tmax = zm / Tp;  // division is monotone: max z/T' = fl(max z / T')
      // sum of exp(z/T' - tmax) as exp2(z * (log2e/T') - tmax * log2e): one
      // FMA and the hardware exp2 per logit (exp2(-inf) = 0)
      float s = 0.f;
      if (zm != kNegInf) {
        const float c = kLog2e / Tp, off = tmax * kLog2e;
#pragma unroll
        for (int t = 0; t < NT; ++t) s += __builtin_amdgcn_exp2f(fmaf(acc[mt][t][i], c, -off));
      }
      s = row16_sum(s);
      if (col == 0) wrec[wq][r] = Rec{zm == kNegInf ? kNegInf : tmax, s, zm, ai};
    }
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  __syncthreads();
  const int nrows = min(kLmTileM, rows - m0);
  if (tid < nrows) {
    Rec rc = wrec[0][tid];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) rec_merge(rc, wrec[wv][tid]);
    float* pr = part + ((size_t)(m0 + tid) * ntiles + nt_idx) * 4;
    *reinterpret_cast<float4*>(pr) = make_float4(rc.tmax, rc.s, rc.zmax, __int_as_float(rc.arg));
  }
}

// fp32: block = kLmTileN vocab columns of one row, two per thread.
// Reference-precision path for small fp32 shapes.
__global__ __launch_bounds__(256) void lmhead_f32_kernel(int rows, int H, int V, float Tp, const float* __restrict__ x,
                                                         const float* __restrict__ w, float* __restrict__ logits,
                                                         float* __restrict__ part, int32_t* status) {
  extern __shared__ float xs[];
  const int ntiles = gridDim.x;
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int k = tid; k < H; k += 256) xs[k] = x[(size_t)m * H + k];
  __syncthreads();
  float zc[2];
  float zm = kNegInf;
  int ai = kIdxNone;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = blockIdx.x * kLmTileN + h * 256 + tid;
    float z = kNegInf;
    if (n < V) {
      const float* wr = w + (size_t)n * H;
      float a = 0.f;
      for (int k = 0; k < H; ++k) a = fmaf(xs[k], wr[k], a);
      logits[(size_t)m * V + n] = a;
      z = a;
      if (!isfinite(z)) { set_status(status, EAGLE_STATUS_NONFINITE); z = kNegInf; }
      if (beats(z, n, zm, ai)) { zm = z; ai = n; }
    }
    zc[h] = z;
  }
  wave_argmax(zm, ai);
  const float tmax = zm / Tp;
  float s = 0.f;
  if (zm != kNegInf)
#pragma unroll
    for (int h = 0; h < 2; ++h) s += (zc[h] == kNegInf) ? 0.f : expf(zc[h] / Tp - tmax);
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

// Tiled GEMM for many rows: logits = X W^T with 256 x 256 output tiles per
// workgroup (4 waves, each a 128 x 128 quadrant of 8 x 8 MFMA tiles with fp32
// accumulators).  The hidden dimension goes in steps of 32 through a 4-stage
// LDS ring filled by direct global-to-LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at the destination + 16 l), issued three steps
// ahead.  Every 1 KB LDS block is one MFMA operand in lane order: A block mt =
// X rows 16 mt.. (lane l: row l % 16, hidden 8 (l / 16)..); B block nt = W rows
// 16 nt.. the same way, which in the packed weight layout is one contiguous
// 1 KB load.  Workgroups are mapped so that the row tiles sharing a vocab tile
// run on one XCD (workgroups go round-robin over the 8 XCDs), keeping that W
// tile in the XCD's L2 while all row tiles read it.  The epilogue writes the
// logits and a stats record per (row, 256-column tile), the same record the
// streaming kernel writes per 512 columns.
constexpr int kGK = 32;        // hidden values per step
constexpr int kGStages = 4;    // LDS ring depth (loads run kGStages - 1 steps ahead)
constexpr int kGBlock = 512;   // bf16 elements of one 1 KB operand block
constexpr int kGThreads = 512;     // 8 waves: 4 row quarters x 2 column halves, two per SIMD
constexpr int kGLoadsPerStep = 4;  // direct loads each wave issues per step (32 blocks / 8 waves)

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations (other counters unconstrained): vmcnt bits [3:0] and [15:14].
EDEV constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <bool PACKED>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_gemm_kernel(
    int rows, int H, int V, float Tp, int nm, int nn, int bm, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ w, float* __restrict__ logits, float* __restrict__ part, int32_t* status) {
  // the ring: four separate arrays, so that the waits for the direct loads into
  // one of them need not cover the loads still flying into the others
  __shared__ __attribute__((aligned(1024))) uint16_t ring0[32 * kGBlock];  // A 16 blocks | B 16 blocks
  __shared__ __attribute__((aligned(1024))) uint16_t ring1[32 * kGBlock];
  __shared__ __attribute__((aligned(1024))) uint16_t ring2[32 * kGBlock];
  __shared__ __attribute__((aligned(1024))) uint16_t ring3[32 * kGBlock];
  __shared__ Rec hrec[2][kGemmTile];

  // XCD-aware tile order: workgroup id = xcd + 8 j.  On each XCD, runs of 32
  // consecutive j (about what its 32 CUs hold at once) form a block of bm row
  // tiles x 32/bm vocab tiles, so every X and W slab read into the XCD's L2
  // serves several workgroups; vocab tiles of XCD x are those = x mod 8.
  const int bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
  const int bnb = 32 / bm, jb = j & 31, blk = j >> 5, nmb = (nm + bm - 1) / bm;
  const int mt_idx = (blk % nmb) * bm + jb / bnb;
  const int nt_idx = ((blk / nmb) * bnb + jb % bnb) * 8 + xcd;
  if (mt_idx >= nm || nt_idx >= nn) return;  // padding of the grid to whole blocks
  const int m0 = mt_idx * kGemmTile, n0 = nt_idx * kGemmTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // rows 64 wm.., columns 128 wn..
  const int col = lane & 15, grp = lane >> 4;
  const int nch = H / 64;
  const int nsteps = H / kGK;
  const int ngroups = (V + 63) / 64;

  // Sources of this wave's 4 blocks per step: A blocks mt = 2 wave + q and
  // B blocks nt = 2 wave + q (q < 2).
  uint32_t xoff[2];  // element offset of this lane's X row (clamped) + its 8-wide hidden offset
#pragma unroll
  for (int q = 0; q < 2; ++q)
    xoff[q] = (uint32_t)min(m0 + (2 * wave + q) * 16 + col, rows - 1) * (uint32_t)H + grp * 8;
  const uint16_t* wsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * wave + q;
    if (PACKED) {  // group nt / 4, load (nt % 4) of a 32-wide half chunk
      const int g = min(n0 / 64 + nt / 4, ngroups - 1);
      wsrc[q] = w + ((size_t)g * nch * 8 + (nt & 3)) * 512 + (size_t)lane * 8;
    } else {
      wsrc[q] = w + (size_t)min(n0 + nt * 16 + col, V - 1) * H + grp * 8;
    }
  }
#define G_ISSUE_Q(st, dst, q)                                                                               \
  {                                                                                                         \
    const int k0 = (st) * kGK;                                                                              \
    __builtin_amdgcn_global_load_lds(x + xoff[q] + k0, dst + (2 * wave + (q)) * kGBlock, 16, 0, 0);        \
    const uint16_t* ws_ = PACKED ? wsrc[q] + ((size_t)((st) >> 1) * 8 + ((st) & 1) * 4) * 512              \
                                 : wsrc[q] + k0;                                                            \
    __builtin_amdgcn_global_load_lds(ws_, dst + (16 + 2 * wave + (q)) * kGBlock, 16, 0, 0);                 \
  }
#define G_ISSUE(st, dst)                                                                                    \
  {                                                                                                         \
    _Pragma("unroll") for (int q = 0; q < 2; ++q) G_ISSUE_Q(st, dst, q)                                     \
  }

  floatx4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One step: wait for this wave's loads of step st (later steps may still
  // fly), barrier (every wave's blocks are in; the buffer of step st - 1 is
  // free), issue step st + 3 into that buffer, then the 64 MFMAs.
#define G_STEP(st, cur, nxt)                                                                               \
  {                                                                                                        \
    const int ahead = min(kGStages - 2, nsteps - 1 - (st));                                                \
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kGLoadsPerStep));                            \
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGLoadsPerStep));                           \
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                                                         \
    /* a bare barrier: the waits above already cover this wave's loads, and a */                          \
    /* fenced barrier would also wait for the steps still in flight */                                     \
    asm volatile("" ::: "memory");                                                                         \
    __builtin_amdgcn_s_barrier();                                                                          \
    asm volatile("" ::: "memory");                                                                         \
    /* all 16 operand reads first: the MFMAs start as the first ones land; */                             \
    /* the direct loads of step st + 3 go out between the first MFMAs */                                   \
    B8 bf[8], af[4];                                                                                       \
    _Pragma("unroll") for (int t = 0; t < 8; ++t)                                                          \
      bf[t].w = *reinterpret_cast<const u32x4*>(cur + (16 + wn * 8 + t) * kGBlock + lane * 8);            \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                                          \
      af[t].w = *reinterpret_cast<const u32x4*>(cur + (wm * 4 + t) * kGBlock + lane * 8);                 \
    _Pragma("unroll") for (int mt = 0; mt < 4; ++mt) {                                                     \
      _Pragma("unroll") for (int nt = 0; nt < 8; ++nt)                                                     \
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt].v, bf[nt].v, acc[mt][nt], 0, 0, 0);   \
      if (mt == 0 && (st) + kGStages - 1 < nsteps) G_ISSUE((st) + kGStages - 1, nxt)                       \
    }                                                                                                      \
  }
  // nsteps = H / 32 is a multiple of 4 (hidden % 128 == 0)
  G_ISSUE(0, ring0)
  G_ISSUE(1, ring1)
  G_ISSUE(2, ring2)
  for (int st = 0; st < nsteps; st += 4) {
    G_STEP(st, ring0, ring3)
    G_STEP(st + 1, ring1, ring0)
    G_STEP(st + 2, ring2, ring1)
    G_STEP(st + 3, ring3, ring2)
  }
#undef G_STEP
#undef G_ISSUE
#undef G_ISSUE_Q

  // Epilogue: logits and the stats of each row over this wave's 128 columns,
  // then the two column halves of the tile merged through LDS.  One row at a
  // time: its 8 values per lane are copied out of the accumulators.
  bool bad = false;
  const int nbase = n0 + wn * 128;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + mt * 16 + grp * 4 + i;
      const int m = m0 + r;
      float zv[8];
      float zm = kNegInf;
      int ai = kIdxNone;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int n = nbase + nt * 16 + col;
        float z = acc[mt][nt][i];
        if (n < V) {
          if (m < rows) logits[(size_t)m * V + n] = z;
          if (!isfinite(z)) { bad = true; z = kNegInf; }
          if (z > zm) { zm = z; ai = n; }  // columns ascend with nt: ties keep the lower id
        } else {
          z = kNegInf;
        }
        zv[nt] = z;
      }
      row16_argmax(zm, ai);
      const float tmax = zm / Tp;
      float s = 0.f;
      if (zm != kNegInf) {
        const float cc = kLog2e / Tp, off = tmax * kLog2e;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) s += __builtin_amdgcn_exp2f(fmaf(zv[nt], cc, -off));
      }
      s = row16_sum(s);
      if (col == 0) hrec[wn][r] = Rec{zm == kNegInf ? kNegInf : tmax, s, zm, ai};
    }
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  __syncthreads();
  const int m = m0 + tid;
  if (tid < kGemmTile && m < rows) {
    Rec rc = hrec[0][tid];
    rec_merge(rc, hrec[1][tid]);
    float* pr = part + ((size_t)m * nn + nt_idx) * 4;
    *reinterpret_cast<float4*>(pr) = make_float4(rc.tmax, rc.s, rc.zmax, __int_as_float(rc.arg));
  }
}

// One workgroup per row: merge the row's per-tile records (fp64 sum).
__global__ __launch_bounds__(256) void lm_finalize_kernel(int rows, int ntiles, const float* __restrict__ part,
                                                          float* __restrict__ row_stats, int32_t* __restrict__ row_argmax) {
  __shared__ float shf[4];
  __shared__ double shd[4];
  __shared__ int shi[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pr = part + (size_t)m * ntiles * 4;
  float tm = kNegInf, zm = kNegInf;
  int ai = kIdxNone;
  for (int t = tid; t < ntiles; t += 256) {
    const float4 v = *reinterpret_cast<const float4*>(pr + (size_t)t * 4);
    tm = fmaxf(tm, v.x);
    if (beats(v.z, __float_as_int(v.w), zm, ai)) { zm = v.z; ai = __float_as_int(v.w); }
  }
  tm = wave_max(tm);
  wave_argmax(zm, ai);
  if (lane == 0) { shf[wave] = tm; shd[wave] = (double)zm; shi[wave] = ai; }
  __syncthreads();
  float M = shf[0];
  float bz = (float)shd[0];
  int ba = shi[0];
  for (int w = 1; w < 4; ++w) {
    M = fmaxf(M, shf[w]);
    if (beats((float)shd[w], shi[w], bz, ba)) { bz = (float)shd[w]; ba = shi[w]; }
  }
  __syncthreads();
  double s = 0.0;
  if (M != kNegInf)
    for (int t = tid; t < ntiles; t += 256) {
      const float tt = pr[(size_t)t * 4], ss = pr[(size_t)t * 4 + 1];
      if (tt != kNegInf) s += (double)ss * exp((double)tt - (double)M);
    }
  s = wave_sum_d(s);
  if (lane == 0) shd[wave] = s;
  __syncthreads();
  if (tid == 0) {
    row_stats[(size_t)m * 2] = M;
    row_stats[(size_t)m * 2 + 1] = (float)((shd[0] + shd[1]) + (shd[2] + shd[3]));
    row_argmax[m] = ba == kIdxNone ? 0 : ba;
  }
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

// Row-major W [V, H] -> packed layout (see lmhead_bf16_kernel): one thread per
// 16-byte unit; rows beyond V are zero.
__global__ __launch_bounds__(256) void pack_w_kernel(int V, int H, const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ wp, size_t units) {
  const int nch = H / kKC;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63);
    const size_t q = u >> 6;
    const int j = (int)(q & 7);
    const size_t gc = q >> 3;
    const int c = (int)(gc % nch);
    const size_t g = gc / nch;
    const size_t row = g * 64 + (j & 3) * 16 + (l & 15);
    const int k = c * kKC + (j >> 2) * 32 + (l >> 4) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < (size_t)V) v = *reinterpret_cast<const u32x4*>(w + row * H + k);
    *reinterpret_cast<u32x4*>(wp + u * 8) = v;
  }
}

}  // namespace

size_t lm_packed_bytes(int V, int H) { return (size_t)((V + 63) / 64) * (H / kKC) * 8 * 64 * 16; }

hipError_t launch_pack_lmhead(int V, int H, const void* w, void* wp, hipStream_t st) {
  const size_t units = lm_packed_bytes(V, H) / 16;
  const int grid = (int)((units + 255) / 256 < 16384 ? (units + 255) / 256 : 16384);
  pack_w_kernel<<<grid, 256, 0, st>>>(V, H, (const uint16_t*)w, (uint16_t*)wp, units);
  return hipGetLastError();
}

hipError_t launch_lmhead(int rows, int H, int V, int dtype, int w_layout, const void* x, const void* w, float T,
                         float* logits, float* row_stats, int32_t* row_argmax, float* probs, float* ws_part,
                         int32_t* status, hipStream_t st) {
  const float Tp = (T > 0.f) ? T : 1.0f;
  int ntiles = lm_ntiles(V);
  if (dtype == EAGLE_BF16 && rows >= kGemmMinRows) {
    const int nm = (rows + kGemmTile - 1) / kGemmTile, nn = lm_gemm_ntiles(V);
    ntiles = nn;
    // blocks of bm row tiles x 32/bm vocab tiles per XCD (16 x 2 measured best at 16 row tiles)
    const int bm = nm >= 16 ? 16 : nm >= 8 ? 8 : 4, bn = 32 / bm;
    const int grid = ((nm + bm - 1) / bm * bm) * ((nn + 8 * bn - 1) / (8 * bn) * (8 * bn));
    const size_t lds = 0;
    if (w_layout == EAGLE_W_PACKED)
      lmhead_gemm_kernel<true><<<grid, kGThreads, lds, st>>>(rows, H, V, Tp, nm, nn, bm, (const uint16_t*)x,
                                                       (const uint16_t*)w, logits, ws_part, status);
    else
      lmhead_gemm_kernel<false><<<grid, kGThreads, lds, st>>>(rows, H, V, Tp, nm, nn, bm, (const uint16_t*)x,
                                                        (const uint16_t*)w, logits, ws_part, status);
  } else if (dtype == EAGLE_BF16) {
    dim3 grid(ntiles, lm_mtiles(rows));
    if (w_layout == EAGLE_W_PACKED)
      lmhead_bf16_kernel<true><<<grid, kLmThreads, 0, st>>>(rows, H, V, Tp, (const uint16_t*)x, (const uint16_t*)w, logits,
                                                     ws_part, status);
    else
      lmhead_bf16_kernel<false><<<grid, kLmThreads, 0, st>>>(rows, H, V, Tp, (const uint16_t*)x, (const uint16_t*)w, logits,
                                                      ws_part, status);
  } else {
    dim3 grid(ntiles, rows);
    lmhead_f32_kernel<<<grid, 256, (size_t)H * sizeof(float), st>>>(rows, H, V, Tp, (const float*)x,
                                                                    (const float*)w, logits, ws_part, status);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // A separate launch merges the per-tile records: the kernel boundary makes
  // every workgroup's records visible (an in-kernel agent-scope fence would
  // write back each XCD's whole L2 per workgroup).
  lm_finalize_kernel<<<rows, 256, 0, st>>>(rows, ntiles, ws_part, row_stats, row_argmax);
  e = hipGetLastError();
  if (e != hipSuccess || probs == nullptr) return e;
  const size_t total = (size_t)rows * V;
  const int grid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  probs_kernel<<<grid, 256, 0, st>>>(rows, V, Tp, logits, row_stats, probs);
  return hipGetLastError();
}

}  // namespace eagle
