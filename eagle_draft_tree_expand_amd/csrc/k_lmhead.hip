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
// hidden chunk ahead of the MFMAs; the X fragments of a chunk are loaded once
// per workgroup and shared through LDS.  The two hidden halves are summed
// through LDS; the epilogue writes the fp32 logits and a per-(row, tile)
// record (max z/T', sum exp, max z, tile); a second small launch (one
// workgroup per row) merges the records into the row statistics and finds the
// argmax column.  The tiled GEMM kernel (lmhead_gemm, many rows) and the fp32
// kernel (lmhead_f32, one thread per two vocab columns) write the same records
// with the argmax column itself.

#include <type_traits>

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
// of an MFMA tile) with the DPP moves of common.h.
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

// Row reductions for the streaming kernel's epilogue: max and sum over the 16
// lanes of a DPP row.
EDEV float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

// Decode one z-packed fragment's lane registers to its 8 bf16 (layout in
// eagle.h).  v is the 16-byte load of the lane: a raw fragment's 16 bytes (low
// bytes of weights 0..3, of 4..7, high bytes of 0..3, of 4..7); a coded
// fragment's 12 bytes from the lane's own position (low bytes 0..3, 4..7,
// codes, then 4 bytes of the next lane), except the last lane, which reads
// from 4 bytes before its 12 so that no load leaves the fragment; `last` marks
// that lane, whose words are rotated into place.  A coded weight's high byte
// is base plus the low three bits of its code (no carry out of a byte: base +
// 7 <= 127), plus the code's top bit moved to bit 7; hb = the fragment's
// header byte.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
EDEV u32x4 zdecode(u32x4 v, uint32_t hb, bool last) {
  const bool raw = (hb & 0x80u) != 0;
  if (!raw && last) v = u32x4{v.y, v.z, v.w, v.x};
  const uint32_t b4 = (hb & 0x7fu) * 0x01010101u;
  const uint32_t c = v.z;
  uint32_t ha = (c & 0x07070707u) + ((c << 4) & 0x80808080u) + b4;
  uint32_t hh = ((c >> 4) & 0x07070707u) + (c & 0x80808080u) + b4;
  if (raw) {
    ha = v.z;
    hh = v.w;
  }
  return u32x4{__builtin_amdgcn_perm(ha, v.x, 0x05010400u), __builtin_amdgcn_perm(ha, v.x, 0x07030602u),
               __builtin_amdgcn_perm(hh, v.y, 0x05010400u), __builtin_amdgcn_perm(hh, v.y, 0x07030602u)};
}

// WL: the weight layout (EAGLE_W_ROWMAJOR, EAGLE_W_PACKED or EAGLE_W_ZPACKED).
template <int WL>
__global__ __launch_bounds__(kLmThreads) void lmhead_bf16_kernel(int rows, int H, int V, float Tp,
                                                                 const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w,
                                                                 float* __restrict__ logits, float* __restrict__ part,
                                                                 int32_t* status, int hk, float* __restrict__ partial,
                                                                 RowMap rm, uint16_t* __restrict__ z16,
                                                                 float* __restrict__ bmax) {
  constexpr bool PACKED = WL != EAGLE_W_ROWMAJOR;
  constexpr bool ZP = WL == EAGLE_W_ZPACKED;
  constexpr int NT = 8;  // 16-column n-tiles per wave: 128 vocab columns
  __shared__ floatx4 xch[4][2][NT][64];  // accumulator exchange between the two hidden halves (64 KB)
  extern __shared__ __attribute__((aligned(16))) unsigned char zh_lds[];  // z-packed: [wave][step][16] headers
  __shared__ u32x4 xst[2][2][8][64];     // X staging: [stage][hidden half][fragment ks*4 + mt][lane] (32 KB)
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
  // hidden slice blockIdx.z of hk values (hk = H without a split; a multiple
  // of 128, so both halves have the same number of chunks)
  const int nchs = hk / kKC;
  const int c0 = blockIdx.z * nchs + kh * (nchs / 2);
  const int nsteps = nchs / 2;
  const int ngroups = (V + 63) / 64;

  // Operand sources of this lane.  A = X rows m0 + mt*16 + col (clamped), k
  // offset grp*8 within each 32-wide k-step.  B = W: the packed layout, where
  // each 64-row group is one contiguous stream (chunk c, load j of group g is
  // the 1 KB at ((g*nch + c)*8 + j)*512 elements, lane l reading its 16 bytes
  // at l*8), or row-major rows n0 + t*16 + col (clamped).
  const uint16_t* wq0 = w + (size_t)min(n0 / 64, ngroups - 1) * nch * 4096;      // this wave's first group
  const uint16_t* wq1 = w + (size_t)min(n0 / 64 + 1, ngroups - 1) * nch * 4096;  // and its second
  size_t wrow[PACKED ? 1 : NT];
#pragma unroll
  for (int t = 0; t < (PACKED ? 1 : NT); ++t) wrow[t] = (size_t)min(n0 + t * 16 + col, V - 1) * H + grp * 8;
  floatx4 acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // X goes through LDS: per step, the 8 A fragments (4 row tiles x 2 k-steps)
  // of each hidden half are loaded once per workgroup, two by each of the four
  // waves of that half, instead of by all four waves.  A fragment is stored
  // in lane order (lane l's 16 bytes at l*16), so the reads are conflict-free.
  // Two stages: step s writes stage s&1, which was last read at step s - 2,
  // before every wave passed the barrier of step s - 1.
  const int xj = wq * 2;  // this wave's fragments j = xj, xj + 1 (j = ks*4 + mt)
  uint32_t xo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = xj + u;
    xo[u] = (uint32_t)min(m0 + (j & 3) * 16 + col, rows - 1) * (uint32_t)H + grp * 8 + (j >> 2) * 32;
  }

  // Every wave streams its 128 W rows over one half of the hidden dimension
  // straight into registers.  One buffer of 16 fragments rotates: as soon as
  // a fragment's four MFMAs of step s are issued, the load of the same
  // fragment for step s + 1 goes out into its registers, so each load flies
  // about one step ahead.  The last step issues no loads.
  // z-packed: the wave's two 64-row groups and the header bytes of its
  // fragments, copied to LDS per step (16 bytes: 8 per group); a step's 16
  // become four scalar words (byte j & 3 of word j >> 2 is fragment j's): hc
  // for the step being multiplied, hn for the one being loaded.  Each W load
  // is one 16-byte load per lane whichever the fragment's form (only its base
  // and lane stride differ), so the loop's counter waits are the packed
  // layout's.
  const int zg0 = min(n0 / 64, ngroups - 1), zg1 = min(n0 / 64 + 1, ngroups - 1);
  const unsigned char* zb = reinterpret_cast<const unsigned char*>(w);
  const ZLayout zl = lm_zlayout(V, H);
  uint32_t hc[4] = {0u, 0u, 0u, 0u}, hn[4] = {0u, 0u, 0u, 0u};
  unsigned char* zh = zh_lds + (size_t)wave * nsteps * 16;
  auto zheaders = [&](int step, uint32_t* h) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(zh + step * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_amdgcn_readfirstlane(v[i]);
  };
  auto zbyte = [&](const uint32_t* h, int j) -> uint32_t { return (h[j >> 2] >> (8 * (j & 3))) & 0xffu; };
  // Buffer loads: the fragment's byte offset in a scalar register, the lane's
  // offset (12 or 16 bytes a lane; the last lane of a coded fragment 4 bytes
  // early) in a vector register; the whole z-packed weight is below 4 GB (the
  // host checks).
  const bool zlast = lane == 63;
  const uint32_t zlc = zlast ? 63u * 12u - 4u : (uint32_t)lane * 12u, zlr = (uint32_t)lane * 16u;
  const __amdgpu_buffer_rsrc_t zrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)zb, (short)0, ZP ? (int)(uint32_t)zl.bytes : 0, 0x00020000);
  auto zload = [&](int step, int j, uint32_t hb) -> u32x4 {
    const uint32_t f = ((uint32_t)((j < 8) ? zg0 : zg1) * (uint32_t)nch + (uint32_t)(c0 + step)) * 8u + (uint32_t)(j & 7);
    const bool raw = (hb & 0x80u) != 0;
    const uint32_t so = raw ? (uint32_t)zl.raw_off + f * 1024u : (uint32_t)zl.slot_off + f * 768u;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zrs, (int)(raw ? zlr : zlc), (int)so, 2));
  };
  if (ZP) {
    for (int st = lane; st < nsteps; st += 64) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(zb + ((size_t)zg0 * nch + c0 + st) * 8);
      const u32x2 b = *reinterpret_cast<const u32x2*>(zb + ((size_t)zg1 * nch + c0 + st) * 8);
      *reinterpret_cast<u32x4*>(zh + st * 16) = u32x4{a.x, a.y, b.x, b.y};
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    zheaders(0, hc);
  }

  u32x4 wf[2 * NT], sx[2];
  auto w_src = [&](int step, int j) -> const u32x4* {
    const int c = c0 + step;
    const int t = (j >> 3) * 4 + (j & 3), ks = (j >> 2) & 1;
    const uint16_t* src = PACKED ? (t < 4 ? wq0 : wq1) + ((size_t)c * 8 + ks * 4 + (t & 3)) * 512 + lane * 8
                                 : w + wrow[PACKED ? 0 : t] + c * kKC + ks * 32;
    return reinterpret_cast<const u32x4*>(src);
  };
  auto x_src = [&](int step, int u) -> const u32x4* {
    return reinterpret_cast<const u32x4*>(x + xo[u] + (c0 + step) * kKC);
  };
  // The prologue issues in the loop's order (X, then W; the scheduling
  // barriers keep it), so the counter waits at the loop head, which must hold
  // for the first iteration too, stay as loose as the loop's.
  sx[0] = *x_src(0, 0);
  sx[1] = *x_src(0, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 2 * NT; ++j) wf[j] = ZP ? zload(0, j, zbyte(hc, j)) : __builtin_nontemporal_load(w_src(0, j));
  __builtin_amdgcn_sched_barrier(0);
  // One step: publish this wave's X fragments, barrier, then 64 MFMAs with A
  // read from LDS.  The barrier is bare: a fenced one would also wait for the
  // next step's loads, which must stay in flight.
  auto step_body = [&](int step, bool more) __attribute__((always_inline)) {
    xst[step & 1][kh][xj][lane] = sx[0];
    xst[step & 1][kh][xj + 1][lane] = sx[1];
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (more) {
      sx[0] = *x_src(step + 1, 0);
      sx[1] = *x_src(step + 1, 1);
    }
    if (ZP && more) zheaders(step + 1, hn);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      B8 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt].w = xst[step & 1][kh][ks * 4 + mt][lane];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int j = (t >> 2) * 8 + ks * 4 + (t & 3);
        B8 bb;
        bb.w = ZP ? zdecode(wf[j], zbyte(hc, j), zlast) : wf[j];
        // z-packed: the decode has consumed the fragment's registers, so its next
        // load can go out before the MFMAs
        if (ZP && more) wf[j] = zload(step + 1, j, zbyte(hn, j));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt].v, bb.v, acc[mt][t], 0, 0, 0);
        if (!ZP && more) wf[j] = __builtin_nontemporal_load(w_src(step + 1, j));
      }
    }
    if (ZP && more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hc[i] = hn[i];
    }
  };
  for (int st = 0; st + 1 < nsteps; ++st) step_body(st, true);
  step_body(nsteps - 1, false);

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

  // A slice of a split hidden dimension: its partial logits, summed and
  // turned into records by the combine launch.
  if (partial != nullptr) {
    float* pz = partial + (size_t)blockIdx.z * rows * V;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + kh * 32 + mt * 16 + grp * 4 + i;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = n0 + t * 16 + col;
          if (m < rows && n < V) pz[(size_t)m * V + n] = acc[mt][t][i];
        }
      }
    return;
  }

  // Epilogue: logits and one record per row over this wave's 128 columns,
  // rows kh*32 + mt*16 + grp*4 + i.  Non-finite logits are caught by one FMA
  // per value (z*0 is NaN exactly for inf and NaN); a wave that has any, or
  // that crosses the vocabulary end, masks them to -inf before the statistics.
  const bool full = n0 + NT * 16 <= V;
  float chk = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + kh * 32 + mt * 16 + grp * 4 + i;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = n0 + t * 16 + col;
        const float z = acc[mt][t][i];
        if (full || n < V) {
          if (m < rows && z16 == nullptr) logits[(size_t)map_row(m, rm) * V + n] = z;
          chk = fmaf(z, 0.f, chk);
        }
      }
    }
  }
  const bool bad = __ballot(chk != chk) != 0;
  if (bad || !full) {
    if (bad && lane == 0) set_status(status, EAGLE_STATUS_NONFINITE);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = acc[mt][t][i];
          acc[mt][t][i] = (n0 + t * 16 + col < V && isfinite(z)) ? z : kNegInf;
        }
  }
  // Per row: max (the record's zmax; max z/T' = fl(max z / T') since division
  // by T' > 0 is monotone), then the sum of exp(z/T' - tmax) as
  // exp2(z * (log2e/T') - tmax * log2e): one FMA and the hardware exp2 per
  // value (exp2(-inf) = 0).  The record's arg names the tile, not the column:
  // the row merge scans the winning tile for the first column holding the max.
  const float cT = kLog2e / Tp;
  if (z16 != nullptr) {
    // Compact rows: this wave's 128 columns are one block.  Per row: the
    // block maximum and the first column holding it (exact, ties to the lower
    // id), the fp16 offsets, and the statistics of the decoded values.
    const int nblk = (V + 127) >> 7, blk = n0 >> 7;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + kh * 32 + mt * 16 + grp * 4 + i;
        float zm = kNegInf;
        int ai = kIdxNone;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (acc[mt][t][i] > zm) { zm = acc[mt][t][i]; ai = n0 + t * 16 + col; }  // columns ascend with t
        row16_argmax(zm, ai);
        const float tmax = zm / Tp;
        const size_t ro = (size_t)map_row(min(m, rows - 1), rm);
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = n0 + t * 16 + col;
          const uint16_t h = cmp_encode(acc[mt][t][i], zm);
          if (m < rows && (full || n < V)) z16[ro * V + n] = h;
          if (zm != kNegInf) sum += __builtin_amdgcn_exp2f(fmaf(cmp_decode(h, zm), cT, -tmax * kLog2e));
        }
        sum = row16_sum(sum);
        if (col == 0) {
          wrec[wq][kh * 32 + mt * 16 + grp * 4 + i] = Rec{zm == kNegInf ? kNegInf : tmax, sum, zm, ai};
          if (m < rows && n0 < V) bmax[ro * nblk + blk] = zm;  // a wave past the vocabulary has no block
        }
      }
    }
  } else {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float zm = acc[mt][0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) zm = fmaxf(zm, acc[mt][t][i]);
      zm = row16_max(zm);
      const float tmax = zm / Tp;
      float sum = 0.f;
      if (zm != kNegInf) {
        const float off = tmax * kLog2e;
#pragma unroll
        for (int t = 0; t < NT; ++t) sum += __builtin_amdgcn_exp2f(fmaf(acc[mt][t][i], cT, -off));
      }
      sum = row16_sum(sum);
      if (col == 0)
        wrec[wq][kh * 32 + mt * 16 + grp * 4 + i] =
            Rec{zm == kNegInf ? kNegInf : tmax, sum, zm, kLmArgTile | (nt_idx * kLmTileN)};
    }
  }
  }
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
                                                         float* __restrict__ part, int32_t* status, RowMap rm) {
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
      logits[(size_t)map_row(m, rm) * V + n] = a;
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
// workgroup (8 waves, two per SIMD, each a 64 x 128 block of 4 x 8 MFMA tiles
// with fp32 accumulators).  The hidden dimension goes in steps of 32 through a 4-stage
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
constexpr int kGBlock = 512;   // bf16 elements of one 1 KB operand block
// Output tiles of TM x 256: 256 x 256 (4 row groups x 2 column groups of
// waves, 8 waves, one workgroup per CU, 4-stage ring) or 128 x 256 (2 x 2, 4
// waves, two workgroups per CU, 3-stage ring of 72 KB); every wave holds a
// 64 x 128 block of 4 x 8 MFMA tiles.  256 x 256 is faster where both fit the
// rows (41.7% against 39% of the bf16 peak at 3904 rows); 128 x 256 serves row
// counts that 256-row tiles would pad by a sixth or more (640 rows: 768
// computed).  A 128 x 512 tile with 8 waves (the 256 x 256 tile's MFMA work,
// no padding at multiples of 128) ran slower than both: 25% more ring bytes
// per step in a 3-stage ring.

// Direct global->LDS load of 16 bytes per lane into lds + 16 * lane, issued
// by hand: the compiler then does not track these LDS writes, and does not
// drain every load still in flight (a vmcnt(0)) before each read of a ring
// stage it cannot tell apart from the stages being filled.  The kernel's own
// vmcnt waits and barriers order them: a stage is read only after every wave
// has waited for its loads into it.  M0 holds the LDS address; one wait state
// separates its write from the load that reads it.
EDEV void dma16_lds(const void* g, const void* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations (other counters unconstrained): vmcnt bits [3:0] and [15:14].
EDEV constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `ahead` steps of L loads each are still in flight
// (ahead <= A; the immediate must be a constant, hence the chain).
template <int L, int A>
EDEV void wait_steps_ahead(int ahead) {
  if constexpr (A == 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (ahead >= A) __builtin_amdgcn_s_waitcnt(vmcnt_imm(A * L));
    else wait_steps_ahead<L, A - 1>(ahead);
  }
}

template <bool PACKED, int TM, int STAGES>
__global__ __launch_bounds__(TM * 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_gemm_kernel(
    int rows, int H, int V, float Tp, int nm, int nn, int bm, int bn, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ w, float* __restrict__ logits, float* __restrict__ part, int32_t* status,
    RowMap rm, int gps, int ks, float* __restrict__ partial, uint16_t* __restrict__ z16, float* __restrict__ bmax) {
  constexpr int TN = kGemmTile, WN = 2;  // two column groups of 128
  constexpr int WAVES = (TM / 64) * WN;
  constexpr int AB = TM / 16, BB = TN / 16;  // A and B blocks per stage
  constexpr int QA = AB / WAVES;         // A blocks each wave loads per step
  constexpr int QB = BB / WAVES;         // B blocks each wave loads per step
  constexpr int kLoads = QA + QB;        // direct loads each wave issues per step
  static_assert(QA >= 1 && QB >= 1 && QA * WAVES == AB && QB * WAVES == BB, "blocks must split evenly over waves");
  // the ring: STAGES stages of A blocks | B blocks
  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][(AB + BB) * kGBlock];
  __shared__ Rec hrec[WN][TM];

  // XCD-aware tile order: workgroup id = xcd + 8 j.  On each XCD, runs of
  // bm x bn consecutive j (at most 32: about what its 32 CUs hold at once)
  // form a block of bm row tiles x bn vocab tiles, so every X and W slab read
  // into the XCD's L2 serves several workgroups; vocab tiles of XCD x are
  // those = x mod 8.  The grid holds whole blocks: bm and bn follow the tile
  // counts so that few of its workgroups are empty.
  // hidden split: workgroups kz*gps .. kz*gps + gps-1 cover hidden slice kz
  // of every tile (128-wide chunks kz C / ks .. (kz + 1) C / ks - 1 of the C =
  // H / 128) and write fp32 partials (partial != null)
  const int kz = (int)blockIdx.x / gps;
  const int bid = (int)blockIdx.x - kz * gps, xcd = bid & 7, j = bid >> 3;
  const int bsz = bm * bn, blk = j / bsz, jb = j - blk * bsz, nmb = (nm + bm - 1) / bm;
  const int mt_idx = (blk % nmb) * bm + jb / bn;
  const int nt_idx = ((blk / nmb) * bn + jb % bn) * 8 + xcd;
  if (mt_idx >= nm || nt_idx >= nn) return;  // padding of the grid to whole blocks
  const int m0 = mt_idx * TM, n0 = nt_idx * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;  // rows 64 wm.., columns 128 wn..
  const int col = lane & 15, grp = lane >> 4;
  const int nch = H / 64;
  const int nch128 = H / 128, c0 = kz * nch128 / ks, c1 = (kz + 1) * nch128 / ks;
  const int nsteps = (c1 - c0) * (128 / kGK);  // a multiple of 4
  const int sb = c0 * (128 / kGK);             // first step of this slice
  const int ngroups = (V + 63) / 64;

  // Sources of this wave's blocks per step: A blocks mt = QA wave + q (q <
  // QA) and B blocks nt = QB wave + q (q < QB).
  uint32_t xoff[QA];  // element offset of this lane's X row (clamped) + its 8-wide hidden offset
#pragma unroll
  for (int q = 0; q < QA; ++q)
    xoff[q] = (uint32_t)min(m0 + (QA * wave + q) * 16 + col, rows - 1) * (uint32_t)H + grp * 8 + sb * kGK;
  const uint16_t* wsrc[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int nt = QB * wave + q;
    if (PACKED) {  // group nt / 4, load (nt % 4) of a 32-wide half chunk
      const int g = min(n0 / 64 + nt / 4, ngroups - 1);
      wsrc[q] = w + ((size_t)g * nch * 8 + (nt & 3) + (size_t)(sb >> 1) * 8) * 512 + (size_t)lane * 8;
    } else {
      wsrc[q] = w + (size_t)min(n0 + nt * 16 + col, V - 1) * H + grp * 8 + sb * kGK;
    }
  }
#define G_ISSUE(st, dst)                                                                                    \
  {                                                                                                         \
    const int k0 = (st) * kGK;                                                                              \
    _Pragma("unroll") for (int q = 0; q < QA; ++q)                                                          \
      dma16_lds(x + xoff[q] + k0, dst + (QA * wave + q) * kGBlock);                                         \
    _Pragma("unroll") for (int q = 0; q < QB; ++q) {                                                        \
      const uint16_t* ws_ = PACKED ? wsrc[q] + ((size_t)((st) >> 1) * 8 + ((st) & 1) * 4) * 512            \
                                   : wsrc[q] + k0;                                                          \
      dma16_lds(ws_, dst + (AB + QB * wave + q) * kGBlock);                                                 \
    }                                                                                                       \
  }

  floatx4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One step: wait for this wave's loads of step st (later steps may still
  // fly), barrier (every wave's blocks are in; the buffer of step st - 1 is
  // free), issue step st + STAGES - 1 into that buffer, then the 32 MFMAs.
#define G_STEP(st, cur, nxt)                                                                               \
  {                                                                                                        \
    wait_steps_ahead<kLoads, STAGES - 2>(min(STAGES - 2, nsteps - 1 - (st)));                              \
    /* a bare barrier: the waits above already cover this wave's loads, and a */                          \
    /* fenced barrier would also wait for the steps still in flight */                                     \
    asm volatile("" ::: "memory");                                                                         \
    __builtin_amdgcn_s_barrier();                                                                          \
    asm volatile("" ::: "memory");                                                                         \
    /* all 16 operand reads first: the MFMAs start as the first ones land; */                             \
    /* the direct loads of step st + 3 go out between the first MFMAs */                                   \
    B8 bf[8], af[4];                                                                                       \
    _Pragma("unroll") for (int t = 0; t < 8; ++t)                                                          \
      bf[t].w = *reinterpret_cast<const u32x4*>(cur + (AB + wn * 8 + t) * kGBlock + lane * 8);            \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                                          \
      af[t].w = *reinterpret_cast<const u32x4*>(cur + (wm * 4 + t) * kGBlock + lane * 8);                 \
    _Pragma("unroll") for (int mt = 0; mt < 4; ++mt) {                                                     \
      _Pragma("unroll") for (int nt = 0; nt < 8; ++nt)                                                     \
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt].v, bf[nt].v, acc[mt][nt], 0, 0, 0);   \
      if (mt == 0 && (st) + STAGES - 1 < nsteps) G_ISSUE((st) + STAGES - 1, nxt)                           \
    }                                                                                                      \
  }
  // nsteps = H / 32 is a multiple of 4 (hidden % 128 == 0)
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nsteps) G_ISSUE(st, ring[st])
  if (STAGES == 4) {
    for (int st = 0; st < nsteps; st += 4) {
      G_STEP(st, ring[0], ring[3])
      G_STEP(st + 1, ring[1], ring[0])
      G_STEP(st + 2, ring[2], ring[1])
      G_STEP(st + 3, ring[3], ring[2])
    }
  } else {
    for (int st = 0; st < nsteps; ++st) {
      const int sc = st % STAGES;
      G_STEP(st, ring[sc], ring[(sc + STAGES - 1) % STAGES])
    }
  }
#undef G_STEP
#undef G_ISSUE

  const int nbase = n0 + wn * 128;
  if (partial != nullptr) {  // a hidden slice: fp32 partials, summed by lm_combine
    float* pz = partial + (size_t)kz * rows * V;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + mt * 16 + grp * 4 + i;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int n = nbase + nt * 16 + col;
          if (m < rows && n < V) pz[(size_t)m * V + n] = acc[mt][nt][i];
        }
      }
    return;
  }

  // Epilogue: logits and the stats of each row over this wave's 128 columns,
  // then the two column halves of the tile merged through LDS.  One row at a
  // time: its 8 values per lane are copied out of the accumulators.
  bool bad = false;
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
          if (m < rows && z16 == nullptr) logits[(size_t)map_row(m, rm) * V + n] = z;
          if (!isfinite(z)) { bad = true; z = kNegInf; }
          if (z > zm) { zm = z; ai = n; }  // columns ascend with nt: ties keep the lower id
        } else {
          z = kNegInf;
        }
        zv[nt] = z;
      }
      row16_argmax(zm, ai);
      const float tmax = zm / Tp;
      if (z16 != nullptr) {
        // compact rows: this wave's 128 columns are one block; the statistics
        // are those of the decoded values
        const size_t ro = (size_t)map_row(min(m, rows - 1), rm);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int n = nbase + nt * 16 + col;
          const uint16_t h = cmp_encode(zv[nt], zm);
          if (m < rows && n < V) z16[ro * V + n] = h;
          zv[nt] = cmp_decode(h, zm);
        }
        if (col == 0 && m < rows && nbase < V) bmax[ro * ((V + 127) >> 7) + (nbase >> 7)] = zm;
      }
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
  if (tid < TM && m < rows) {
    Rec rc = hrec[0][tid];
    rec_merge(rc, hrec[1][tid]);
    float* pr = part + ((size_t)m * nn + nt_idx) * 4;
    *reinterpret_cast<float4*>(pr) = make_float4(rc.tmax, rc.s, rc.zmax, __int_as_float(rc.arg));
  }
}

// Split hidden dimension: one workgroup per (512-column tile, row) sums the
// KS partial logits in slice order, writes the logits and the tile's record
// (the streaming kernel's: max z/T', sum exp, max z, tile).
__global__ __launch_bounds__(256) void lm_combine_kernel(int rows, int V, int KS, float Tp,
                                                         const float* __restrict__ partial, float* __restrict__ logits,
                                                         float* __restrict__ part, int32_t* status, RowMap rm) {
  __shared__ float shm[4], shs[4];
  const int tile = blockIdx.x, m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = tile * kLmTileN;
  float z[2];
  bool bad = false;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = n0 + h * 256 + tid;
    float v = kNegInf;
    if (n < V) {
      // eight slices' loads in flight at a time; the sum keeps slice order
      float acc = 0.f;
      const float* pp = partial + (size_t)m * V + n;
      const size_t sl = (size_t)rows * V;
      for (int kz0 = 0; kz0 < KS; kz0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = kz0 + j < KS ? pp[(size_t)(kz0 + j) * sl] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (kz0 + j < KS) acc += v[j];
      }
      logits[(size_t)map_row(m, rm) * V + n] = acc;
      v = acc;
      if (!isfinite(v)) { bad = true; v = kNegInf; }
    }
    z[h] = v;
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  float zm = wave_max(fmaxf(z[0], z[1]));
  if (lane == 0) shm[wave] = zm;
  __syncthreads();
  zm = fmaxf(fmaxf(shm[0], shm[1]), fmaxf(shm[2], shm[3]));
  const float tmax = zm / Tp;
  float sum = 0.f;
  if (zm != kNegInf) {
    const float cT = kLog2e / Tp, off = tmax * kLog2e;
    sum = __builtin_amdgcn_exp2f(fmaf(z[0], cT, -off)) + __builtin_amdgcn_exp2f(fmaf(z[1], cT, -off));
  }
  sum = wave_sum(sum);
  if (lane == 0) shs[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    const float s = (shs[0] + shs[1]) + (shs[2] + shs[3]);
    float* pr = part + ((size_t)m * gridDim.x + tile) * 4;
    *reinterpret_cast<float4*>(pr) =
        make_float4(zm == kNegInf ? kNegInf : tmax, s, zm, __int_as_float(kLmArgTile | n0));
  }
}

// lm_combine_kernel for compact rows: the summed logits of one 512-column
// tile of one row become four 128-column blocks (fp16 offsets + block maxima);
// the tile's record holds the statistics of the decoded values and the exact
// argmax column.
__global__ __launch_bounds__(256) void lm_combine_compact_kernel(int rows, int V, int KS, float Tp,
                                                                 const float* __restrict__ partial,
                                                                 uint16_t* __restrict__ z16, float* __restrict__ bmax,
                                                                 float* __restrict__ part, int32_t* status,
                                                                 RowMap rm) {
  __shared__ float shm[2][4], shs[4], sha[4];
  __shared__ int shi[4];
  const int tile = blockIdx.x, m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = tile * kLmTileN;
  const size_t ro = (size_t)map_row(m, rm);
  const int nblk = (V + 127) >> 7;
  float z[2];
  bool bad = false;
  float bz = kNegInf;
  int bi = kIdxNone;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = n0 + h * 256 + tid;
    float v = kNegInf;
    if (n < V) {
      float acc = 0.f;
      const float* pp = partial + (size_t)m * V + n;
      const size_t sl = (size_t)rows * V;
      for (int kz0 = 0; kz0 < KS; kz0 += 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = kz0 + j < KS ? pp[(size_t)(kz0 + j) * sl] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (kz0 + j < KS) acc += x[j];
      }
      v = acc;
      if (!isfinite(v)) { bad = true; v = kNegInf; }
    }
    z[h] = v;
    if (v > bz) { bz = v; bi = n; }  // h ascends with the column: ties keep the lower id
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  // block maxima: block 2h + (wave >> 1) spans waves 2(wave >> 1), 2(wave >> 1) + 1 of half h
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float wm = wave_max(z[h]);
    if (lane == 0) shm[h][wave] = wm;
  }
  wave_argmax(bz, bi);
  if (lane == 0) { sha[wave] = bz; shi[wave] = bi; }
  __syncthreads();
  float sum = 0.f;
  float zt[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w0 = wave & ~1;
    const float mb = fmaxf(shm[h][w0], shm[h][w0 + 1]);
    const int n = n0 + h * 256 + tid;
    const uint16_t code = cmp_encode(z[h], mb);
    if (n < V) z16[ro * V + n] = code;
    if ((tid & 127) == 0 && n < V) bmax[ro * nblk + (n >> 7)] = mb;
    zt[h] = cmp_decode(code, mb);
  }
  // the tile maximum over the four blocks (equal in every thread)
  float zmax = kNegInf;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int w = 0; w < 4; ++w) zmax = fmaxf(zmax, shm[h][w]);
  const float tmax = zmax / Tp;
  if (zmax != kNegInf) {
    const float cT = kLog2e / Tp, off = tmax * kLog2e;
    sum = __builtin_amdgcn_exp2f(fmaf(zt[0], cT, -off)) + __builtin_amdgcn_exp2f(fmaf(zt[1], cT, -off));
  }
  sum = wave_sum(sum);
  if (lane == 0) shs[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    const float s = (shs[0] + shs[1]) + (shs[2] + shs[3]);
    float az = sha[0];
    int ai = shi[0];
    for (int w = 1; w < 4; ++w)
      if (beats(sha[w], shi[w], az, ai)) { az = sha[w]; ai = shi[w]; }
    float* pr = part + ((size_t)m * gridDim.x + tile) * 4;
    *reinterpret_cast<float4*>(pr) = make_float4(zmax == kNegInf ? kNegInf : tmax, s, zmax, __int_as_float(ai));
  }
}

// One workgroup per row: merge the row's per-tile records (fp64 sum).
__global__ __launch_bounds__(256) void lm_finalize_kernel(int rows, int ntiles, int V, const float* __restrict__ part,
                                                          const float* __restrict__ logits, float* __restrict__ row_stats,
                                                          int32_t* __restrict__ row_argmax, RowMap rm) {
  __shared__ float shf[4];
  __shared__ double shd[4];
  __shared__ int shi[4];
  __shared__ int shc[4];
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
  const double ssum = (shd[0] + shd[1]) + (shd[2] + shd[3]);
  // A tile record names the first tile holding the row max (ties between
  // tiles go to the lower one); its first column equal to that max is the
  // argmax.  Non-finite logits never equal the (finite) max.
  int arg = ba == kIdxNone ? 0 : ba;
  if (ba != kIdxNone && (ba & kLmArgTile)) {
    const int c0 = ba & ~kLmArgTile, c1 = min(c0 + kLmTileN, V);
    int first = kIdxNone;
    if (bz != kNegInf)
      for (int n = c0 + tid; n < c1; n += 256)
        if (logits[(size_t)map_row(m, rm) * V + n] == bz) { first = n; break; }
    first = wave_min_i(first);
    if (lane == 0) shc[wave] = first;
    __syncthreads();
    first = min(min(shc[0], shc[1]), min(shc[2], shc[3]));
    arg = first == kIdxNone ? 0 : first;
  }
  if (tid == 0) {
    row_stats[(size_t)m * 2] = M;
    row_stats[(size_t)m * 2 + 1] = (float)ssum;
    row_argmax[m] = arg;
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

// Row-major W [V, H] -> z-packed layout (eagle.h): one wave per fragment,
// lane l taking the same 8 weights as in the packed layout.  The wave's
// extremes of e >> 1 decide the fragment's form; rows beyond V are zero.
__global__ __launch_bounds__(256) void zpack_w_kernel(int V, int H, const uint16_t* __restrict__ w,
                                                      unsigned char* __restrict__ wz, ZLayout zl,
                                                      int32_t* __restrict__ raw_count) {
  const int nch = H / kKC;
  const int l = threadIdx.x & 63;
  for (size_t f = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; f < zl.nfrag;
       f += ((size_t)gridDim.x * blockDim.x) >> 6) {
    const int j = (int)(f & 7);
    const size_t gc = f >> 3;
    const int c = (int)(gc % nch);
    const size_t g = gc / nch;
    const size_t row = g * 64 + (j & 3) * 16 + (l & 15);
    const int k = c * kKC + (j >> 2) * 32 + (l >> 4) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < (size_t)V) v = *reinterpret_cast<const u32x4*>(w + row * H + k);
    uint32_t hi[8], lo[8];
    int emax = 0, emin = 127;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (v[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      lo[i] = h & 0xffu;
      hi[i] = h >> 8;
      emax = max(emax, (int)(hi[i] & 0x7fu));
      emin = min(emin, (int)(hi[i] & 0x7fu));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      emax = max(emax, __shfl_xor(emax, o));
      emin = min(emin, __shfl_xor(emin, o));
    }
    const int base = max(emax - 7, 0);
    const bool raw = emin < base;
    const uint32_t l0 = lo[0] | lo[1] << 8 | lo[2] << 16 | lo[3] << 24;
    const uint32_t l1 = lo[4] | lo[5] << 8 | lo[6] << 16 | lo[7] << 24;
    if (raw) {
      const uint32_t h0 = hi[0] | hi[1] << 8 | hi[2] << 16 | hi[3] << 24;
      const uint32_t h1 = hi[4] | hi[5] << 8 | hi[6] << 16 | hi[7] << 24;
      *reinterpret_cast<u32x4*>(wz + zl.raw_off + f * 1024 + l * 16) = u32x4{l0, l1, h0, h1};
    } else {
      uint32_t codes = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t code = ((hi[i] >> 7) << 3) | ((hi[i] & 0x7fu) - (uint32_t)base);
        codes |= code << (8 * (i & 3) + 4 * (i >> 2));
      }
      uint32_t* o = reinterpret_cast<uint32_t*>(wz + zl.slot_off + f * 768 + l * 12);
      o[0] = l0;
      o[1] = l1;
      o[2] = codes;
    }
    if (l == 0) {
      wz[f] = (unsigned char)(raw ? 0x80 : base);
      if (raw && raw_count != nullptr) atomicAdd(raw_count, 1);
    }
  }
}

}  // namespace

hipError_t launch_zpack_lmhead(int V, int H, const void* w, void* wz, int32_t* raw_count, hipStream_t st) {
  const ZLayout zl = lm_zlayout(V, H);
  if (raw_count != nullptr) {
    hipError_t e = launch_zero_ints(raw_count, 1, st);
    if (e != hipSuccess) return e;
  }
  const size_t threads = zl.nfrag * 64;
  const int grid = (int)((threads + 255) / 256 < 16384 ? (threads + 255) / 256 : 16384);
  zpack_w_kernel<<<grid, 256, 0, st>>>(V, H, (const uint16_t*)w, (unsigned char*)wz, zl, raw_count);
  return hipGetLastError();
}

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
  return launch_lmhead_map(rows, H, V, dtype, w_layout, x, w, T, logits, row_stats, row_argmax, probs, ws_part, status,
                           RowMap{1 << 30, 0, 0}, st);
}

hipError_t launch_lmhead_map(int rows, int H, int V, int dtype, int w_layout, const void* x, const void* w, float T,
                             float* logits, float* row_stats, int32_t* row_argmax, float* probs, float* ws_part,
                             int32_t* status, RowMap rm, hipStream_t st) {
  return launch_lmhead_impl(rows, H, V, dtype, w_layout, x, w, T, logits, row_stats, row_argmax, probs, ws_part,
                            status, rm, nullptr, nullptr, nullptr, st);
}

hipError_t launch_lmhead_compact(int rows, int H, int V, int w_layout, const void* x, const void* w, float T,
                                 uint16_t* z16, float* bmax, float* row_stats, int32_t* row_argmax, float* ws_part,
                                 int32_t* status, hipStream_t st) {
  return launch_lmhead_impl(rows, H, V, EAGLE_BF16, w_layout, x, w, T, nullptr, row_stats, row_argmax, nullptr,
                            ws_part, status, RowMap{1 << 30, 0, 0}, nullptr, z16, bmax, st);
}

hipError_t launch_product(int rows, int H, int V, const void* x, const void* w_packed, float* out, float* ws_part,
                          int32_t* status, ProductOut* po, hipStream_t st) {
  int ks = 1;
  hipError_t e = launch_lmhead_impl(rows, H, V, EAGLE_BF16, EAGLE_W_PACKED, x, w_packed, 1.f, out, nullptr, nullptr,
                                    nullptr, ws_part, status, RowMap{1 << 30, 0, 0}, &ks, nullptr, nullptr, st);
  po->ks = ks;
  po->src = ks > 1 ? ws_part + lm_rec_floats(rows, V) : out;
  po->slice = (size_t)rows * V;
  return e;
}

hipError_t launch_lmhead_impl(int rows, int H, int V, int dtype, int w_layout, const void* x, const void* w, float T,
                              float* logits, float* row_stats, int32_t* row_argmax, float* probs, float* ws_part,
                              int32_t* status, RowMap rm, int* defer_ks, uint16_t* z16, float* bmax,
                              hipStream_t st) {
  const float Tp = (T > 0.f) ? T : 1.0f;
  int ntiles = lm_ntiles(V);
  if (dtype == EAGLE_BF16 && rows >= kGemmMinRows) {
    if (w_layout == EAGLE_W_ZPACKED) return hipErrorInvalidValue;  // the host checks reject this first
    // plain products with few tiles split the hidden dimension (no statistics then)
    const GemmPlan gp = gemm_plan(rows, V, H, row_stats != nullptr);
    const int TM = gp.tm, ks = gp.ks;
    const int nm = (rows + TM - 1) / TM, nn = lm_gemm_ntiles(V);
    ntiles = nn;
    // blocks of bm row tiles x bn vocab tiles per XCD (16 x 2 measured best at
    // 16 row tiles).  Up to 16 row tiles go in one block; more take the bm in
    // 8..16 that pads them least.  bn is the largest width <= 32 / bm that
    // pads the XCD's vocab tiles by at most a sixteenth, else the least padding.
    const int nn8 = (nn + 7) / 8;  // vocab tiles of XCD 0 (the most of any XCD)
    auto padded = [](int n, int b) { return (n + b - 1) / b * b; };
    int bm = nm;
    if (nm > 16) {
      bm = 16;
      for (int c = 15; c >= 8; --c)
        if (padded(nm, c) < padded(nm, bm)) bm = c;
    }
    int bn = 1;
    for (int c = 2; c <= 32 / bm && c <= nn8; ++c)
      if (padded(nn8, c) < padded(nn8, bn) || 16 * (padded(nn8, c) - nn8) <= nn8) bn = c;
    const int gps = ((nm + bm - 1) / bm * bm) * ((nn8 + bn - 1) / bn * bn) * 8;
    float* partial = ks > 1 ? ws_part + lm_rec_floats(rows, V) : nullptr;
    const size_t lds = 0;
#define EAGLE_GEMM(PK, M, SG)                                                                                   \
  lmhead_gemm_kernel<PK, M, SG><<<gps * ks, M * 2, lds, st>>>(                                                   \
      rows, H, V, Tp, nm, nn, bm, bn, (const uint16_t*)x, (const uint16_t*)w, logits, ws_part, status, rm, gps, ks, \
      partial, z16, bmax)
    if (w_layout == EAGLE_W_PACKED) {
      if (TM == 256) EAGLE_GEMM(true, 256, 4);
      else EAGLE_GEMM(true, 128, 3);
    } else {
      if (TM == 256) EAGLE_GEMM(false, 256, 4);
      else EAGLE_GEMM(false, 128, 3);
    }
#undef EAGLE_GEMM
    if (defer_ks) *defer_ks = ks;
    if (ks > 1 && !defer_ks) {  // plain products only (statistics take ks = 1): never compact
      hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      lm_combine_kernel<<<dim3(lm_ntiles(V), rows), 256, 0, st>>>(rows, V, ks, Tp, partial, logits, ws_part, status,
                                                                  rm);
    }
  } else if (dtype == EAGLE_BF16) {
    const int ks = lm_ksplit(rows, V, H);
    float* partial = ks > 1 ? ws_part + lm_rec_floats(rows, V) : nullptr;
    dim3 grid(ntiles, lm_mtiles(rows), ks);
    // z-packed: the header bytes of every wave's steps in dynamic LDS
    const size_t zlds = w_layout == EAGLE_W_ZPACKED ? (size_t)8 * (H / ks / kKC / 2) * 16 : 0;
#define EAGLE_STREAM(WLAY)                                                                                     \
  lmhead_bf16_kernel<WLAY><<<grid, kLmThreads, zlds, st>>>(rows, H, V, Tp, (const uint16_t*)x, (const uint16_t*)w, \
                                                           logits, ws_part, status, H / ks, partial, rm, z16, bmax)
    if (w_layout == EAGLE_W_ZPACKED) EAGLE_STREAM(EAGLE_W_ZPACKED);
    else if (w_layout == EAGLE_W_PACKED) EAGLE_STREAM(EAGLE_W_PACKED);
    else EAGLE_STREAM(EAGLE_W_ROWMAJOR);
#undef EAGLE_STREAM
    if (defer_ks) *defer_ks = ks;
    if (ks > 1 && !defer_ks) {
      hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      if (z16 != nullptr)
        lm_combine_compact_kernel<<<dim3(ntiles, rows), 256, 0, st>>>(rows, V, ks, Tp, partial, z16, bmax, ws_part,
                                                                      status, rm);
      else
        lm_combine_kernel<<<dim3(ntiles, rows), 256, 0, st>>>(rows, V, ks, Tp, partial, logits, ws_part, status, rm);
    }
  } else {
    dim3 grid(ntiles, rows);
    lmhead_f32_kernel<<<grid, 256, (size_t)H * sizeof(float), st>>>(rows, H, V, Tp, (const float*)x,
                                                                    (const float*)w, logits, ws_part, status, rm);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Without row statistics the call is a plain product (the records stay unused).
  if (row_stats == nullptr) return e;
  // A separate launch merges the per-tile records: the kernel boundary makes
  // every workgroup's records visible (an in-kernel agent-scope fence would
  // write back each XCD's whole L2 per workgroup).
  lm_finalize_kernel<<<rows, 256, 0, st>>>(rows, ntiles, V, ws_part, logits, row_stats, row_argmax, rm);
  e = hipGetLastError();
  if (e != hipSuccess || probs == nullptr) return e;
  const size_t total = (size_t)rows * V;
  const int grid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  probs_kernel<<<grid, 256, 0, st>>>(rows, V, Tp, logits, row_stats, probs);
  return hipGetLastError();
}

}  // namespace eagle
