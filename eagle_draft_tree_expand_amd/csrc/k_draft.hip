// Synthetic EAGLE draft head, one depth of the draft tree per call: the
// decoder-layer forward of that depth's frontier nodes and their draft rows.
//
// Method: EAGLE-1 notes ("EAGLE: Speculative Sampling Requires Rethinking
// Feature Uncertainty"), section 3.1: the head concatenates a feature with the
// embedding of the token one step ahead, an FC layer maps the 2H values to H,
// one decoder layer predicts the next feature and the target's LM head turns
// it into the draft distribution; predicted features are fed back in.
// EAGLE-3 notes, inference pipeline: a drafted token's feature is the head's
// own output.  EAGLE-2 notes, "Expanding the Draft Tree": one draft forward per
// depth, over the k nodes expanded at that depth.
//
// Per depth d (R = B * kd frontier rows, kd = 1 at the root, else k), every
// step on the caller's stream:
//   draft_in      x0 = [f ; E[x]] (bf16) of each frontier node, its slot's
//                 ancestor mask row (the parent's row plus itself); at d = 0
//                 also the per-round slot state (zero k/v rows, root-only
//                 masks) so that not-yet-drafted slots stay finite
//   GEMM fc       u = x0 Wfc^T                    (bf16 MFMA, fp32 out)
//   norm          n1 = bf16(rms(u))
//   GEMM qkv      [q k v] = n1 Wqkv^T
//   draft_qkv     bf16 q rows of the frontier; k/v rows into the
//                 slot-indexed tree buffers
//   attention     the frontier's queries over the draft prefix and the slot
//                 keys, each under its slot's mask (its root path)
//   GEMM o        y = o Wo^T;  norm: h = u + y, n2 = bf16(rms(h))
//   GEMM gate_up  [g u] = n2 Wgu^T;  draft_silu: bf16(silu(g) * u)
//   GEMM down     y = m Wd^T;  norm: a = h + y -> bf16 feature of the slot
//   LM head       draft rows z = a W^T written at their slots of [B, S, V]
// The GEMMs are the streaming LM-head kernel (weights read once, straight
// from HBM into registers; the hidden dimension split over workgroups for the
// narrow outputs), or the tiled GEMM for many rows.  A split product's fp32
// slices are summed by the kernel that consumes it (norm, draft_qkv,
// draft_silu), not by a launch of their own.  At batch 1 every step is
// weight- or launch-bound.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kDT = 256;  // threads of the row kernels

EDEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
EDEV void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// One workgroup per frontier row r (request b = r / kd, slot s0 + r % kd).
__global__ __launch_bounds__(kDT) void draft_in_kernel(
    int depth, int kd, int s0, int S, int k, int P, int H, int V, int KV, int W,
    const int32_t* __restrict__ root, const uint16_t* __restrict__ root_feat, const int32_t* __restrict__ pool_tok,
    const int32_t* __restrict__ slot_src, const uint16_t* __restrict__ embed, uint16_t* __restrict__ slot_feat,
    uint64_t* __restrict__ slot_mask, uint16_t* __restrict__ slot_k, uint16_t* __restrict__ slot_v,
    int32_t* __restrict__ idx, uint16_t* __restrict__ x0, int32_t* status) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int b = r / kd, s = s0 + (r - b * kd);
  const size_t srow = (size_t)b * S + s;
  int tok, ps = -1;
  if (depth == 0) {
    tok = root[b];
  } else {
    const int e = slot_src[srow];
    const bool ok = e >= 0 && e < P;
    if (!ok && tid == 0) set_status(status, EAGLE_STATUS_BAD_TREE);
    tok = ok ? pool_tok[(size_t)b * P + e] : 0;
    ps = ok ? e / k : 0;
  }
  if (tok < 0 || tok >= V) {
    if (tid == 0) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
    tok = tok < 0 ? 0 : V - 1;
  }
  if (tid == 0) idx[r] = (int32_t)srow;
  // x0 = [f ; E[tok]] in 16-byte units (H is a multiple of 128)
  const uint16_t* f = depth == 0 ? root_feat + (size_t)b * H : slot_feat + ((size_t)b * S + ps) * H;
  const uint16_t* e = embed + (size_t)tok * H;
  uint16_t* xr = x0 + (size_t)r * 2 * H;
  const int hu = H / 8;
  for (int u = tid; u < 2 * hu; u += kDT) {
    const uint4 v = u < hu ? ld16(f + u * 8) : ld16(e + (u - hu) * 8);
    st16(xr + u * 8, v);
  }
  // mask row: the parent's ancestors (a slot of an earlier depth) plus itself
  for (int w = tid; w < W; w += kDT) {
    uint64_t m = depth == 0 ? 0ull : slot_mask[((size_t)b * S + ps) * W + w];
    if (w == (s >> 6)) m |= 1ull << (s & 63);
    slot_mask[srow * W + w] = m;
  }
  if (depth != 0) return;
  // Round start: slots 1..S-1 of this request are not drafted yet.  Their
  // mask rows see the root only and their k/v rows are zero, so that the
  // attention reads finite values in every slot (masked keys still pass
  // through the MFMAs with weight 0).
  for (int x = tid; x < (S - 1) * W; x += kDT) {
    const int s1 = 1 + x / W, w = x - (s1 - 1) * W;
    slot_mask[((size_t)b * S + s1) * W + w] = w == 0 ? 1ull : 0ull;
  }
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  const size_t kn = (size_t)(S - 1) * KV / 8;
  uint16_t* k1 = slot_k + ((size_t)b * S + 1) * KV;
  uint16_t* v1 = slot_v + ((size_t)b * S + 1) * KV;
  for (size_t u = tid; u < kn; u += kDT) {
    st16(k1 + u * 8, z);
    st16(v1 + u * 8, z);
  }
}

// The products' hidden-split slices are summed here, in slice order (eight
// slices' loads in flight), by the kernel that consumes the product: x = sum
// over kz < ks of src[kz * slice + e].  (Slice order is kept whatever the
// number in flight, so the sums do not depend on it.)
struct Slices {
  const float* src;
  int ks;
  size_t slice;
};

template <int NB>  // slices' loads in flight
EDEV float4 sum_slices4(const Slices& p, size_t e) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* q = p.src + e;
  for (int kz0 = 0; kz0 < p.ks; kz0 += NB) {
    float4 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      v[j] = kz0 + j < p.ks ? *reinterpret_cast<const float4*>(q + (size_t)(kz0 + j) * p.slice)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (kz0 + j < p.ks) { acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w; }
  }
  return acc;
}

EDEV float2 sum_slices2(const Slices& p, size_t e) {
  float2 acc = make_float2(0.f, 0.f);
  const float* q = p.src + e;
  for (int kz0 = 0; kz0 < p.ks; kz0 += 8) {
    float2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = kz0 + j < p.ks ? *reinterpret_cast<const float2*>(q + (size_t)(kz0 + j) * p.slice) : make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (kz0 + j < p.ks) { acc.x += v[j].x; acc.y += v[j].y; }
  }
  return acc;
}

EDEV bool finite4(float4 v) { return isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w); }

constexpr int kNT = 1024;          // threads of the norm kernel
// hidden sizes up to kNT * 16 = 16384 are held in registers (4 float4 per thread)

// One workgroup per row r: h = (the product's row) + res (res optional);
// writes any of hout = h, nout = bf16(h / sqrt(mean(h^2) + 1e-6)), xout =
// bf16(h), and bf16(h) to the slot-indexed feature row fout[idx[r]].
__global__ __launch_bounds__(kNT) void draft_norm_kernel(int H, Slices p, const float* __restrict__ res,
                                                         float* __restrict__ hout, uint16_t* __restrict__ nout,
                                                         uint16_t* __restrict__ xout, uint16_t* __restrict__ fout,
                                                         const int32_t* __restrict__ idx, int32_t* status) {
  __shared__ float red[kNT / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4 h[4];
  float ss = 0.f;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = (j * kNT + tid) * 4;
    if (i >= H) continue;
    float4 v = sum_slices4<16>(p, (size_t)r * H + i);
    if (res) {
      const float4 w = *reinterpret_cast<const float4*>(res + (size_t)r * H + i);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    bad |= !finite4(v);
    h[j] = v;
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    if (hout) *reinterpret_cast<float4*>(hout + (size_t)r * H + i) = v;
    const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    if (xout) *reinterpret_cast<uint2*>(xout + (size_t)r * H + i) = make_uint2(lo, hi);
    if (fout) *reinterpret_cast<uint2*>(fout + (size_t)idx[r] * H + i) = make_uint2(lo, hi);
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
  if (!nout) return;
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = (j * kNT + tid) * 4;
    if (i >= H) continue;
    const float4 v = h[j];
    const uint32_t lo = (uint32_t)f32_to_bf16(v.x * inv) | ((uint32_t)f32_to_bf16(v.y * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v.z * inv) | ((uint32_t)f32_to_bf16(v.w * inv) << 16);
    *reinterpret_cast<uint2*>(nout + (size_t)r * H + i) = make_uint2(lo, hi);
  }
}

// The [q | k | v] product rows to bf16: q to row r of the frontier's queries,
// k and v to the rows of slot idx[r]; one thread per pair of columns.
__global__ __launch_bounds__(kDT) void draft_qkv_kernel(int R, int Q, int KV, Slices p,
                                                        const int32_t* __restrict__ idx, uint16_t* __restrict__ sq,
                                                        uint16_t* __restrict__ sk, uint16_t* __restrict__ sv,
                                                        int32_t* status) {
  const int n = Q + 2 * KV, hp = n / 2;
  const size_t total = (size_t)R * hp;
  bool bad = false;
  for (size_t x = (size_t)blockIdx.x * kDT + threadIdx.x; x < total; x += (size_t)gridDim.x * kDT) {
    const int r = (int)(x / hp), i = (int)(x - (size_t)r * hp) * 2;
    const float2 v = sum_slices2(p, (size_t)r * n + i);
    bad |= !(isfinite(v.x) && isfinite(v.y));
    const size_t o = (size_t)idx[r];
    const uint32_t pk = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    uint16_t* dst = i < Q ? sq + (size_t)r * Q + i : i < Q + KV ? sk + o * KV + (i - Q) : sv + o * KV + (i - Q - KV);
    *reinterpret_cast<uint32_t*>(dst) = pk;
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
}

// bf16(silu(g) * u) from the [g | u] product rows (I each); one thread per
// pair of columns over all rows.
__global__ __launch_bounds__(kDT) void draft_silu_kernel(int R, int I, Slices p, uint16_t* __restrict__ out,
                                                         int32_t* status) {
  const int hp = I / 2;
  const size_t total = (size_t)R * hp;
  bool bad = false;
  for (size_t x = (size_t)blockIdx.x * kDT + threadIdx.x; x < total; x += (size_t)gridDim.x * kDT) {
    const int r = (int)(x / hp), i = (int)(x - (size_t)r * hp) * 2;
    const float2 gv = sum_slices2(p, (size_t)r * 2 * I + i), uv = sum_slices2(p, (size_t)r * 2 * I + I + i);
    bad |= !(isfinite(gv.x) && isfinite(gv.y) && isfinite(uv.x) && isfinite(uv.y));
    const float a = gv.x / (1.0f + expf(-gv.x)) * uv.x, c = gv.y / (1.0f + expf(-gv.y)) * uv.y;
    *reinterpret_cast<uint32_t*>(out + (size_t)r * I + i) =
        (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(c) << 16);
  }
  if (bad) set_status(status, EAGLE_STATUS_NONFINITE);
}

int grid_for(size_t items) { return (int)((items + kDT - 1) / kDT < 2048 ? (items + kDT - 1) / kDT : 2048); }

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

DraftLayout draft_layout(int B, int S, int k, int V, int H, int hq, int hkv, int dh, int I, int max_prefix) {
  DraftLayout L;
  const size_t Q = (size_t)hq * dh, KV = (size_t)hkv * dh, W = (size_t)(S + 63) / 64;
  const size_t BS = (size_t)B * S, R = (size_t)B * (k > 1 ? k : 1);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += up256(bytes); return at; };
  L.slot_k = take(BS * KV * 2);
  L.slot_v = take(BS * KV * 2);
  L.slot_feat = take(BS * H * 2);
  L.slot_mask = take(BS * W * 8);
  L.idx = take(R * 4);
  L.x0 = take(R * 2 * H * 2);
  L.u = take(R * H * 4);
  L.n1 = take(R * H * 2);
  L.qkv = take(R * (Q + 2 * KV) * 4);
  L.qc = take(R * Q * 2);
  L.og = take(R * Q * 2);
  L.h = take(R * H * 4);
  L.n2 = take(R * H * 2);
  L.gu = take(R * 2 * (size_t)I * 4);
  L.mm = take(R * (size_t)I * 2);
  L.y = take(R * H * 4);
  L.xa = take(R * H * 2);
  size_t g = 0;
  const int rs[2] = {B, (int)R};
  for (int t = 0; t < 2; ++t) {
    const int r = rs[t];
    const size_t c[6] = {lm_ws_bytes(r, H, 2 * H), lm_ws_bytes(r, (int)(Q + 2 * KV), H), lm_ws_bytes(r, H, (int)Q),
                         lm_ws_bytes(r, 2 * I, H), lm_ws_bytes(r, H, I), lm_ws_bytes(r, V, H)};
    for (size_t x : c) g = x > g ? x : g;
  }
  L.gemm = take(g);
  // the largest query window (k frontier nodes); depth 0 plans for one
  L.attn = take(attn_ws_bytes(B, hkv, dh, attn_plan(B, k, hq, hkv, dh, max_prefix, EAGLE_BF16)));
  L.total = o;
  return L;
}

hipError_t launch_draft_forward(const DraftArgs& a, hipStream_t st) {
  const DraftLayout& L = a.lay;
  char* base = static_cast<char*>(a.ws);
  auto P16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  auto PF = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const int B = a.B, S = a.S, k = a.k, H = a.H, I = a.I;
  const int Q = a.hq * a.dh, KV = a.hkv * a.dh, W = (S + 63) / 64, P = S * k;
  const int kd = a.depth == 0 ? 1 : k, s0 = a.depth == 0 ? 0 : 1 + (a.depth - 1) * k;
  const int R = B * kd;
  int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
  float* gws = PF(L.gemm);
  const RowMap id{1 << 30, 0, 0};
  hipError_t e;
#define EAGLE_CK(x) \
  do {              \
    e = (x);        \
    if (e != hipSuccess) return e; \
  } while (0)

  draft_in_kernel<<<R, kDT, 0, st>>>(a.depth, kd, s0, S, k, P, H, a.V, KV, W, a.root, (const uint16_t*)a.root_feat,
                                     a.pool_tok, a.slot_src, (const uint16_t*)a.w.embed, P16(L.slot_feat),
                                     reinterpret_cast<uint64_t*>(base + L.slot_mask), P16(L.slot_k), P16(L.slot_v),
                                     idx, P16(L.x0), a.status);
  EAGLE_CK(hipGetLastError());
  ProductOut po;
  auto sl = [&]() { return Slices{po.src, po.ks, po.slice}; };
  EAGLE_CK(launch_product(R, 2 * H, H, P16(L.x0), a.w.fc, PF(L.u), gws, a.status, &po, st));
  // u (kept as the residual) and n1 = bf16(rms(u))
  draft_norm_kernel<<<R, kNT, 0, st>>>(H, sl(), nullptr, PF(L.u), P16(L.n1), nullptr, nullptr, idx, a.status);
  EAGLE_CK(hipGetLastError());
  EAGLE_CK(launch_product(R, H, Q + 2 * KV, P16(L.n1), a.w.qkv, PF(L.qkv), gws, a.status, &po, st));
  draft_qkv_kernel<<<grid_for((size_t)R * (Q + 2 * KV) / 2), kDT, 0, st>>>(R, Q, KV, sl(), idx, P16(L.qc),
                                                                          P16(L.slot_k), P16(L.slot_v), a.status);
  EAGLE_CK(hipGetLastError());
  // the frontier's kd queries are tree nodes s0 .. s0+kd-1 of the S slots;
  // the output rows come out in frontier order, ready for the o product
  EAGLE_CK(launch_attention_window(B, S, kd, s0, a.hq, a.hkv, a.dh, a.max_prefix, EAGLE_BF16, P16(L.qc), a.k_prefix,
                                   a.v_prefix, a.prefix_len, P16(L.slot_k), P16(L.slot_v),
                                   reinterpret_cast<const uint64_t*>(base + L.slot_mask), a.scale, P16(L.og),
                                   PF(L.attn), attn_plan(B, kd, a.hq, a.hkv, a.dh, a.max_prefix, EAGLE_BF16),
                                   a.status, st));
  EAGLE_CK(launch_product(R, Q, H, P16(L.og), a.w.o, PF(L.y), gws, a.status, &po, st));
  // h = u + o Wo^T and n2 = bf16(rms(h))
  draft_norm_kernel<<<R, kNT, 0, st>>>(H, sl(), PF(L.u), PF(L.h), P16(L.n2), nullptr, nullptr, idx, a.status);
  EAGLE_CK(hipGetLastError());
  EAGLE_CK(launch_product(R, H, 2 * I, P16(L.n2), a.w.gate_up, PF(L.gu), gws, a.status, &po, st));
  draft_silu_kernel<<<grid_for((size_t)R * I / 2), kDT, 0, st>>>(R, I, sl(), P16(L.mm), a.status);
  EAGLE_CK(hipGetLastError());
  EAGLE_CK(launch_product(R, I, H, P16(L.mm), a.w.down, PF(L.y), gws, a.status, &po, st));
  // a = h + m Wd^T: bf16 to the LM-head input and to the slot's feature
  draft_norm_kernel<<<R, kNT, 0, st>>>(H, sl(), PF(L.h), nullptr, nullptr, P16(L.xa), P16(L.slot_feat), idx,
                                       a.status);
  EAGLE_CK(hipGetLastError());
  // draft rows of the frontier at their slots: row r -> (r / kd) * S + s0 + r % kd
  const bool lz = a.w.lm_head_z != nullptr && R <= EAGLE_ZPACK_MAX_ROWS;
  EAGLE_CK(launch_lmhead_map(R, H, a.V, EAGLE_BF16, lz ? EAGLE_W_ZPACKED : EAGLE_W_PACKED, P16(L.xa),
                             lz ? a.w.lm_head_z : a.w.lm_head, 1.f, a.rows, nullptr, nullptr, nullptr, gws, a.status,
                             RowMap{kd, S, s0}, st));
#undef EAGLE_CK
  return hipSuccess;
}

}  // namespace eagle
