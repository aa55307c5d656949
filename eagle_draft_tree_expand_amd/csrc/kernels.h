// Host-side launchers of the libeagle kernels (one definition per .hip file).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/eagle.h"

namespace eagle {

// ---- expansion (k_expand.hip) ----
constexpr int kExpThreads = 256;
constexpr int kExpChunk = 4096;          // vocab entries per scan workgroup (16 per thread)
constexpr int kExpUnitsPerChunk = 4;     // one candidate record per wave
constexpr int kExpExtra = 2;             // extra candidates kept per wave beyond k
constexpr int kExpRescanCap = 2048;      // candidate capacity of the rare full-row re-scan

inline int exp_chunks(int V) { return (V + kExpChunk - 1) / kExpChunk; }
inline int exp_kp(int k) { return k + kExpExtra; }
inline size_t exp_unit_floats(int k) { return 2 + 2 * (size_t)exp_kp(k); }
inline size_t exp_ws_bytes(int B, int S, int V, int k) {
  return (size_t)B * S * exp_chunks(V) * kExpUnitsPerChunk * exp_unit_floats(k) * sizeof(float);
}

hipError_t launch_expand(int B, int S, int V, int D, int k, int m, float T, uint64_t seed,
                         uint64_t round_id, const float* rows, const uint32_t* bound, const int32_t* root,
                         int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                         int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                         int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                         float* slot_stats, float* ws_units, int32_t* status, hipStream_t st,
                         const int32_t* prefix_len = nullptr, uint64_t* mask = nullptr, int32_t* pos = nullptr);

// Depth by depth: children of depth `depth`'s frontier slots (rows at their
// slots of the [B, S, V] buffer), then the next depth's frontier into slot_src.
// bound: sampling-warp bounds of the [B, S] slot rows (those of this depth's
// slots are read), or null for no warp.
hipError_t launch_expand_depth(int B, int S, int V, int D, int k, int m, float T, uint64_t seed, uint64_t round_id,
                               int depth, const float* rows, const uint32_t* bound, int32_t* pool_tok, float* pool_q,
                               int32_t* slot_src, float* slot_stats, float* ws_units, int32_t* status, hipStream_t st);
// Rerank and flatten a complete pool.
hipError_t launch_expand_finish(int B, int S, int V, int D, int k, int m, const int32_t* root, int32_t* node_tok,
                                int32_t* node_parent, int32_t* node_depth, int32_t* node_sib, int32_t* node_slot,
                                float* node_value, float* node_q, const int32_t* pool_tok, const float* pool_q,
                                int32_t* pool_flat, int32_t* slot_src, int32_t* status, hipStream_t st);

// Static (caller-given) tree shape, derived on the host from its parent array
// and passed to the assembly kernel by value (node tables of at most
// EAGLE_MAX_NODES entries).
struct StaticShape {
  int n, S, kmax, D;
  int16_t parent[EAGLE_MAX_NODES];     // -1 for the root
  int16_t slot[EAGLE_MAX_NODES];       // slot of node i, -1 without children
  int16_t slot_node[EAGLE_MAX_NODES];  // node of slot s
  uint8_t sib[EAGLE_MAX_NODES];        // rank among its parent's children
  uint8_t depth[EAGLE_MAX_NODES];
  uint8_t slot_k[EAGLE_MAX_NODES];     // children of slot s
};
// Children of every slot (top-kmax per row), then the nodes of the shape.
hipError_t launch_expand_static(int B, int V, const StaticShape& sh, float T, uint64_t seed, uint64_t round_id,
                                const float* rows, const int32_t* root, int32_t* node_tok, int32_t* node_parent,
                                int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value,
                                float* node_q, int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                                float* slot_stats, float* ws_units, int32_t* status, hipStream_t st);

// ---- mask + gather (k_mask.hip) ----
hipError_t launch_tree_mask(int B, int n, const int32_t* parent, const int32_t* depth,
                            const int32_t* prefix_len, uint64_t* mask, int32_t* pos,
                            int32_t* status, hipStream_t st);
constexpr int kGatherMaxTables = 4;
struct GatherSet {
  const void* table[kGatherMaxTables];
  void* out[kGatherMaxTables];
  int row_units[kGatherMaxTables];
  int n;
};
hipError_t launch_gather(int n_rows, GatherSet gs, int table_rows, const int32_t* idx, int32_t* status,
                         hipStream_t st);
hipError_t launch_zero_ints(int32_t* p, size_t n, hipStream_t st);

// ---- post-accept commit (k_commit.hip) ----
constexpr int kCommitThreads = 256;
hipError_t launch_commit(int B, int n, int hkv, int head_dim, int max_prefix, int hidden, int D, int esz,
                         const int32_t* accept_len, const int32_t* accept_path, const void* kt, const void* vt,
                         const void* x, void* kp, void* vp, int32_t* prefix_len, void* feat, int32_t* status,
                         hipStream_t st);

// ---- attention (k_attn.hip) ----
struct AttnPlan {
  int rows;        // query rows per (request, kv head) = n * (hq / hkv)
  int rows_pad;    // rows rounded up to the MFMA tile
  int split_keys;  // prefix keys per split workgroup
  int nsplit;      // prefix splits (+1 split for the tree keys)
  int threads;     // bf16 split workgroup: 256 or 512 threads
  int qt;          // bf16: 16-row query tiles per wave (1 or 2)
};
AttnPlan attn_plan(int B, int n, int hq, int hkv, int head_dim, int max_prefix, int dtype);
inline size_t attn_ws_bytes(int B, int hkv, int head_dim, const AttnPlan& pl) {
  return (size_t)B * hkv * (pl.nsplit + 1) * pl.rows_pad * (head_dim + 2) * sizeof(float);
}
hipError_t launch_attention(int B, int n, int hq, int hkv, int head_dim, int max_prefix, int dtype,
                            const void* q, const void* kp, const void* vp, const int32_t* plen,
                            const void* kt, const void* vt, const uint64_t* mask, float scale,
                            void* out, float* ws, const AttnPlan& pl, int32_t* status,
                            hipStream_t st);
// Queries for a window of nq consecutive tree nodes qoff .. qoff+nq-1 only:
// q [B, nq, hq, dh] and out [B, nq, hq, dh] hold those nodes' rows, the mask
// rows are theirs in the [B, n, W] mask, all n tree keys stay; the plan is
// attn_plan(B, nq, ...).
hipError_t launch_attention_window(int B, int n, int nq, int qoff, int hq, int hkv, int head_dim, int max_prefix,
                                   int dtype, const void* q, const void* kp, const void* vp, const int32_t* plen,
                                   const void* kt, const void* vt, const uint64_t* mask, float scale, void* out,
                                   float* ws, const AttnPlan& pl, int32_t* status, hipStream_t st);

// ---- LM head (k_lmhead.hip) ----
constexpr int kLmTileN = 512;            // vocab columns per workgroup (one stats record per row)
constexpr int kLmTileM = 64;             // rows per workgroup
constexpr int kLmThreads = 512;          // bf16: 4 column quarters x 2 hidden halves
// Record arg of the streaming bf16 kernel: this bit plus the tile's first
// column; the row merge finds the column by scanning that tile's logits.
constexpr int kLmArgTile = 1 << 30;
inline int lm_ntiles(int V) { return (V + kLmTileN - 1) / kLmTileN; }
inline int lm_mtiles(int rows) { return (rows + kLmTileM - 1) / kLmTileM; }
// Large row counts (many requests per round) take a tiled GEMM: TM x 256
// output tiles, one stats record per (row, 256-column tile).
constexpr int kGemmTile = 256;
constexpr int kGemmMinRows = 193;        // from 4 row tiles of the streaming kernel on
inline int lm_gemm_ntiles(int V) { return (V + kGemmTile - 1) / kGemmTile; }
// Small vocabularies leave most CUs idle with one workgroup per (row tile,
// vocab tile): the bf16 streaming kernel then splits the hidden dimension over
// KS workgroups (slices of H/KS, a multiple of 128) that write fp32 partial
// logits; a combine launch sums them in a fixed order.
inline int lm_ksplit(int rows, int V, int H) {
  if (rows >= kGemmMinRows) return 1;
  int ks = 256 / (lm_ntiles(V) * lm_mtiles(rows));
  if (ks > 32) ks = 32;
  if (ks > H / 256) ks = H / 256;  // slices of at least 256: two chunks per hidden half to pipeline
  while (ks > 1 && H % (ks * 128) != 0) --ks;
  return ks < 1 ? 1 : ks;
}
// Tile and hidden split of the tiled GEMM.  Row tiles of 256 (8 waves, one
// workgroup per CU) or 128 (4 waves, two per CU); products without row
// statistics may split the hidden dimension into KS <= 8 slices of whole
// 128-wide chunks (lengths differ by at most one chunk), each writing an fp32
// partial that its consumer sums.  The plan minimises a measured cost model:
// rounds of workgroup slots x chunks per slice x the time of one chunk on a
// full CU (3.9 us at TM 256, 4.5 us at TM 128: two 128-row tiles per CU), plus
// writing and reading each partial beyond the first at about 4 TB/s.
struct GemmPlan {
  int tm, ks;
};
inline GemmPlan gemm_plan(int rows, int V, int H, bool stats) {
  const int C = H / 128;
  const long nn = lm_gemm_ntiles(V);
  GemmPlan best{256, 1};
  double best_us = 1e300;
  for (int tm : {256, 128}) {
    const long tiles = (rows + tm - 1) / tm * nn, slots = tm == 128 ? 512 : 256;
    const double chunk_us = tm == 128 ? 4.5 : 3.9;
    for (int ks = 1; ks <= (stats ? 1 : 8) && ks <= C; ++ks) {
      const double us = (double)((tiles * ks + slots - 1) / slots) * ((C + ks - 1) / ks) * chunk_us +
                        (ks - 1) * (double)rows * V * 8.0 / 4e6;
      if (us < best_us) { best = GemmPlan{tm, ks}; best_us = us; }
    }
  }
  return best;
}
inline int lm_gemm_ksplit(int rows, int V, int H) {
  return rows < kGemmMinRows ? 1 : gemm_plan(rows, V, H, false).ks;
}
inline size_t lm_rec_floats(int rows, int V) { return (size_t)rows * lm_gemm_ntiles(V) * 4; }
inline size_t lm_ws_bytes(int rows, int V, int H) {
  const int k1 = lm_ksplit(rows, V, H), k2 = lm_gemm_ksplit(rows, V, H);
  const int ks = k1 > k2 ? k1 : k2;
  return (lm_rec_floats(rows, V) + (ks > 1 ? (size_t)ks * rows * V : 0)) * sizeof(float);
}
hipError_t launch_lmhead(int rows, int hidden, int V, int dtype, int w_layout, const void* x, const void* w,
                         float T, float* logits, float* row_stats, int32_t* row_argmax,
                         float* probs, float* ws_part, int32_t* status, hipStream_t st);
// Output row of product row m: (m / grp) * gstride + off + m % grp, so that
// rows of a few consecutive tree slots per request land in a [B, S, V] buffer.
struct RowMap {
  int grp, gstride, off;
};
__host__ __device__ inline int map_row(int m, RowMap rm) {
  return m < rm.grp ? rm.off + m : (m / rm.grp) * rm.gstride + rm.off + m % rm.grp;  // no division in one group
}
// The same with an output row map; row_stats == nullptr skips the statistics
// (a plain product X W^T), and probs must then be null as well.
hipError_t launch_lmhead_map(int rows, int hidden, int V, int dtype, int w_layout, const void* x, const void* w,
                             float T, float* logits, float* row_stats, int32_t* row_argmax, float* probs,
                             float* ws_part, int32_t* status, RowMap rm, hipStream_t st);
hipError_t launch_lmhead_impl(int rows, int hidden, int V, int dtype, int w_layout, const void* x, const void* w,
                              float T, float* logits, float* row_stats, int32_t* row_argmax, float* probs,
                              float* ws_part, int32_t* status, RowMap rm, int* defer_ks, uint16_t* z16, float* bmax,
                              hipStream_t st);
// Compact rows instead of fp32 logits (bf16 only): z16 [rows, V] fp16 offsets
// from the 128-column block maxima bmax [rows, ceil(V / 128)]; row statistics
// of the decoded values and the exact argmax.
hipError_t launch_lmhead_compact(int rows, int hidden, int V, int w_layout, const void* x, const void* w, float T,
                                 uint16_t* z16, float* bmax, float* row_stats, int32_t* row_argmax, float* ws_part,
                                 int32_t* status, hipStream_t st);
// A plain bf16 product out = X W^T (W packed) whose hidden-split slices, if
// any, are left unsummed: the result is sum over kz < ks of src[kz * slice + r * V + n]
// (ks = 1: src = out).  The caller's next kernel sums them.
struct ProductOut {
  int ks;
  const float* src;
  size_t slice;
};
hipError_t launch_product(int rows, int hidden, int V, const void* x, const void* w_packed, float* out, float* ws_part,
                          int32_t* status, ProductOut* po, hipStream_t st);
size_t lm_packed_bytes(int V, int hidden);
hipError_t launch_pack_lmhead(int V, int hidden, const void* w, void* wp, hipStream_t st);
// Lossless 12-bit form of the packed weight (EAGLE_W_ZPACKED): byte offsets of
// its three areas for (V, hidden) and its size.
struct ZLayout {
  size_t nfrag, slot_off, raw_off, bytes;
};
__host__ __device__ inline ZLayout lm_zlayout(int V, int hidden) {
  ZLayout z;
  z.nfrag = (size_t)((V + 63) / 64) * (hidden / 8);
  z.slot_off = (z.nfrag + 16 + 255) / 256 * 256;
  z.raw_off = (z.slot_off + z.nfrag * 768 + 16 + 255) / 256 * 256;
  z.bytes = z.raw_off + z.nfrag * 1024;
  return z;
}
hipError_t launch_zpack_lmhead(int V, int hidden, const void* w, void* wz, int32_t* raw_count, hipStream_t st);

// ---- sampling warps (k_warp.hip) ----
int warp_mass_shift(int V);
hipError_t launch_warp(int rows, int V, int top_k, float top_p, int min_keep, float T, const float* z, float* stats,
                       uint32_t* bound, int32_t* status, hipStream_t st);
// The same on `rows` rows picked by a row map: workgroup i warps row
// map_row(i, rm) of z, stats and bound.
hipError_t launch_warp_map(int rows, int V, int top_k, float top_p, int min_keep, float T, const float* z,
                           float* stats, uint32_t* bound, int32_t* status, RowMap rm, hipStream_t st);

// ---- synthetic EAGLE draft head (k_draft.hip) ----
// Byte offsets in the draft workspace: per-round slot state (kept across the
// depths of a round) and per-depth scratch sized for B * k frontier rows.
struct DraftLayout {
  size_t slot_k, slot_v, slot_feat, slot_mask;
  size_t idx, x0, u, n1, qkv, qc, og, h, n2, gu, mm, y, xa, gemm, attn, total;
};
DraftLayout draft_layout(int B, int S, int k, int V, int H, int hq, int hkv, int dh, int I, int max_prefix);
struct DraftArgs {
  int B, S, k, V, H, hq, hkv, dh, I, max_prefix, depth;
  float scale;
  eagle_draft_weights w;
  const int32_t* root;
  const void* root_feat;
  const void *k_prefix, *v_prefix;
  const int32_t* prefix_len;
  const int32_t *pool_tok, *slot_src;
  float* rows;
  void* ws;
  DraftLayout lay;
  int32_t* status;
};
hipError_t launch_draft_forward(const DraftArgs& a, hipStream_t st);

// ---- acceptance (k_accept.hip) ----
constexpr int kAccMaxGroup = 64;         // workgroups per request in the cooperative walk
// Per-request mailbox of the walk.  Mailbox b sits b + 1 mailboxes before the
// 256-byte-aligned end of the workspace, a place fixed by the workspace size
// alone, so calls with different batches on one workspace find the same words.
struct Mailbox {
  uint64_t bank[2][kAccMaxGroup];
  uint64_t result;
  uint32_t epoch;
  uint32_t pad[13];
};
inline size_t accept_mail_bytes(int B) { return (size_t)B * sizeof(Mailbox); }
hipError_t launch_accept(int B, int N, int V, int D, int k, int S, float T, const int32_t* node_tok,
                         const int32_t* node_parent, const int32_t* node_slot,
                         const int32_t* pool_tok, const int32_t* pool_flat, const float* tlog,
                         const float* tstats, const int32_t* targmax, const float* dlog,
                         const float* sstats, const uint32_t* tbound, const uint32_t* dbound,
                         const uint16_t* thp, const float* tbm,  // compact target rows (null: tlog)
                         const float* uniforms, void* mail, int32_t* accept_len,
                         int32_t* accept_path, int32_t* committed, int32_t* n_committed,
                         int32_t* near_tie, int32_t* status, hipStream_t st);

}  // namespace eagle
