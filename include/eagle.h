/*
 * eagle.h — C ABI of libeagle: one EAGLE-style draft-tree round on an MI355X
 * (gfx950).
 *
 * Five stream-ordered entry points run the round on device memory:
 *
 *   eagle_expand_tree      draft rows -> dynamic draft tree (expand, rerank, flatten)
 *   eagle_build_tree_mask  parent links -> ancestor-only attention mask + positions
 *   eagle_tree_attention   one tree-masked attention pass over prefix KV + tree
 *   eagle_lmhead_softmax   LM-head logits + per-row softmax statistics + argmax
 *   eagle_verify_accept    recursive speculative sampling down the tree
 *
 * plus workspace helpers and row-gather helpers, and the steps around the
 * round:
 *
 *   eagle_sampling_warp (+ the _warped variants of expand and accept)
 *                          top-k / nucleus applied to both distributions
 *   eagle_commit_accepted  the accepted path appended to the prefix cache
 *   eagle_draft_forward, eagle_expand_depth(_warped), eagle_expand_finish
 *                          the tree drafted depth by depth by a synthetic
 *                          EAGLE draft head
 *
 * Conventions (all entry points):
 *   - Every pointer argument named as a tensor is DEVICE memory owned by the
 *     caller; the library never allocates, frees or retains it.  Parameter
 *     structs (eagle_tree_params) are HOST memory, read during the call only.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).  Nothing is synchronised.
 *   - Tensors are dense, row-major, with the shapes given below; int32 ids,
 *     fp32 logits and statistics, activations and weights in the dtype named
 *     by an `eagle_dtype` argument (bf16 = raw 16-bit patterns).
 *   - Return value: EAGLE_OK (0) or a negative EAGLE_ERR_* code.  Argument
 *     checks happen on the host before anything is enqueued; a call that
 *     returns an error has enqueued nothing.
 *   - Data-dependent conditions found on the device (a token id out of range,
 *     a non-finite logit, ...) do not abort: they OR EAGLE_STATUS_* bits into
 *     *dev_status (an optional device int32, may be NULL), to be read by the
 *     caller after synchronising.
 *   - Workspace: `ws` is caller-provided device scratch of `ws_bytes` bytes,
 *     sized with eagle_workspace_size(...) for the largest round it serves.
 *     Before its first use it must be initialised once with
 *     eagle_workspace_init: the acceptance walk keeps per-request mailboxes
 *     that persist across calls, mailbox b at b + 1 mailboxes before the
 *     256-byte-aligned end of the buffer.  Their place depends on ws_bytes
 *     only, so every call on one buffer must pass the same ws_bytes (after a
 *     change, initialise again); a smaller batch uses a subset of the same
 *     mailboxes.  Calls that share one workspace must be ordered (same
 *     stream); calls on different streams need different workspaces.
 *   - Calls are deterministic: identical inputs give bit-identical outputs.
 *   - Tracing: with EAGLE_ROCTX set (and not "0") in the environment, every
 *     entry point that enqueues work pushes a roctx range named after itself
 *     (the library loads ROCm's roctx library on the first such call);
 *     otherwise no tracing library is loaded.
 *
 * Sources of the method (cited by page title and section):
 *   [E1] "EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
 *        (papercache.org notes).
 *   [E2] "EAGLE-2: Faster Inference of Language Models with Dynamic Draft
 *        Trees" (tom-jerr.github.io notes).
 *   [HW] "LLM 推测性解码原理解读" (hubwiz.com blog on speculative decoding and
 *        EAGLE-3).
 *
 * Symbols: B batch, V vocab, D depth (draft levels), k children per expanded
 * node, m selected draft nodes, N = m + 1 tree nodes (flat index 0 = root,
 * the last committed token), S = 1 + (D-1)k expanded slots, P = S*k pool
 * entries (every child ever created), W = ceil(N/64) mask words.
 */
#ifndef EAGLE_H
#define EAGLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes -------------------------------------------------------- */
#define EAGLE_OK             0
#define EAGLE_ERR_NULL      -1  /* a required pointer is NULL                    */
#define EAGLE_ERR_SHAPE     -2  /* a size is out of range or inconsistent        */
#define EAGLE_ERR_DTYPE     -3  /* unsupported dtype for this entry point/shape  */
#define EAGLE_ERR_WORKSPACE -4  /* workspace missing or smaller than required    */
#define EAGLE_ERR_LAUNCH    -5  /* the HIP runtime refused a launch              */
#define EAGLE_ERR_ALIGN     -6  /* a tensor pointer is not 16-byte aligned       */
#define EAGLE_ERR_TOO_LARGE -7  /* sizes beyond the no-allocation scratch limit  */

/* ---- device status bits (OR-ed into *dev_status) ------------------------- */
#define EAGLE_STATUS_TOKEN_RANGE   0x1  /* an input token id was outside [0, V)          */
#define EAGLE_STATUS_NONFINITE     0x2  /* a logit was NaN/Inf (treated as -inf)         */
#define EAGLE_STATUS_ZERO_RESIDUAL 0x4  /* residual mass 0 after a rejection: P kept     */
#define EAGLE_STATUS_TOPK_RESCAN   0x8  /* child selection re-scanned a row (info only)  */
#define EAGLE_STATUS_BAD_TREE      0x10 /* parent links not a valid flattened tree       */
#define EAGLE_STATUS_CAND_OVERFLOW 0x20 /* child re-scan candidate list overflowed       */
#define EAGLE_STATUS_SYNC_TIMEOUT  0x40 /* a walk workgroup gave up waiting for its group */
#define EAGLE_STATUS_CACHE_FULL    0x80 /* a prefix cache had no room for the commit     */
#define EAGLE_STATUS_LDS_INDEX     0x100 /* debug library only: an LDS index of the tree
                                            assembly or the walk left its array (clamped) */

/* ---- limits -------------------------------------------------------------- */
#define EAGLE_MAX_TOPK   16
#define EAGLE_MAX_DEPTH  16
#define EAGLE_MAX_NODES  256        /* N = m + 1 */
#define EAGLE_MAX_POOL   4096       /* P = S * k */
#define EAGLE_MAX_VOCAB  (1 << 19)

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;

/* Layout of the LM-head weight.  ROWMAJOR: [vocab, hidden] as given.
 * PACKED: produced once by eagle_lmhead_pack_weight (bf16 only): every group
 * of 64 vocab rows becomes one contiguous stream ordered exactly as the MFMA
 * operand loads consume it, so each wave reads 1 KB contiguous per load. */
typedef enum { EAGLE_W_ROWMAJOR = 0, EAGLE_W_PACKED = 1, EAGLE_W_ZPACKED = 2 } eagle_w_layout;
/* ZPACKED: the PACKED order stored losslessly in 12 bits per weight where
 * possible, made once by eagle_lmhead_zpack_weight (bf16 only).  The packed
 * layout's unit is a fragment of 512 weights (64 lanes x 8 consecutive hidden
 * values).  A bf16 weight is s | e (8 bits) | f (7 bits); its low byte
 * (e & 1, f) is kept as is, and its high byte (s, e >> 1) becomes a 4-bit code
 * (s, then e >> 1 minus a per-fragment base, 0..7).  A fragment whose e >> 1
 * values span more than 8 keeps its high bytes whole ("raw").  Decoding
 * restores every bit, so products equal those of the PACKED layout exactly;
 * the streaming kernel reads 768 bytes per coded fragment instead of 1024.
 * Byte layout for F fragments (F = ceil(vocab / 64) * hidden / 8):
 *   [0, F)                     one byte per fragment: bit 7 raw, bits 0..6 base;
 *   slot area (256-aligned)    768 bytes per fragment, lane l's 12 at 12 l:
 *                              the low bytes of weights 0..3, of 4..7, then the
 *                              codes (weight i < 4 in the low nibble of byte i,
 *                              weight i >= 4 in the high nibble of byte i - 4);
 *   raw area (256-aligned)     1024 bytes per fragment, lane l's 16 at 16 l: the
 *                              low bytes of weights 0..3, of 4..7, the high
 *                              bytes of 0..3, of 4..7 (written for raw
 *                              fragments only).
 * The raw area is sized for every fragment to be raw, so the form takes about
 * 1.75 times the PACKED bytes in memory; a launch reads only each fragment's
 * own form.  Only eagle_lmhead_softmax and eagle_lmhead_softmax_compact with
 * at most EAGLE_ZPACK_MAX_ROWS rows and hidden <= 16384 read this layout. */
#define EAGLE_ZPACK_MAX_ROWS 192

/* Parameters of one round (host struct).
 *   temperature > 0: sampling at temperature T (both the target and the draft
 *   distributions are softmax(logits / T), [HW] section 2);
 *   temperature == 0: greedy (children = top-k logits, acceptance = argmax
 *   match, [E1] appendix A.1; tree values then use confidences at T = 1).
 *   seed, round_id: key and counter words of the Philox4x32-10 draws that
 *   sample non-greedy children. */
typedef struct eagle_tree_params {
    int32_t  batch;        /* B >= 1                         */
    int32_t  vocab;        /* V, k <= V <= EAGLE_MAX_VOCAB   */
    int32_t  depth;        /* D, 1..EAGLE_MAX_DEPTH          */
    int32_t  topk;         /* k, 1..EAGLE_MAX_TOPK           */
    int32_t  m;            /* 1 <= m <= P, m + 1 <= EAGLE_MAX_NODES */
    float    temperature;  /* T >= 0                         */
    uint64_t seed;
    uint64_t round_id;
} eagle_tree_params;

/* Bytes of workspace that every entry point below needs for a round of these
 * sizes (the maximum over the entry points; the same buffer may serve all of
 * them in stream order).  hq/hkv/head_dim/max_prefix describe the verify
 * attention, hidden the LM-head input width.  Returns 0 on invalid sizes. */
size_t eagle_workspace_size(const eagle_tree_params* p, int32_t hq, int32_t hkv,
                            int32_t head_dim, int32_t max_prefix, int32_t hidden);

/* Zero the whole workspace (enqueued on `stream` as a fill kernel, not a
 * memset).  Call once after allocating a workspace. */
int eagle_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Dynamic draft-tree expansion, rerank and flattening for every request.
 * Source: [E2] "Expanding the Draft Tree" (value V_i = product of draft
 * confidences on the root path; expand the current layer's top-k by value),
 * "Rerank draft tokens" (keep the top-m by value, shallower first at equal
 * value, giving a connected tree), "Tree Attention Mask" (flatten);
 * [E1] appendix A.1 (greedy: top-k children; otherwise k sampled children).
 *
 * In:  draft_logits [B, S, V] fp32: row s of request b holds the draft logits
 *        at the node expanded as slot s.  Slot 0 is the root; the frontier
 *        node of rank i at depth d (1 <= d < D) is slot 1 + (d-1)k + i.
 *      root_token [B] int32.
 * Out: node_tok, node_parent (-1 for the root), node_depth, node_sib (rank
 *        among its parent's children in sampling order, -1 root), node_slot
 *        (slot the node was expanded as, -1 if never expanded): [B, N] int32;
 *      node_value, node_q: [B, N] fp32 (path value, own confidence; 1 at root);
 *      pool_tok [B, S, k] int32: children of each slot in sampling order;
 *      pool_q [B, S, k] fp32: their confidences;
 *      pool_flat [B, S, k] int32: flat index of each child or -1 if pruned;
 *      slot_src [B, S] int32: pool index (s' * k + j) of the node slot s
 *        expands (-1 for slot 0);
 *      slot_stats [B, S, 2] fp32: (max_v t_v, sum_v exp(t_v - max)) of each
 *        slot row, t = logits / T' (T' = T, or 1 when greedy).
 * Flat order: root, then by (depth, parent's flat index, sibling rank).
 * Non-greedy children are the k largest Gumbel keys fp32(z_v / T) + g_v,
 * g = -ln(-ln u_v), u_v from Philox4x32-10 with counter (v >> 2, s, b,
 * round_id mod 2^32), key (seed low, seed high), output word v & 3, mapped to
 * (2 * (x >> 9) + 1) * 2^-24; keys are compared in fp64, ties to the lower id.
 * Status: TOKEN_RANGE (root id), NONFINITE, TOPK_RESCAN, CAND_OVERFLOW. */
int eagle_expand_tree(const eagle_tree_params* p, const float* draft_logits,
                      const int32_t* root_token,
                      int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                      int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                      int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                      float* slot_stats, void* ws, size_t ws_bytes, int32_t* dev_status,
                      void* stream);

/* eagle_expand_tree with the draft rows warped (top-k / nucleus) before the
 * children are drawn (T > 0; greedy ignores it).
 * Source: [HW] section 2 (both distributions are adjusted the same way
 * before the test).
 * draft_bound [B * S, 2] uint32: per slot row, the kept prefix written by
 * eagle_sampling_warp on draft_logits (same temperature, min_keep = k);
 * NULL is no warp.  Tokens the warp drops get t = -inf: they are never
 * children and leave slot_stats, which become the warped softmax's (M, S),
 * and pool_q, the warped confidences.  Everything else as eagle_expand_tree. */
int eagle_expand_tree_warped(const eagle_tree_params* p, const float* draft_logits, const uint32_t* draft_bound,
                             const int32_t* root_token, int32_t* node_tok, int32_t* node_parent,
                             int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value,
                             float* node_q, int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                             float* slot_stats, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* eagle_expand_tree followed by eagle_build_tree_mask in one call: the
 * assembly step, which already holds the flattened tree, also writes the
 * ancestor-only mask [B, N, ceil(N/64)] and the positions [B, N]
 * (prefix_len[b] + depth), bit for bit what eagle_build_tree_mask writes for
 * the tree it returns.  Source: [E2] "Tree Attention Mask" (flatten the tree
 * and mask it to ancestors).  One launch fewer per round.  No sampling warp.
 * Everything else as eagle_expand_tree. */
int eagle_expand_tree_masked(const eagle_tree_params* p, const float* draft_logits, const int32_t* root_token,
                             const int32_t* prefix_len, int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                             int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                             int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                             float* slot_stats, uint64_t* mask, int32_t* pos, void* ws, size_t ws_bytes,
                             int32_t* dev_status, void* stream);

/* eagle_expand_tree for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no `ws` argument; the expansion's candidate records go to a
 * static device array of EAGLE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on every GPU it runs on until the process ends.  The call itself
 * allocates nothing.  Limit: B * S * ceil(V / 4096) * 4 * (2 + 2 (k + 2)) * 4
 * bytes of records must fit (the 8B shape: 0.95 MB per request, so up to 70
 * requests); larger sizes return EAGLE_ERR_TOO_LARGE before any launch.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads without ordering) race and must be
 * serialised by the caller.  Outputs, status and errors as eagle_expand_tree
 * (no sampling warp); the results are bit-identical to it. */
#define EAGLE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int eagle_expand_tree_noalloc(const eagle_tree_params* p, const float* draft_logits,
                              const int32_t* root_token,
                              int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                              int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                              int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                              float* slot_stats, int32_t* dev_status, void* stream);

/* ---- static (EAGLE-1) draft trees --------------------------------------
 * Source: [E1] appendix A.1 (the draft tree has a fixed shape from which each
 * node's child count k is read, k = 4 at the root; greedy drafting takes the
 * top-k tokens as children, sampling drafts k tokens; 5 draft passes fill
 * it) and [E1] section 4.3.1 / ablation (tree against chain drafts).
 *
 * A shape is given by its parent array `shape_parent` [n] (HOST memory, read
 * during the call): node 0 is the root (parent -1), 0 <= parent[i] < i, at most
 * EAGLE_MAX_TOPK children per node and depth at most EAGLE_MAX_DEPTH; siblings
 * rank by flat index.  The nodes with children are the slots, numbered in flat
 * order; slot s has k_s children and its draft row is row s of
 * draft_logits [B, n_slots, V].  The flattened tree IS the shape: node i of
 * every request is shape node i (its mask is the shape's ancestor relation). */

/* Slots, depth and largest child count of a shape, and each slot's child
 * count into slot_k [n_slots] (host, nullable).  EAGLE_ERR_SHAPE if the shape
 * is not a valid flattened tree. */
int eagle_static_tree_info(int32_t n, const int32_t* shape_parent, int32_t* n_slots, int32_t* depth,
                           int32_t* kmax, int32_t* slot_k);

/* eagle_workspace_size for a round on a static shape (the expansion's records
 * are sized for its n_slots slots and largest child count). */
size_t eagle_static_workspace_size(const eagle_tree_params* p, int32_t n, const int32_t* shape_parent, int32_t hq,
                                   int32_t hkv, int32_t head_dim, int32_t max_prefix, int32_t hidden);

/* Fill a static shape for every request.  p->topk must be the shape's largest
 * child count kmax, p->depth its depth, p->m = n - 1 (else EAGLE_ERR_SHAPE).
 * Slot s's children are the first k_s of its row's sampling order: the top
 * k_s logits (greedy) or the k_s largest Gumbel keys, with the same keys,
 * Philox counters (slot index s) and tie rules as eagle_expand_tree.
 * Out: node_* [B, n] as eagle_expand_tree (node_value = fp32 product of the
 *        confidences on the root path, node_slot = the node's slot or -1);
 *      pool_tok, pool_q, pool_flat [B, n_slots, kmax]: slot s's draws in
 *        sampling order in entries 0..k_s-1, -1 / 0 / -1 past them;
 *      slot_src [B, n_slots] (pool index of the node each slot expands, -1
 *        for the root), slot_stats [B, n_slots, 2].
 * Workspace: eagle_static_workspace_size.  Status: TOKEN_RANGE, NONFINITE,
 * TOPK_RESCAN, CAND_OVERFLOW. */
int eagle_expand_static(const eagle_tree_params* p, int32_t n, const int32_t* shape_parent,
                        const float* draft_logits, const int32_t* root_token, int32_t* node_tok, int32_t* node_parent,
                        int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                        int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src, float* slot_stats,
                        void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* eagle_verify_accept on a static tree of n_slots slots (p as for
 * eagle_expand_static; uniforms [B, n, kmax + 1], the last column for the
 * residual or bonus draw).  A slot's candidates are its k_s draws: the walk
 * tries them in sampling order and, when all k_s are rejected, draws from the
 * residual.  No sampling warp. */
int eagle_verify_accept_static(const eagle_tree_params* p, int32_t n_slots, const int32_t* node_tok,
                               const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                               const int32_t* pool_flat, const float* target_logits, const float* target_stats,
                               const int32_t* target_argmax, const float* draft_logits, const float* slot_stats,
                               const float* uniforms, int32_t* accept_len, int32_t* accept_path, int32_t* committed,
                               int32_t* n_committed, int32_t* near_tie, void* ws, size_t ws_bytes,
                               int32_t* dev_status, void* stream);

/* Ancestor-only tree attention mask and positions.
 * Source: [E2] "Tree Attention Mask" (each token sees only its ancestors,
 * never another branch); [HW] section 5.
 * In:  node_parent [B, n] int32 (flattened order: parent index < own index,
 *        -1 for node 0), node_depth [B, n] int32, prefix_len [B] int32.
 * Out: mask [B, n, W] uint64: bit j of row i is set iff j == i or j is an
 *        ancestor of i (bit j % 64 of word j / 64);
 *      pos [B, n] int32 = prefix_len[b] + depth.
 * Status: BAD_TREE if a parent index is not in [0, i) (row i then sees itself only). */
int eagle_build_tree_mask(int32_t batch, int32_t n, const int32_t* node_parent,
                          const int32_t* node_depth, const int32_t* prefix_len,
                          uint64_t* mask, int32_t* pos, int32_t* dev_status, void* stream);

/* One tree-masked attention pass of the tree queries over the prefix KV and
 * the tree itself.  Source: [E1] sections 3.1/3.3 (tree attention scores the
 * whole draft tree in one target forward); [HW] section 5 (every root-to-leaf
 * path is scored as if it were an independent sequence).
 * In:  q [B, n, hq, head_dim]; k_prefix, v_prefix [B, hkv, max_prefix, head_dim]
 *        (first prefix_len[b] positions used); prefix_len [B] int32 (0..max_prefix);
 *      k_tree, v_tree [B, n, hkv, head_dim]; mask [B, n, W] uint64 as above;
 *      scale: score = scale * (q . k).  Query head h reads kv head h / (hq / hkv).
 * Out: out [B, n, hq, head_dim], same dtype as q.
 * dtype: EAGLE_BF16 (head_dim 64 or 128, MFMA) or EAGLE_F32 (head_dim <= 128).
 * Softmax and accumulation are fp32. */
int eagle_tree_attention(int32_t batch, int32_t n, int32_t hq, int32_t hkv, int32_t head_dim,
                         int32_t max_prefix, int32_t dtype, const void* q,
                         const void* k_prefix, const void* v_prefix, const int32_t* prefix_len,
                         const void* k_tree, const void* v_tree, const uint64_t* mask,
                         float scale, void* out, void* ws, size_t ws_bytes,
                         int32_t* dev_status, void* stream);

/* LM-head logits at every row and the statistics of softmax(logits / T').
 * Source: [E1] background A3: p_{j+1} = LMHead(f_j) at every position.
 * In:  x [rows, hidden], w (dtype) in layout w_layout: [vocab, hidden]
 *        row-major, or EAGLE_W_PACKED (bf16, from eagle_lmhead_pack_weight);
 *      temperature T >= 0 (T' = T, or 1 when T == 0).
 * Out: logits [rows, vocab] fp32 (= x . w^T, fp32 accumulation);
 *      row_stats [rows, 2] fp32: (M, S) = (max_v z_v / T', sum_v exp(z_v/T' - M));
 *      row_argmax [rows] int32: argmax_v z_v, lowest id on ties;
 *      probs [rows, vocab] fp32 or NULL: exp(z/T' - M) / S when non-NULL.
 * Status: NONFINITE (a NaN/Inf logit stays as computed in `logits` and counts
 * as -inf in row_stats and row_argmax; a row with no finite logit gets
 * M = -inf and argmax 0).
 * dtype EAGLE_BF16 needs hidden % 128 == 0; fp32 needs hidden <= 16384. */
int eagle_lmhead_softmax(int32_t rows, int32_t hidden, int32_t vocab, int32_t dtype,
                         const void* x, const void* w, int32_t w_layout, float temperature,
                         float* logits, float* row_stats, int32_t* row_argmax, float* probs,
                         void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* Bytes of the packed LM-head weight for (vocab, hidden) in bf16 (0 if the
 * shape or dtype has no packed form). */
size_t eagle_lmhead_packed_bytes(int32_t vocab, int32_t hidden, int32_t dtype);

/* eagle_lmhead_softmax without fp32 logit rows (bf16 only): every row is
 * stored compact, 2 bytes per logit.  Source: [E1] A3 and 3.3 (one verify
 * pass gives the target distribution at every tree node; the walk reads it at
 * the candidates and, after a rejection, over the whole vocabulary).
 * Out: target_z16 [rows, vocab] (fp16 bit patterns, 8-byte aligned): logit v
 *        as fp16(z_v - m), m the largest finite logit of its 128-column block
 *        (columns 128 b .. 128 b + 127), rounded to nearest even; -inf for a
 *        non-finite logit or a block without a finite one;
 *      block_max [rows, ceil(vocab / 128)] fp32: the block maxima m;
 *      row_stats [rows, 2]: (max, sum exp) of the DECODED row
 *        z~ = fp32(m + fp32(offset)) at T' (the block maxima decode exactly, so
 *        the max equals eagle_lmhead_softmax's);
 *      row_argmax [rows]: the first column holding the row's largest logit,
 *        exactly as eagle_lmhead_softmax (computed from the fp32 logits).
 * For tokens whose probability is at least 1e-6 of the row's largest, the
 * decoded row's probabilities are within 1.4% of the fp32 row's.  Everything
 * else (workspace, status) as eagle_lmhead_softmax. */
int eagle_lmhead_softmax_compact(int32_t rows, int32_t hidden, int32_t vocab, const void* x, const void* w,
                                 int32_t w_layout, float temperature, uint16_t* target_z16, float* block_max,
                                 float* row_stats, int32_t* row_argmax, void* ws, size_t ws_bytes,
                                 int32_t* dev_status, void* stream);

/* Pack a row-major bf16 LM-head weight w [vocab, hidden] into w_packed
 * (eagle_lmhead_packed_bytes bytes, 16-byte aligned; rows past vocab are
 * zero-filled).  A one-time layout transform done when weights are loaded. */
int eagle_lmhead_pack_weight(int32_t vocab, int32_t hidden, int32_t dtype, const void* w,
                             void* w_packed, void* stream);

/* Bytes of the z-packed LM-head weight (EAGLE_W_ZPACKED) for a bf16
 * (vocab, hidden) shape (0 if the shape has no packed form). */
size_t eagle_lmhead_zpack_bytes(int32_t vocab, int32_t hidden);

/* Write the z-packed form of a row-major bf16 LM-head weight w [vocab, hidden]
 * into w_z (eagle_lmhead_zpack_bytes bytes, 256-byte aligned; rows past vocab
 * are zero).  A one-time layout transform done when weights are loaded, as
 * eagle_lmhead_pack_weight; asynchronous on `stream`.  If raw_fragments is
 * non-NULL the call also counts the raw fragments into *raw_fragments (device
 * int32, set to 0 by the call before counting), so a caller can report how
 * many fragments the 12-bit form covers. */
int eagle_lmhead_zpack_weight(int32_t vocab, int32_t hidden, const void* w, void* w_z,
                              int32_t* raw_fragments, void* stream);

/* Recursive speculative sampling down each request's tree.
 * Source: [E1] background A3 (accept x with probability min(1, p(x)/q(x));
 * on rejection draw from norm(max(0, p - q))), section 3.3 and appendix A.2
 * (at each tree node try the k candidates in turn against the adjusted
 * distribution; draw from it only when all are rejected); [HW] section 1
 * (bonus token when the walk ends at a leaf; at least 1 and at most
 * accepted + 1 committed tokens); greedy ([E1] A.1): follow the child equal
 * to the target argmax.
 * Candidates of node u are all k sampled children of its slot, in sampling
 * order, including pruned ones; accepting a pruned child commits it and ends
 * the walk.  A pool row's candidate list ends at its first negative entry
 * (a static tree's slot with fewer than k draws; see eagle_expand_static).  After rejecting x_j the draft law loses x_j and is renormalised
 * (draws without replacement).  Trial j at node u uses uniforms[b, u, j]; the
 * final draw (residual or bonus) uses uniforms[b, u, k] by inverse CDF in
 * token-id order (first token whose cumulative mass exceeds u * total).
 * In:  tree arrays from eagle_expand_tree (node_tok, node_parent, node_slot
 *        [B, N]; pool_tok, pool_flat [B, S, k]);
 *      target_logits [B*N, V] fp32 (row b*N + u = verify logits at flat node u),
 *      target_stats [B*N, 2] and target_argmax [B*N] from eagle_lmhead_softmax
 *        (argmax is read only when greedy);
 *      draft_logits [B, S, V] fp32 and slot_stats [B, S, 2] (as for expand);
 *      uniforms [B, N, k + 1] fp32 in [0, 1) (unused when greedy).
 * Out: accept_len [B] (accepted tree nodes), accept_path [B, D] (their flat
 *        indices, -1 padded), committed [B, D + 1] (committed tokens, -1
 *        padded), n_committed [B] = accept_len + 1, near_tie [B] (decisions
 *        whose uniform lay within 1e-6 of the deciding threshold).
 * Status: ZERO_RESIDUAL, TOKEN_RANGE. */
int eagle_verify_accept(const eagle_tree_params* p, const int32_t* node_tok,
                        const int32_t* node_parent, const int32_t* node_slot,
                        const int32_t* pool_tok, const int32_t* pool_flat,
                        const float* target_logits, const float* target_stats,
                        const int32_t* target_argmax, const float* draft_logits,
                        const float* slot_stats, const float* uniforms,
                        int32_t* accept_len, int32_t* accept_path, int32_t* committed,
                        int32_t* n_committed, int32_t* near_tie, void* ws, size_t ws_bytes,
                        int32_t* dev_status, void* stream);

/* eagle_verify_accept on compact target rows (eagle_lmhead_softmax_compact):
 * every target probability the walk uses (acceptance ratios, residual sums,
 * draws) is exp(z~/T' - M) / S of the decoded row z~ with the statistics of
 * that same row, so the walk samples exactly from the decoded distribution.
 * n_slots = 0: a dynamic tree (S = 1 + (D - 1) k); n_slots > 0: a static
 * tree of that many slots (eagle_expand_static).  No sampling warp.
 * Everything else as eagle_verify_accept. */
int eagle_verify_accept_compact(const eagle_tree_params* p, int32_t n_slots, const int32_t* node_tok,
                                const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                                const int32_t* pool_flat, const uint16_t* target_z16, const float* block_max,
                                const float* target_stats, const int32_t* target_argmax, const float* draft_logits,
                                const float* slot_stats, const float* uniforms, int32_t* accept_len,
                                int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
                                void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* eagle_verify_accept with both distributions warped (top-k / nucleus)
 * before the walk (T > 0; greedy ignores it).
 * Source: [HW] section 2 (temperature, top-k or nucleus sampling stays
 * exact when both distributions are adjusted the same way before the test).
 * target_bound [B * N, 2] and draft_bound [B * S, 2] uint32: the kept
 * prefixes eagle_sampling_warp wrote for the target rows and the draft slot
 * rows (same temperature and warp, min_keep = k); NULL is no warp for that
 * side.  target_stats and slot_stats must then be the warped (M, S) (from
 * eagle_sampling_warp and eagle_expand_tree_warped).  Tokens a warp drops
 * have probability 0 in every acceptance ratio, residual and draw.
 * Everything else as eagle_verify_accept. */
int eagle_verify_accept_warped(const eagle_tree_params* p, const uint32_t* target_bound, const uint32_t* draft_bound,
                               const int32_t* node_tok, const int32_t* node_parent, const int32_t* node_slot,
                               const int32_t* pool_tok, const int32_t* pool_flat, const float* target_logits,
                               const float* target_stats, const int32_t* target_argmax, const float* draft_logits,
                               const float* slot_stats, const float* uniforms, int32_t* accept_len,
                               int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
                               void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* Row gather: out[r, :] = table[idx[r], :] for r < n_rows (row_elems elements
 * of `dtype` per row).  The verify layer's tree queries/keys/values are
 * per-token rows looked up this way.  Ids outside [0, table_rows) give a zero
 * row and set TOKEN_RANGE. */
int eagle_gather_rows(int32_t n_rows, int32_t row_elems, int32_t dtype, const void* table,
                      int32_t table_rows, const int32_t* idx, void* out, int32_t* dev_status,
                      void* stream);

/* Several row gathers with one id list in one launch: for t < n_tables (at
 * most 4), outs[t][r, :] = tables[t][idx[r], :] for r < n_rows, with
 * row_elems[t] elements of `dtype` per row.  row_elems, tables and outs are
 * HOST arrays of n_tables entries (tables/outs holding device pointers); all
 * tables have table_rows rows.  The verify layer's tree queries, keys and
 * values (per-token rows, the synthetic stand-in for the target layer's
 * projections) are gathered this way in one launch.  Ids outside
 * [0, table_rows) give zero rows and set TOKEN_RANGE.  Errors as
 * eagle_gather_rows; n_tables outside [1, 4] is a SHAPE error. */
int eagle_gather_rows_multi(int32_t n_tables, int32_t n_rows, int32_t dtype, int32_t table_rows,
                            const int32_t* idx, const int32_t* row_elems, const void* const* tables,
                            void* const* outs, int32_t* dev_status, void* stream);

/* Sampling warp of logits rows: top-k, then nucleus (top-p), keeping at least
 * min_keep tokens.
 * Source: [HW] section 2 (with temperature, top-k or nucleus sampling the
 * output stays exact when both distributions are adjusted the same way
 * before the acceptance test).
 * Each row's tokens are ordered by (t desc, id asc), t = fp32(z / T') with
 * T' = T (T > 0) or 1.  top-k keeps the first min(top_k, vocab) (top_k = 0:
 * all); the nucleus keeps the shortest prefix of those whose mass
 * exp(t - max t) reaches top_p of their total, the crossing token included
 * (top_p = 1: no nucleus cut); at least min_keep are kept.
 * In:  logits [rows, vocab] fp32 (NaN/Inf count as -inf, status NONFINITE).
 * Out: row_stats [rows, 2] fp32: (M, S) = (max t, sum of exp(t - M) over the
 *        kept tokens), the statistics of the warped softmax;
 *      bound [rows, 2] uint32: (code_b, id_b) of the last kept token, code =
 *        the order-preserving unsigned image of fp32 t (bits ^ 0x80000000
 *        for t >= +0, ~bits for t < 0; -0 counts as +0).  Token v is kept iff
 *        code_v > code_b, or code_v == code_b and v <= id_b.
 * Needs 1 <= min_keep <= vocab, top_k == 0 or top_k >= min_keep,
 * 0 < top_p <= 1.  A tree with top-k k draws its k children without
 * replacement from the warped draft rows, so min_keep = k there.  Nucleus
 * masses are summed as exact fixed-point integers (2^(62 - ceil(log2 vocab))
 * per unit), so the cut is the same on every run. */
int eagle_sampling_warp(int32_t rows, int32_t vocab, int32_t top_k, float top_p, int32_t min_keep, float temperature,
                        const float* logits, float* row_stats, uint32_t* bound, int32_t* dev_status, void* stream);

/* Commit the accepted path to the context, after eagle_verify_accept.
 * Source: [E1] section 3.3 (the accepted tokens and their features are kept
 * for the next drafting round); [HW] section 5 (the longest consistent path
 * is committed, the other branches are discarded, and drafting resumes from
 * the longer context).
 * Committed rows of request b: the root (flat node 0, the last token of the
 * previous round, whose key/value the verify pass computed) and then
 * accept_path[b, 0 .. a-1] with a = accept_len[b].  The draft token drawn
 * after them (residual or bonus) has no key/value yet: it is the next
 * round's root.
 * In:  accept_len [B], accept_path [B, depth] as eagle_verify_accept writes
 *        them (entries past a are ignored);
 *      k_tree, v_tree [B, n, hkv, head_dim] (the verify pass's tree keys and
 *        values); x [B, n, hidden] (the LM-head inputs of the tree nodes).
 * In/out: k_prefix, v_prefix [B, hkv, max_prefix, head_dim] get row r of the
 *        path at position prefix_len[b] + r (other positions untouched);
 *      prefix_len [B] grows by a + 1.
 * Out: feat [B, depth + 1, hidden]: row r = x[b, node r] for r <= a, zero after.
 * Status: BAD_TREE (a outside [0, depth] or a path node outside [1, n): that
 *        request commits nothing and its features are zero); CACHE_FULL
 *        (prefix_len[b] + a + 1 > max_prefix: cache and length unchanged,
 *        features still written).
 * dtype EAGLE_BF16 or EAGLE_F32 for keys, values and features alike;
 * head_dim and hidden must span whole 16-byte units and every tensor pointer
 * must be 16-byte aligned (EAGLE_ERR_ALIGN).  The tree, cache and feature
 * buffers must not overlap.  depth <= EAGLE_MAX_DEPTH, n <= EAGLE_MAX_NODES;
 * batch 0 is a no-op. */
int eagle_commit_accepted(int32_t batch, int32_t n, int32_t hkv, int32_t head_dim, int32_t max_prefix,
                          int32_t hidden, int32_t depth, int32_t dtype, const int32_t* accept_len,
                          const int32_t* accept_path, const void* k_tree, const void* v_tree, const void* x,
                          void* k_prefix, void* v_prefix, int32_t* prefix_len, void* feat, int32_t* dev_status,
                          void* stream);

/* ---- per-depth drafting with a synthetic EAGLE draft head ------------------
 * [E1] section 3.1, [E2] "Expanding the Draft Tree", [HW] EAGLE-3 inference
 * pipeline: the tree is drafted one depth at a time.  Depth 0 drafts the root
 * (slot 0); depth d >= 1 drafts the k frontier nodes the expansion picked,
 * at slots 1 + (d-1)k .. dk.  Per depth, in this order:
 *   eagle_draft_forward  the head's forward for that depth's frontier nodes,
 *                        writing their draft rows at their slots;
 *   eagle_expand_depth   their children (as eagle_expand_tree picks them from
 *                        the same rows) and, below depth D-1, the next
 *                        depth's frontier (slot_src of its slots);
 * and after depth D-1 eagle_expand_finish reranks and flattens the pool
 * exactly as eagle_expand_tree does.  Given the same draft rows, the three
 * give eagle_expand_tree's outputs; with eagle_expand_depth_warped in place
 * of eagle_expand_depth, eagle_expand_tree_warped's (the depth's rows warped
 * as eagle_sampling_warp warps them).
 *
 * The head (random weights; the pages name its parts, not their internals):
 *   u = Wfc [f ; E[x]];  h = u + Wo attn(rms(u));
 *   a = h + Wd (silu(Wg rms(h)) * Wu rms(h));  draft row z = Wlm a,
 * rms(x) = x / sqrt(mean(x^2) + 1e-6), grouped-query attention with scale
 * 1/sqrt(head_dim) and no positional rotation over the draft's prefix K/V of
 * the request and the nodes of the node's own root path (itself included).
 * f = root_feat[b] for the root, else the head's output a at the parent; x =
 * the node's token.  Activations are bf16 at every matmul input (and a as fed
 * on), accumulation fp32. */
typedef struct {
    int32_t hidden;      /* H, a multiple of 128, at most 16384                */
    int32_t hq, hkv;     /* query / key-value heads, hq % hkv == 0              */
    int32_t head_dim;    /* 64 or 128; hq * head_dim a multiple of 128          */
    int32_t inter;       /* MLP width I, a multiple of 128                      */
    int32_t max_prefix;  /* position stride of the draft prefix K/V cache       */
} eagle_draft_dims;

/* Weights, DEVICE memory, bf16.  `embed` is row-major [vocab, H]; the others
 * are in the packed layout eagle_lmhead_pack_weight makes from a row-major
 * [out, in] matrix (out = its "vocab", in = its "hidden"). */
typedef struct {
    const void* embed;    /* [vocab, H] row-major                                 */
    const void* fc;       /* [H, 2H]: columns 0..H-1 take f, H..2H-1 take E[x]    */
    const void* qkv;      /* [(hq + 2 hkv) head_dim, H]: q rows, then k, then v   */
    const void* o;        /* [H, hq head_dim]                                     */
    const void* gate_up;  /* [2 I, H]: gate rows, then up rows                    */
    const void* down;     /* [H, I]                                               */
    const void* lm_head;  /* [vocab, H] (the target's LM head)                    */
    const void* lm_head_z;  /* the same in the z-packed form (EAGLE_W_ZPACKED, from
                               eagle_lmhead_zpack_weight), or NULL: read instead of
                               lm_head by depths of at most EAGLE_ZPACK_MAX_ROWS
                               rows; 256-byte aligned                           */
} eagle_draft_weights;

/* Bytes of the draft workspace for p's batch/vocab/depth/k (0 if invalid).  It
 * holds the per-slot state of a round (q/k/v, features and ancestor masks of
 * the drafted slots) and per-depth scratch; it needs no initialisation. */
size_t eagle_draft_workspace_size(const eagle_tree_params* p, const eagle_draft_dims* dims);

/* Where the drafting keeps each intermediate of its last eagle_draft_forward
 * call: byte offsets into the draft workspace, for inspection (staged checks
 * of one kernel at a time on the values the previous one wrote).  Writes
 * min(n, EAGLE_DRAFT_NBUF) offsets to `offsets` (host memory) in this order
 * and returns how many it wrote, or a negative EAGLE_ERR_* code:
 *   0 slot_k, 1 slot_v [B, S, hkv*dh] bf16 (per-slot keys/values),
 *   2 slot_feat [B, S, H] bf16 (each drafted slot's head output),
 *   3 slot_mask [B, S, ceil(S/64)] uint64 (each slot's root path),
 *   4 idx [R] int32 (b * S + slot of frontier row r; R = B at depth 0, else B*k),
 *   5 x0 [R, 2H] bf16 = [feature ; embedding],
 *   6 u [R, H] fp32 = x0 Wfc^T,      7 n1 [R, H] bf16 = rms-normalised u,
 *   8 (product scratch),             9 q [R, hq*dh] bf16 = n1 Wq^T,
 *  10 attention output [R, hq*dh] bf16,
 *  11 h [R, H] fp32 = u + attention Wo^T,   12 n2 [R, H] bf16 = rms(h),
 *  13 (product scratch),            14 m [R, I] bf16 = silu(n2 Wg^T) * (n2 Wu^T),
 *  15 (product scratch),            16 a [R, H] bf16 = h + m Wd^T.
 * The values stay until the next call on the workspace. */
#define EAGLE_DRAFT_NBUF 17
int eagle_draft_workspace_layout(const eagle_tree_params* p, const eagle_draft_dims* dims, size_t* offsets,
                                 int32_t n);

/* The draft head's forward for depth `depth` (0 <= depth < D).
 * In:  root_token [B] int32; root_feat [B, H] bf16 (the feature entering the
 *        root's step); k_prefix, v_prefix [B, hkv, max_prefix, head_dim] bf16
 *        (the draft's own cache) with prefix_len [B] (clamped to max_prefix);
 *      pool_tok [B, P] and slot_src [B, S] as eagle_expand_depth left them
 *        after depth - 1 (unused at depth 0).
 * Out: draft_logits [B, S, V] fp32: the rows of this depth's slots.
 * In/out: ws (draft workspace, ws_bytes >= eagle_draft_workspace_size): the
 *        slot state of depths 0..depth-1 is read and this depth's is added;
 *        depth 0 resets it.  One round's depths must run in order on one
 *        stream with one workspace.
 * Status: BAD_TREE (a frontier slot with no pool entry), TOKEN_RANGE,
 *        NONFINITE (a non-finite product anywhere in the layer). */
int eagle_draft_forward(const eagle_tree_params* p, int32_t depth, const eagle_draft_dims* dims,
                        const eagle_draft_weights* w, const int32_t* root_token, const void* root_feat,
                        const void* k_prefix, const void* v_prefix, const int32_t* prefix_len,
                        const int32_t* pool_tok, const int32_t* slot_src, float* draft_logits, void* ws,
                        size_t ws_bytes, int32_t* dev_status, void* stream);

/* Children of depth `depth`'s frontier slots from their rows of draft_logits
 * [B, S, V] (the same selection, confidences and statistics as
 * eagle_expand_tree), written to pool_tok/pool_q [B, S, k] and slot_stats
 * [B, S, 2] at those slots; for depth < D-1 also the next depth's frontier:
 * slot_src [B, S] of its k slots (ranks of the newest layer by value, as in
 * eagle_expand_tree).  ws: the round workspace (eagle_workspace_size). */
int eagle_expand_depth(const eagle_tree_params* p, int32_t depth, const float* draft_logits, int32_t* pool_tok,
                       float* pool_q, int32_t* slot_src, float* slot_stats, void* ws, size_t ws_bytes,
                       int32_t* dev_status, void* stream);

/* eagle_expand_depth with the sampling warp of [HW] section 2 on the draft
 * rows: this depth's frontier rows (slot 0 at depth 0, slots 1 + (d-1)k ..
 * dk at depth d >= 1, of every request) are warped first, exactly as
 * eagle_sampling_warp(top_k, top_p, min_keep = k, temperature) warps them,
 * their bounds written to draft_bound [B, S, 2] uint32 at those slots (the
 * other slots are left alone; after depth D-1 the buffer holds every
 * expanded slot's bound, as eagle_verify_accept_warped takes them), and the
 * children are drawn from the warped rows as eagle_expand_tree_warped draws
 * them.  Needs temperature > 0 (a warp applies to sampling), top_k == 0 or
 * top_k >= k, 0 < top_p <= 1 (else SHAPE), and a workspace of
 * eagle_workspace_size (it also holds the warped rows' statistics).
 * Everything else as eagle_expand_depth. */
int eagle_expand_depth_warped(const eagle_tree_params* p, int32_t depth, int32_t top_k, float top_p,
                              const float* draft_logits, uint32_t* draft_bound, int32_t* pool_tok, float* pool_q,
                              int32_t* slot_src, float* slot_stats, void* ws, size_t ws_bytes, int32_t* dev_status,
                              void* stream);

/* Rerank and flatten the complete pool (after depth D-1): the node arrays,
 * pool_flat and slot_src exactly as eagle_expand_tree writes them. */
int eagle_expand_finish(const eagle_tree_params* p, const int32_t* root_token, const int32_t* pool_tok,
                        const float* pool_q, int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                        int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_flat,
                        int32_t* slot_src, int32_t* dev_status, void* stream);

/* Human-readable name of a return code. */
const char* eagle_error_string(int32_t code);

/* ABI version: (major << 16) | minor. */
int32_t eagle_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H */
