// Host side of libeagle: the C ABI declared in include/eagle.h.  Every entry
// point validates its arguments on the host (before any HIP call), carves its
// scratch out of the caller's workspace and enqueues its kernels on the
// caller's stream.
#include <dlfcn.h>
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace eagle;

// Scratch of eagle_expand_tree_noalloc: one static device array per GPU
// (64 MiB, held by every GPU the library runs on until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device may reach a
// kernel, a fill or a copy.
static __device__ __align__(256) unsigned char scratch[EAGLE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = EAGLE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and cached.  Returns null on failure.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Optional roctx ranges around the calls that enqueue work: with EAGLE_ROCTX
// set (and not "0") in the environment, the first call loads the roctx
// library of ROCm and each such call pushes a range named after itself
// (rocprofv3 --marker-trace records them on the host timeline).  Otherwise
// nothing is loaded and a call pays one check of a resolved pointer.
struct RoctxApi {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const RoctxApi& roctx_api() {
  static const RoctxApi api = [] {
    RoctxApi r;
    const char* on = getenv("EAGLE_ROCTX");
    if (!on || !*on || (on[0] == '0' && on[1] == 0)) return r;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (!h) return r;
    r.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!r.push || !r.pop) r.push = nullptr, r.pop = nullptr;
    return r;
  }();
  return api;
}

class CallRange {
 public:
  explicit CallRange(const char* name) : api_(roctx_api()) {
    if (api_.push) api_.push(name);
  }
  ~CallRange() {
    if (api_.push) api_.pop();
  }

 private:
  const RoctxApi& api_;
};
#define EAGLE_CALL_RANGE() CallRange eagle_call_range_(__func__)

constexpr size_t kCounterBytes = 64 * 1024;           // ticket counters at the workspace head

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by expand and accept.
int check_tree_params(const eagle_tree_params* p) {
  if (!p) return EAGLE_ERR_NULL;
  const int64_t B = p->batch, V = p->vocab, D = p->depth, k = p->topk, m = p->m;
  if (B < 1 || B > (1 << 20)) return EAGLE_ERR_SHAPE;
  if (k < 1 || k > EAGLE_MAX_TOPK) return EAGLE_ERR_SHAPE;
  if (D < 1 || D > EAGLE_MAX_DEPTH) return EAGLE_ERR_SHAPE;
  if (V < k || V > EAGLE_MAX_VOCAB) return EAGLE_ERR_SHAPE;
  const int64_t S = 1 + (D - 1) * k, P = S * k;
  if (P > EAGLE_MAX_POOL) return EAGLE_ERR_SHAPE;
  if (m < 1 || m > P || m + 1 > EAGLE_MAX_NODES) return EAGLE_ERR_SHAPE;
  if (!(p->temperature >= 0.f) || !isfinite(p->temperature)) return EAGLE_ERR_SHAPE;
  return EAGLE_OK;
}

int check_attn(int32_t B, int32_t n, int32_t hq, int32_t hkv, int32_t dh, int32_t Lmax, int32_t dtype) {
  if (B < 1 || n < 1 || n > EAGLE_MAX_NODES || hq < 1 || hkv < 1 || hq % hkv != 0 || Lmax < 0) return EAGLE_ERR_SHAPE;
  if ((int64_t)n * (hq / hkv) > (1 << 16)) return EAGLE_ERR_SHAPE;
  if (dtype == EAGLE_BF16) {
    if (dh != 64 && dh != 128) return EAGLE_ERR_DTYPE;
  } else if (dtype == EAGLE_F32) {
    if (dh != 16 && dh != 32 && dh != 64 && dh != 128) return EAGLE_ERR_DTYPE;
  } else {
    return EAGLE_ERR_DTYPE;
  }
  return EAGLE_OK;
}

int check_lm(int32_t rows, int32_t hidden, int32_t vocab, int32_t dtype) {
  if (rows < 1 || hidden < 1 || vocab < 1 || vocab > (1 << 24)) return EAGLE_ERR_SHAPE;
  if (dtype == EAGLE_BF16) {
    if (hidden % 128 != 0) return EAGLE_ERR_SHAPE;
    if ((int64_t)rows * hidden >= ((int64_t)1 << 31)) return EAGLE_ERR_SHAPE;  // 32-bit X offsets
  } else if (dtype == EAGLE_F32) {
    if (hidden > 16384) return EAGLE_ERR_SHAPE;  // the fp32 path keeps one input row in LDS
  } else {
    return EAGLE_ERR_DTYPE;
  }
  if ((int64_t)lm_mtiles(rows) > 65535) return EAGLE_ERR_SHAPE;
  return EAGLE_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? EAGLE_OK : EAGLE_ERR_LAUNCH; }

float* stage_area(void* ws) { return reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes); }

// A static tree's tables from its parent array (host memory): node 0 is the
// root (-1), 0 <= parent[i] < i; siblings rank in flat order; slots are the
// nodes with children, in flat order.
int static_shape(int32_t n, const int32_t* parent, StaticShape* sh) {
  if (!parent || !sh) return EAGLE_ERR_NULL;
  if (n < 2 || n > EAGLE_MAX_NODES) return EAGLE_ERR_SHAPE;
  if (parent[0] != -1) return EAGLE_ERR_SHAPE;
  int nchild[EAGLE_MAX_NODES] = {0};
  sh->n = n;
  sh->parent[0] = -1;
  sh->depth[0] = 0;
  sh->sib[0] = 0;
  int D = 0;
  for (int i = 1; i < n; ++i) {
    const int a = parent[i];
    if (a < 0 || a >= i) return EAGLE_ERR_SHAPE;
    const int d = sh->depth[a] + 1;
    if (d > EAGLE_MAX_DEPTH || nchild[a] >= EAGLE_MAX_TOPK) return EAGLE_ERR_SHAPE;
    sh->parent[i] = (int16_t)a;
    sh->depth[i] = (uint8_t)d;
    sh->sib[i] = (uint8_t)nchild[a]++;
    D = d > D ? d : D;
  }
  int S = 0, kmax = 0;
  for (int i = 0; i < n; ++i) {
    sh->slot[i] = -1;
    if (nchild[i] > 0) {
      sh->slot[i] = (int16_t)S;
      sh->slot_node[S] = (int16_t)i;
      sh->slot_k[S] = (uint8_t)nchild[i];
      kmax = nchild[i] > kmax ? nchild[i] : kmax;
      ++S;
    }
  }
  sh->S = S;
  sh->kmax = kmax;
  sh->D = D;
  return EAGLE_OK;
}

// Round parameters of a static tree (batch, vocabulary, k = the shape's
// largest child count, depth, m = n - 1, temperature).
int check_static_params(const eagle_tree_params* p) {
  if (!p) return EAGLE_ERR_NULL;
  if (p->batch < 1 || p->batch > (1 << 20)) return EAGLE_ERR_SHAPE;
  if (p->topk < 1 || p->topk > EAGLE_MAX_TOPK || p->depth < 1 || p->depth > EAGLE_MAX_DEPTH) return EAGLE_ERR_SHAPE;
  if (p->vocab < p->topk || p->vocab > EAGLE_MAX_VOCAB) return EAGLE_ERR_SHAPE;
  if (p->m < 1 || p->m + 1 > EAGLE_MAX_NODES) return EAGLE_ERR_SHAPE;
  if (!(p->temperature >= 0.f) || !isfinite(p->temperature)) return EAGLE_ERR_SHAPE;
  return EAGLE_OK;
}

int check_static(const eagle_tree_params* p, int32_t n, const int32_t* parent, StaticShape* sh) {
  int rc = check_static_params(p);
  if (rc != EAGLE_OK) return rc;
  rc = static_shape(n, parent, sh);
  if (rc != EAGLE_OK) return rc;
  if (p->m != n - 1 || p->topk != sh->kmax || p->depth != sh->D) return EAGLE_ERR_SHAPE;
  return EAGLE_OK;
}

// Shape checks of the draft head; fills the layout on success.
int check_draft(const eagle_tree_params* p, const eagle_draft_dims* d, DraftLayout* lay) {
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (!d) return EAGLE_ERR_NULL;
  const int B = p->batch, k = p->topk, D = p->depth, V = p->vocab;
  const int S = 1 + (D - 1) * k;
  const int64_t H = d->hidden, I = d->inter, Q = (int64_t)d->hq * d->head_dim;
  if (H < 128 || H % 128 != 0 || H > 16384 || I < 128 || I % 128 != 0 || I > (1 << 18)) return EAGLE_ERR_SHAPE;
  if (d->max_prefix < 1) return EAGLE_ERR_SHAPE;
  rc = check_attn(B, S, d->hq, d->hkv, d->head_dim, d->max_prefix, EAGLE_BF16);
  if (rc != EAGLE_OK) return rc;
  if (Q % 128 != 0) return EAGLE_ERR_SHAPE;
  const int64_t QKV = Q + 2LL * d->hkv * d->head_dim;
  const int R = B * k;
  if (check_lm(R, (int)(2 * H), (int)H, EAGLE_BF16) != EAGLE_OK || check_lm(R, (int)H, (int)QKV, EAGLE_BF16) != EAGLE_OK ||
      check_lm(R, (int)Q, (int)H, EAGLE_BF16) != EAGLE_OK || check_lm(R, (int)H, (int)(2 * I), EAGLE_BF16) != EAGLE_OK ||
      check_lm(R, (int)I, (int)H, EAGLE_BF16) != EAGLE_OK || check_lm(R, (int)H, V, EAGLE_BF16) != EAGLE_OK)
    return EAGLE_ERR_SHAPE;
  if ((int64_t)B * S * (QKV > 2 * H ? QKV : 2 * H) >= ((int64_t)1 << 31)) return EAGLE_ERR_SHAPE;
  *lay = draft_layout(B, S, k, V, (int)H, d->hq, d->hkv, d->head_dim, (int)I, d->max_prefix);
  return EAGLE_OK;
}

}  // namespace

extern "C" {

int32_t eagle_abi_version(void) { return (1 << 16) | 6; }

const char* eagle_error_string(int32_t code) {
  switch (code) {
    case EAGLE_OK: return "ok";
    case EAGLE_ERR_NULL: return "null pointer";
    case EAGLE_ERR_SHAPE: return "invalid shape";
    case EAGLE_ERR_DTYPE: return "unsupported dtype";
    case EAGLE_ERR_WORKSPACE: return "workspace too small";
    case EAGLE_ERR_LAUNCH: return "kernel launch failed";
    case EAGLE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case EAGLE_ERR_TOO_LARGE: return "sizes need more than the no-allocation scratch holds";
    default: return "unknown error";
  }
}

size_t eagle_workspace_size(const eagle_tree_params* p, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_prefix,
                            int32_t hidden) {
  if (check_tree_params(p) != EAGLE_OK) return 0;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k, N = p->m + 1;
  // the expansion's records, and after them the warped statistics of
  // eagle_expand_depth_warped
  size_t need = (exp_ws_bytes(B, S, V, k) + 255) / 256 * 256 + (size_t)B * S * 2 * sizeof(float);
  if (hq > 0 && hkv > 0 && head_dim > 0) {
    const int dt = head_dim == 64 || head_dim == 128 ? EAGLE_BF16 : EAGLE_F32;
    if (check_attn(B, N, hq, hkv, head_dim, max_prefix, dt) != EAGLE_OK) return 0;
    const AttnPlan pl = attn_plan(B, N, hq, hkv, head_dim, max_prefix, dt);
    const size_t a = attn_ws_bytes(B, hkv, head_dim, pl);
    if (a > need) need = a;
  }
  if (hidden > 0) {
    const size_t l = lm_ws_bytes(B * N, V, hidden);
    if (l > need) need = l;
  }
  need = (need + 255) / 256 * 256;
  return (kCounterBytes + need + accept_mail_bytes(B) + 255) / 256 * 256;
}

int eagle_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  EAGLE_CALL_RANGE();
  if (!ws) return EAGLE_ERR_NULL;
  if (ws_bytes < kCounterBytes || ws_bytes % 4 != 0) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_zero_ints(static_cast<int32_t*>(ws), ws_bytes / 4, (hipStream_t)stream));
}

int eagle_expand_tree(const eagle_tree_params* p, const float* draft_logits, const int32_t* root_token,
                      int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
                      int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_tok, float* pool_q,
                      int32_t* pool_flat, int32_t* slot_src, float* slot_stats, void* ws, size_t ws_bytes,
                      int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  return eagle_expand_tree_warped(p, draft_logits, nullptr, root_token, node_tok, node_parent, node_depth, node_sib,
                                  node_slot, node_value, node_q, pool_tok, pool_q, pool_flat, slot_src, slot_stats, ws,
                                  ws_bytes, dev_status, stream);
}

int eagle_expand_tree_warped(const eagle_tree_params* p, const float* draft_logits, const uint32_t* draft_bound,
                             const int32_t* root_token, int32_t* node_tok, int32_t* node_parent,
                             int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value,
                             float* node_q, int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                             float* slot_stats, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (!draft_logits || !root_token || !node_tok || !node_parent || !node_depth || !node_sib || !node_slot ||
      !node_value || !node_q || !pool_tok || !pool_q || !pool_flat || !slot_src || !slot_stats || !ws)
    return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k;
  if (ws_bytes < kCounterBytes + exp_ws_bytes(B, S, V, k)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_expand(B, S, V, D, k, p->m, p->temperature, p->seed, p->round_id, draft_logits,
                                     draft_bound, root_token, node_tok, node_parent, node_depth, node_sib, node_slot, node_value,
                                     node_q, pool_tok, pool_q, pool_flat, slot_src, slot_stats, stage_area(ws),
                                     dev_status, (hipStream_t)stream));
}

int eagle_expand_tree_masked(const eagle_tree_params* p, const float* draft_logits, const int32_t* root_token,
                             const int32_t* prefix_len, int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                             int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                             int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src,
                             float* slot_stats, uint64_t* mask, int32_t* pos, void* ws, size_t ws_bytes,
                             int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (!draft_logits || !root_token || !prefix_len || !node_tok || !node_parent || !node_depth || !node_sib ||
      !node_slot || !node_value || !node_q || !pool_tok || !pool_q || !pool_flat || !slot_src || !slot_stats ||
      !mask || !pos || !ws)
    return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k;
  if (ws_bytes < kCounterBytes + exp_ws_bytes(B, S, V, k)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_expand(B, S, V, D, k, p->m, p->temperature, p->seed, p->round_id, draft_logits,
                                     nullptr, root_token, node_tok, node_parent, node_depth, node_sib, node_slot,
                                     node_value, node_q, pool_tok, pool_q, pool_flat, slot_src, slot_stats,
                                     stage_area(ws), dev_status, (hipStream_t)stream, prefix_len, mask, pos));
}

int eagle_expand_tree_noalloc(const eagle_tree_params* p, const float* draft_logits, const int32_t* root_token,
                              int32_t* node_tok, int32_t* node_parent, int32_t* node_depth, int32_t* node_sib,
                              int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_tok,
                              float* pool_q, int32_t* pool_flat, int32_t* slot_src, float* slot_stats,
                              int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (!draft_logits || !root_token || !node_tok || !node_parent || !node_depth || !node_sib || !node_slot ||
      !node_value || !node_q || !pool_tok || !pool_q || !pool_flat || !slot_src || !slot_stats)
    return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k;
  if (exp_ws_bytes(B, S, V, k) > kNoAllocScratchBytes) return EAGLE_ERR_TOO_LARGE;
  // The candidate records are written by the scan before the merge reads
  // them, so the array needs no clearing between calls.
  void* ws = noalloc_scratch();
  if (!ws) return EAGLE_ERR_LAUNCH;
  return launch_status(launch_expand(B, S, V, D, k, p->m, p->temperature, p->seed, p->round_id, draft_logits,
                                     nullptr, root_token, node_tok, node_parent, node_depth, node_sib, node_slot,
                                     node_value, node_q, pool_tok, pool_q, pool_flat, slot_src, slot_stats,
                                     static_cast<float*>(ws), dev_status, (hipStream_t)stream));
}

int eagle_static_tree_info(int32_t n, const int32_t* shape_parent, int32_t* n_slots, int32_t* depth, int32_t* kmax,
                           int32_t* slot_k) {
  StaticShape sh;
  const int rc = static_shape(n, shape_parent, &sh);
  if (rc != EAGLE_OK) return rc;
  if (n_slots) *n_slots = sh.S;
  if (depth) *depth = sh.D;
  if (kmax) *kmax = sh.kmax;
  if (slot_k)
    for (int s = 0; s < sh.S; ++s) slot_k[s] = sh.slot_k[s];
  return EAGLE_OK;
}

size_t eagle_static_workspace_size(const eagle_tree_params* p, int32_t n, const int32_t* shape_parent, int32_t hq,
                                   int32_t hkv, int32_t head_dim, int32_t max_prefix, int32_t hidden) {
  StaticShape sh;
  if (check_static(p, n, shape_parent, &sh) != EAGLE_OK) return 0;
  const int B = p->batch, V = p->vocab;
  size_t need = exp_ws_bytes(B, sh.S, V, sh.kmax);
  if (hq > 0 && hkv > 0 && head_dim > 0) {
    const int dt = head_dim == 64 || head_dim == 128 ? EAGLE_BF16 : EAGLE_F32;
    if (check_attn(B, n, hq, hkv, head_dim, max_prefix, dt) != EAGLE_OK) return 0;
    const AttnPlan pl = attn_plan(B, n, hq, hkv, head_dim, max_prefix, dt);
    const size_t a = attn_ws_bytes(B, hkv, head_dim, pl);
    if (a > need) need = a;
  }
  if (hidden > 0) {
    const size_t l = lm_ws_bytes(B * n, V, hidden);
    if (l > need) need = l;
  }
  need = (need + 255) / 256 * 256;
  return (kCounterBytes + need + accept_mail_bytes(B) + 255) / 256 * 256;
}

int eagle_expand_static(const eagle_tree_params* p, int32_t n, const int32_t* shape_parent,
                        const float* draft_logits, const int32_t* root_token, int32_t* node_tok, int32_t* node_parent,
                        int32_t* node_depth, int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q,
                        int32_t* pool_tok, float* pool_q, int32_t* pool_flat, int32_t* slot_src, float* slot_stats,
                        void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  StaticShape sh;
  int rc = check_static(p, n, shape_parent, &sh);
  if (rc != EAGLE_OK) return rc;
  if (!draft_logits || !root_token || !node_tok || !node_parent || !node_depth || !node_sib || !node_slot ||
      !node_value || !node_q || !pool_tok || !pool_q || !pool_flat || !slot_src || !slot_stats || !ws)
    return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  if (ws_bytes < kCounterBytes + exp_ws_bytes(p->batch, sh.S, p->vocab, sh.kmax)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_expand_static(p->batch, p->vocab, sh, p->temperature, p->seed, p->round_id,
                                            draft_logits, root_token, node_tok, node_parent, node_depth, node_sib,
                                            node_slot, node_value, node_q, pool_tok, pool_q, pool_flat, slot_src,
                                            slot_stats, stage_area(ws), dev_status, (hipStream_t)stream));
}

int eagle_verify_accept_static(const eagle_tree_params* p, int32_t n_slots, const int32_t* node_tok,
                               const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                               const int32_t* pool_flat, const float* target_logits, const float* target_stats,
                               const int32_t* target_argmax, const float* draft_logits, const float* slot_stats,
                               const float* uniforms, int32_t* accept_len, int32_t* accept_path, int32_t* committed,
                               int32_t* n_committed, int32_t* near_tie, void* ws, size_t ws_bytes,
                               int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_static_params(p);
  if (rc != EAGLE_OK) return rc;
  if (n_slots < 1 || n_slots > p->m + 1) return EAGLE_ERR_SHAPE;
  const bool greedy = !(p->temperature > 0.f);
  if (!node_tok || !node_parent || !node_slot || !pool_tok || !pool_flat || !accept_len || !accept_path ||
      !committed || !n_committed || !near_tie || !ws)
    return EAGLE_ERR_NULL;
  if (greedy ? !target_argmax : (!target_logits || !target_stats || !draft_logits || !slot_stats || !uniforms))
    return EAGLE_ERR_NULL;
  const size_t mail = accept_mail_bytes(p->batch);
  const size_t end = ws_bytes & ~(size_t)255;
  if (end < kCounterBytes + mail) return EAGLE_ERR_WORKSPACE;
  void* mailbox = static_cast<char*>(ws) + end;
  return launch_status(launch_accept(p->batch, p->m + 1, p->vocab, p->depth, p->topk, n_slots, p->temperature,
                                     node_tok, node_parent, node_slot, pool_tok, pool_flat, target_logits,
                                     target_stats, target_argmax, draft_logits, slot_stats, nullptr, nullptr, nullptr,
                                     nullptr, uniforms, mailbox, accept_len, accept_path, committed, n_committed,
                                     near_tie, dev_status, (hipStream_t)stream));
}

int eagle_build_tree_mask(int32_t batch, int32_t n, const int32_t* node_parent, const int32_t* node_depth,
                          const int32_t* prefix_len, uint64_t* mask, int32_t* pos, int32_t* dev_status,
                          void* stream) {
  EAGLE_CALL_RANGE();
  if (batch < 1 || n < 1 || n > EAGLE_MAX_NODES) return EAGLE_ERR_SHAPE;
  if (!node_parent || !node_depth || !prefix_len || !mask || !pos) return EAGLE_ERR_NULL;
  return launch_status(launch_tree_mask(batch, n, node_parent, node_depth, prefix_len, mask, pos, dev_status,
                                        (hipStream_t)stream));
}

int eagle_tree_attention(int32_t batch, int32_t n, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_prefix,
                         int32_t dtype, const void* q, const void* k_prefix, const void* v_prefix,
                         const int32_t* prefix_len, const void* k_tree, const void* v_tree, const uint64_t* mask,
                         float scale, void* out, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_attn(batch, n, hq, hkv, head_dim, max_prefix, dtype);
  if (rc != EAGLE_OK) return rc;
  if (!isfinite(scale)) return EAGLE_ERR_SHAPE;
  if (!q || !prefix_len || !k_tree || !v_tree || !mask || !out || !ws) return EAGLE_ERR_NULL;
  if (max_prefix > 0 && (!k_prefix || !v_prefix)) return EAGLE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
      (max_prefix > 0 && (!aligned16(k_prefix) || !aligned16(v_prefix))))
    return EAGLE_ERR_ALIGN;
  const AttnPlan pl = attn_plan(batch, n, hq, hkv, head_dim, max_prefix, dtype);
  if (ws_bytes < kCounterBytes + attn_ws_bytes(batch, hkv, head_dim, pl)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_attention(batch, n, hq, hkv, head_dim, max_prefix, dtype, q, k_prefix, v_prefix,
                                        prefix_len, k_tree, v_tree, mask, scale, out, stage_area(ws), pl, dev_status,
                                        (hipStream_t)stream));
}

int eagle_lmhead_softmax(int32_t rows, int32_t hidden, int32_t vocab, int32_t dtype, const void* x, const void* w,
                         int32_t w_layout, float temperature, float* logits, float* row_stats, int32_t* row_argmax,
                         float* probs, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_lm(rows, hidden, vocab, dtype);
  if (rc != EAGLE_OK) return rc;
  if (w_layout != EAGLE_W_ROWMAJOR && w_layout != EAGLE_W_PACKED && w_layout != EAGLE_W_ZPACKED) return EAGLE_ERR_SHAPE;
  if (w_layout != EAGLE_W_ROWMAJOR && dtype != EAGLE_BF16) return EAGLE_ERR_DTYPE;
  if (w_layout == EAGLE_W_ZPACKED && (rows > EAGLE_ZPACK_MAX_ROWS || hidden > 16384 || lm_zlayout(vocab, hidden).bytes > 0xffffffffu)) return EAGLE_ERR_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return EAGLE_ERR_SHAPE;
  if (!x || !w || !logits || !row_stats || !row_argmax || !ws) return EAGLE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w)) return EAGLE_ERR_ALIGN;
  if (ws_bytes < kCounterBytes + lm_ws_bytes(rows, vocab, hidden)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_lmhead(rows, hidden, vocab, dtype, w_layout, x, w, temperature, logits, row_stats,
                                     row_argmax, probs, stage_area(ws), dev_status, (hipStream_t)stream));
}

int eagle_lmhead_softmax_compact(int32_t rows, int32_t hidden, int32_t vocab, const void* x, const void* w,
                                 int32_t w_layout, float temperature, uint16_t* target_z16, float* block_max,
                                 float* row_stats, int32_t* row_argmax, void* ws, size_t ws_bytes,
                                 int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_lm(rows, hidden, vocab, EAGLE_BF16);
  if (rc != EAGLE_OK) return rc;
  if (w_layout != EAGLE_W_ROWMAJOR && w_layout != EAGLE_W_PACKED && w_layout != EAGLE_W_ZPACKED) return EAGLE_ERR_SHAPE;
  if (w_layout == EAGLE_W_ZPACKED && (rows > EAGLE_ZPACK_MAX_ROWS || hidden > 16384 || lm_zlayout(vocab, hidden).bytes > 0xffffffffu)) return EAGLE_ERR_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return EAGLE_ERR_SHAPE;
  if (!x || !w || !target_z16 || !block_max || !row_stats || !row_argmax || !ws) return EAGLE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)target_z16 & 7) != 0 || ((uintptr_t)block_max & 3) != 0)
    return EAGLE_ERR_ALIGN;
  if (ws_bytes < kCounterBytes + lm_ws_bytes(rows, vocab, hidden)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_lmhead_compact(rows, hidden, vocab, w_layout, x, w, temperature, target_z16,
                                             block_max, row_stats, row_argmax, stage_area(ws), dev_status,
                                             (hipStream_t)stream));
}

int eagle_verify_accept_compact(const eagle_tree_params* p, int32_t n_slots, const int32_t* node_tok,
                                const int32_t* node_parent, const int32_t* node_slot, const int32_t* pool_tok,
                                const int32_t* pool_flat, const uint16_t* target_z16, const float* block_max,
                                const float* target_stats, const int32_t* target_argmax, const float* draft_logits,
                                const float* slot_stats, const float* uniforms, int32_t* accept_len,
                                int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
                                void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = n_slots > 0 ? check_static_params(p) : check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (n_slots < 0 || n_slots > p->m + 1) return EAGLE_ERR_SHAPE;
  const int S = n_slots > 0 ? n_slots : 1 + (p->depth - 1) * p->topk;
  const bool greedy = !(p->temperature > 0.f);
  if (!node_tok || !node_parent || !node_slot || !pool_tok || !pool_flat || !accept_len || !accept_path ||
      !committed || !n_committed || !near_tie || !ws)
    return EAGLE_ERR_NULL;
  if (greedy ? !target_argmax
             : (!target_z16 || !block_max || !target_stats || !draft_logits || !slot_stats || !uniforms))
    return EAGLE_ERR_NULL;
  const size_t mail = accept_mail_bytes(p->batch);
  const size_t end = ws_bytes & ~(size_t)255;
  if (end < kCounterBytes + mail) return EAGLE_ERR_WORKSPACE;
  void* mailbox = static_cast<char*>(ws) + end;
  return launch_status(launch_accept(p->batch, p->m + 1, p->vocab, p->depth, p->topk, S, p->temperature, node_tok,
                                     node_parent, node_slot, pool_tok, pool_flat, nullptr, target_stats,
                                     target_argmax, draft_logits, slot_stats, nullptr, nullptr,
                                     greedy ? nullptr : target_z16, greedy ? nullptr : block_max, uniforms, mailbox,
                                     accept_len, accept_path, committed, n_committed, near_tie, dev_status,
                                     (hipStream_t)stream));
}

size_t eagle_lmhead_packed_bytes(int32_t vocab, int32_t hidden, int32_t dtype) {
  if (dtype != EAGLE_BF16 || check_lm(1, hidden, vocab, dtype) != EAGLE_OK) return 0;
  return lm_packed_bytes(vocab, hidden);
}

int eagle_lmhead_pack_weight(int32_t vocab, int32_t hidden, int32_t dtype, const void* w, void* w_packed,
                             void* stream) {
  EAGLE_CALL_RANGE();
  if (dtype != EAGLE_BF16) return EAGLE_ERR_DTYPE;
  int rc = check_lm(1, hidden, vocab, dtype);
  if (rc != EAGLE_OK) return rc;
  if (!w || !w_packed) return EAGLE_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_packed)) return EAGLE_ERR_ALIGN;
  return launch_status(launch_pack_lmhead(vocab, hidden, w, w_packed, (hipStream_t)stream));
}

size_t eagle_lmhead_zpack_bytes(int32_t vocab, int32_t hidden) {
  if (check_lm(1, hidden, vocab, EAGLE_BF16) != EAGLE_OK || hidden > 16384) return 0;
  if (lm_zlayout(vocab, hidden).bytes > 0xffffffffu) return 0;  // one buffer resource spans it
  return lm_zlayout(vocab, hidden).bytes;
}

int eagle_lmhead_zpack_weight(int32_t vocab, int32_t hidden, const void* w, void* w_z, int32_t* raw_fragments,
                              void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_lm(1, hidden, vocab, EAGLE_BF16);
  if (rc != EAGLE_OK) return rc;
  if (hidden > 16384 || lm_zlayout(vocab, hidden).bytes > 0xffffffffu) return EAGLE_ERR_SHAPE;
  if (!w || !w_z) return EAGLE_ERR_NULL;
  if (!aligned16(w) || ((uintptr_t)w_z & 255) != 0 || ((uintptr_t)raw_fragments & 3) != 0) return EAGLE_ERR_ALIGN;
  return launch_status(launch_zpack_lmhead(vocab, hidden, w, w_z, raw_fragments, (hipStream_t)stream));
}

int eagle_verify_accept(const eagle_tree_params* p, const int32_t* node_tok, const int32_t* node_parent,
                        const int32_t* node_slot, const int32_t* pool_tok, const int32_t* pool_flat,
                        const float* target_logits, const float* target_stats, const int32_t* target_argmax,
                        const float* draft_logits, const float* slot_stats, const float* uniforms,
                        int32_t* accept_len, int32_t* accept_path, int32_t* committed, int32_t* n_committed,
                        int32_t* near_tie, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  return eagle_verify_accept_warped(p, nullptr, nullptr, node_tok, node_parent, node_slot, pool_tok, pool_flat,
                                    target_logits, target_stats, target_argmax, draft_logits, slot_stats, uniforms,
                                    accept_len, accept_path, committed, n_committed, near_tie, ws, ws_bytes,
                                    dev_status, stream);
}

int eagle_verify_accept_warped(const eagle_tree_params* p, const uint32_t* target_bound, const uint32_t* draft_bound,
                               const int32_t* node_tok, const int32_t* node_parent, const int32_t* node_slot,
                               const int32_t* pool_tok, const int32_t* pool_flat, const float* target_logits,
                               const float* target_stats, const int32_t* target_argmax, const float* draft_logits,
                               const float* slot_stats, const float* uniforms, int32_t* accept_len,
                               int32_t* accept_path, int32_t* committed, int32_t* n_committed, int32_t* near_tie,
                               void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  const bool greedy = !(p->temperature > 0.f);
  if (!node_tok || !node_parent || !node_slot || !pool_tok || !pool_flat || !accept_len || !accept_path ||
      !committed || !n_committed || !near_tie || !ws)
    return EAGLE_ERR_NULL;
  if (greedy ? !target_argmax : (!target_logits || !target_stats || !draft_logits || !slot_stats || !uniforms))
    return EAGLE_ERR_NULL;
  // Mailbox b sits at a fixed distance from the 256-byte-aligned end of the
  // workspace (b + 1 mailboxes back), whatever the batch of this call.
  const size_t mail = accept_mail_bytes(p->batch);
  const size_t end = ws_bytes & ~(size_t)255;
  if (end < kCounterBytes + mail) return EAGLE_ERR_WORKSPACE;
  void* mailbox = static_cast<char*>(ws) + end;
  return launch_status(launch_accept(p->batch, p->m + 1, p->vocab, p->depth, p->topk,
                                     1 + (p->depth - 1) * p->topk, p->temperature, node_tok,
                                     node_parent, node_slot, pool_tok, pool_flat, target_logits, target_stats,
                                     target_argmax, draft_logits, slot_stats, greedy ? nullptr : target_bound,
                                     greedy ? nullptr : draft_bound, nullptr, nullptr, uniforms, mailbox, accept_len,
                                     accept_path, committed, n_committed, near_tie, dev_status,
                                     (hipStream_t)stream));
}

int eagle_gather_rows(int32_t n_rows, int32_t row_elems, int32_t dtype, const void* table, int32_t table_rows,
                      const int32_t* idx, void* out, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  if (n_rows < 0 || row_elems < 1 || table_rows < 1) return EAGLE_ERR_SHAPE;
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return EAGLE_ERR_DTYPE;
  if (n_rows == 0) return EAGLE_OK;
  if (!table || !idx || !out) return EAGLE_ERR_NULL;
  const int esz = dtype == EAGLE_F32 ? 4 : 2;
  GatherSet gs{};
  gs.n = 1;
  gs.table[0] = table;
  gs.out[0] = out;
  gs.row_units[0] = row_elems * esz;
  return launch_status(launch_gather(n_rows, gs, table_rows, idx, dev_status, (hipStream_t)stream));
}

int eagle_gather_rows_multi(int32_t n_tables, int32_t n_rows, int32_t dtype, int32_t table_rows, const int32_t* idx,
                            const int32_t* row_elems, const void* const* tables, void* const* outs,
                            int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  if (n_tables < 1 || n_tables > kGatherMaxTables || n_rows < 0 || table_rows < 1) return EAGLE_ERR_SHAPE;
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return EAGLE_ERR_DTYPE;
  if (!row_elems || !tables || !outs) return EAGLE_ERR_NULL;
  const int esz = dtype == EAGLE_F32 ? 4 : 2;
  GatherSet gs{};
  gs.n = n_tables;
  for (int t = 0; t < n_tables; ++t) {
    if (row_elems[t] < 1) return EAGLE_ERR_SHAPE;
    if (n_rows > 0 && (!tables[t] || !outs[t])) return EAGLE_ERR_NULL;
    gs.table[t] = tables[t];
    gs.out[t] = outs[t];
    gs.row_units[t] = row_elems[t] * esz;
  }
  if (n_rows == 0) return EAGLE_OK;
  if (!idx) return EAGLE_ERR_NULL;
  return launch_status(launch_gather(n_rows, gs, table_rows, idx, dev_status, (hipStream_t)stream));
}

int eagle_commit_accepted(int32_t batch, int32_t n, int32_t hkv, int32_t head_dim, int32_t max_prefix,
                          int32_t hidden, int32_t depth, int32_t dtype, const int32_t* accept_len,
                          const int32_t* accept_path, const void* k_tree, const void* v_tree, const void* x,
                          void* k_prefix, void* v_prefix, int32_t* prefix_len, void* feat, int32_t* dev_status,
                          void* stream) {
  EAGLE_CALL_RANGE();
  if (batch < 0 || batch > (1 << 20) || n < 1 || n > EAGLE_MAX_NODES || hkv < 1 || head_dim < 1 ||
      max_prefix < 1 || hidden < 1 || depth < 1 || depth > EAGLE_MAX_DEPTH)
    return EAGLE_ERR_SHAPE;
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return EAGLE_ERR_DTYPE;
  const int64_t esz = dtype == EAGLE_F32 ? 4 : 2;
  if ((head_dim * esz) % 16 != 0 || (hidden * esz) % 16 != 0) return EAGLE_ERR_ALIGN;
  // 32-bit unit offsets inside one request's tree rows; 64-bit elsewhere
  if ((int64_t)n * hkv * head_dim * esz / 16 >= ((int64_t)1 << 31) ||
      (int64_t)n * hidden * esz / 16 >= ((int64_t)1 << 31))
    return EAGLE_ERR_SHAPE;
  if (batch == 0) return EAGLE_OK;
  if (!accept_len || !accept_path || !k_tree || !v_tree || !x || !k_prefix || !v_prefix || !prefix_len || !feat)
    return EAGLE_ERR_NULL;
  if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(x) || !aligned16(k_prefix) || !aligned16(v_prefix) ||
      !aligned16(feat))
    return EAGLE_ERR_ALIGN;
  return launch_status(launch_commit(batch, n, hkv, head_dim, max_prefix, hidden, depth, (int)esz, accept_len,
                                     accept_path, k_tree, v_tree, x, k_prefix, v_prefix, prefix_len, feat,
                                     dev_status, (hipStream_t)stream));
}

int eagle_sampling_warp(int32_t rows, int32_t vocab, int32_t top_k, float top_p, int32_t min_keep, float temperature,
                        const float* logits, float* row_stats, uint32_t* bound, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  if (rows < 0 || rows > (1 << 24) || vocab < 1 || vocab > EAGLE_MAX_VOCAB || top_k < 0) return EAGLE_ERR_SHAPE;
  if (!(top_p > 0.f) || !(top_p <= 1.f) || min_keep < 1 || min_keep > vocab) return EAGLE_ERR_SHAPE;
  if (top_k != 0 && top_k < min_keep) return EAGLE_ERR_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return EAGLE_ERR_SHAPE;
  if (rows == 0) return EAGLE_OK;
  if (!logits || !row_stats || !bound) return EAGLE_ERR_NULL;
  return launch_status(launch_warp(rows, vocab, top_k, top_p, min_keep, temperature, logits, row_stats, bound,
                                   dev_status, (hipStream_t)stream));
}

size_t eagle_draft_workspace_size(const eagle_tree_params* p, const eagle_draft_dims* dims) {
  DraftLayout lay;
  if (check_draft(p, dims, &lay) != EAGLE_OK) return 0;
  return lay.total;
}

int eagle_draft_workspace_layout(const eagle_tree_params* p, const eagle_draft_dims* dims, size_t* offsets,
                                 int32_t n) {
  DraftLayout lay;
  int rc = check_draft(p, dims, &lay);
  if (rc != EAGLE_OK) return rc;
  if (n < 0) return EAGLE_ERR_SHAPE;
  if (n > 0 && !offsets) return EAGLE_ERR_NULL;
  const size_t all[EAGLE_DRAFT_NBUF] = {lay.slot_k, lay.slot_v, lay.slot_feat, lay.slot_mask, lay.idx, lay.x0,
                                        lay.u,      lay.n1,     lay.qkv,       lay.qc,        lay.og,  lay.h,
                                        lay.n2,     lay.gu,     lay.mm,        lay.y,         lay.xa};
  const int w = n < EAGLE_DRAFT_NBUF ? n : EAGLE_DRAFT_NBUF;
  for (int i = 0; i < w; ++i) offsets[i] = all[i];
  return w;
}

int eagle_draft_forward(const eagle_tree_params* p, int32_t depth, const eagle_draft_dims* dims,
                        const eagle_draft_weights* w, const int32_t* root_token, const void* root_feat,
                        const void* k_prefix, const void* v_prefix, const int32_t* prefix_len,
                        const int32_t* pool_tok, const int32_t* slot_src, float* draft_logits, void* ws,
                        size_t ws_bytes, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  DraftLayout lay;
  int rc = check_draft(p, dims, &lay);
  if (rc != EAGLE_OK) return rc;
  if (depth < 0 || depth >= p->depth) return EAGLE_ERR_SHAPE;
  if (!w || !w->embed || !w->fc || !w->qkv || !w->o || !w->gate_up || !w->down || !w->lm_head) return EAGLE_ERR_NULL;
  if (!root_token || !root_feat || !k_prefix || !v_prefix || !prefix_len || !draft_logits || !ws)
    return EAGLE_ERR_NULL;
  if (depth > 0 && (!pool_tok || !slot_src)) return EAGLE_ERR_NULL;
  const void* al[] = {w->embed, w->fc, w->qkv, w->o, w->gate_up, w->down, w->lm_head, root_feat, k_prefix, v_prefix,
                      draft_logits, ws};
  for (const void* q : al)
    if (!aligned16(q)) return EAGLE_ERR_ALIGN;
  if (w->lm_head_z != nullptr && (((uintptr_t)w->lm_head_z & 255) != 0)) return EAGLE_ERR_ALIGN;
  if (w->lm_head_z != nullptr && lm_zlayout(p->vocab, dims->hidden).bytes > 0xffffffffu) return EAGLE_ERR_SHAPE;
  if (ws_bytes < lay.total) return EAGLE_ERR_WORKSPACE;
  DraftArgs a;
  a.B = p->batch;
  a.k = p->topk;
  a.S = 1 + (p->depth - 1) * p->topk;
  a.V = p->vocab;
  a.H = dims->hidden;
  a.hq = dims->hq;
  a.hkv = dims->hkv;
  a.dh = dims->head_dim;
  a.I = dims->inter;
  a.max_prefix = dims->max_prefix;
  a.depth = depth;
  a.scale = 1.0f / sqrtf((float)dims->head_dim);
  a.w = *w;
  a.root = root_token;
  a.root_feat = root_feat;
  a.k_prefix = k_prefix;
  a.v_prefix = v_prefix;
  a.prefix_len = prefix_len;
  a.pool_tok = pool_tok;
  a.slot_src = slot_src;
  a.rows = draft_logits;
  a.ws = ws;
  a.lay = lay;
  a.status = dev_status;
  return launch_status(launch_draft_forward(a, (hipStream_t)stream));
}

int eagle_expand_depth(const eagle_tree_params* p, int32_t depth, const float* draft_logits, int32_t* pool_tok,
                       float* pool_q, int32_t* slot_src, float* slot_stats, void* ws, size_t ws_bytes,
                       int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (depth < 0 || depth >= p->depth) return EAGLE_ERR_SHAPE;
  if (!draft_logits || !pool_tok || !pool_q || !slot_src || !slot_stats || !ws) return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k;
  if (ws_bytes < kCounterBytes + exp_ws_bytes(B, S, V, k)) return EAGLE_ERR_WORKSPACE;
  return launch_status(launch_expand_depth(B, S, V, D, k, p->m, p->temperature, p->seed, p->round_id, depth,
                                           draft_logits, nullptr, pool_tok, pool_q, slot_src, slot_stats,
                                           stage_area(ws), dev_status, (hipStream_t)stream));
}

int eagle_expand_depth_warped(const eagle_tree_params* p, int32_t depth, int32_t top_k, float top_p,
                              const float* draft_logits, uint32_t* draft_bound, int32_t* pool_tok, float* pool_q,
                              int32_t* slot_src, float* slot_stats, void* ws, size_t ws_bytes, int32_t* dev_status,
                              void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (depth < 0 || depth >= p->depth) return EAGLE_ERR_SHAPE;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  if (!(p->temperature > 0.f)) return EAGLE_ERR_SHAPE;  // a warp applies to sampling only
  if (top_k < 0 || (top_k != 0 && top_k < k) || !(top_p > 0.f) || !(top_p <= 1.f)) return EAGLE_ERR_SHAPE;
  if (!draft_logits || !draft_bound || !pool_tok || !pool_q || !slot_src || !slot_stats || !ws) return EAGLE_ERR_NULL;
  if (!aligned16(draft_logits)) return EAGLE_ERR_ALIGN;
  const int S = 1 + (D - 1) * k;
  const size_t units = (exp_ws_bytes(B, S, V, k) + 255) / 256 * 256;
  if (ws_bytes < kCounterBytes + units + (size_t)B * S * 2 * sizeof(float)) return EAGLE_ERR_WORKSPACE;
  // this depth's frontier rows: slot s0 + i of request b for i < n
  const int s0 = depth == 0 ? 0 : 1 + (depth - 1) * k, n = depth == 0 ? 1 : k;
  float* wstats = reinterpret_cast<float*>(reinterpret_cast<char*>(stage_area(ws)) + units);  // [B, S, 2]
  hipError_t e = launch_warp_map(B * n, V, top_k, top_p, k, p->temperature, draft_logits, wstats, draft_bound,
                                 dev_status, RowMap{n, S, s0}, (hipStream_t)stream);
  if (e != hipSuccess) return launch_status(e);
  return launch_status(launch_expand_depth(B, S, V, D, k, p->m, p->temperature, p->seed, p->round_id, depth,
                                           draft_logits, draft_bound, pool_tok, pool_q, slot_src, slot_stats,
                                           stage_area(ws), dev_status, (hipStream_t)stream));
}

int eagle_expand_finish(const eagle_tree_params* p, const int32_t* root_token, const int32_t* pool_tok,
                        const float* pool_q, int32_t* node_tok, int32_t* node_parent, int32_t* node_depth,
                        int32_t* node_sib, int32_t* node_slot, float* node_value, float* node_q, int32_t* pool_flat,
                        int32_t* slot_src, int32_t* dev_status, void* stream) {
  EAGLE_CALL_RANGE();
  int rc = check_tree_params(p);
  if (rc != EAGLE_OK) return rc;
  if (!root_token || !pool_tok || !pool_q || !node_tok || !node_parent || !node_depth || !node_sib || !node_slot ||
      !node_value || !node_q || !pool_flat || !slot_src)
    return EAGLE_ERR_NULL;
  const int B = p->batch, V = p->vocab, k = p->topk, D = p->depth;
  const int S = 1 + (D - 1) * k;
  return launch_status(launch_expand_finish(B, S, V, D, k, p->m, root_token, node_tok, node_parent, node_depth,
                                            node_sib, node_slot, node_value, node_q, pool_tok, pool_q, pool_flat,
                                            slot_src, dev_status, (hipStream_t)stream));
}

}  // extern "C"
