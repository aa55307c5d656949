// Post-accept commit: the accepted path becomes part of the context.
// EAGLE-1 notes, section 3.3: the accepted tokens and their features are kept
// for the next drafting round; hubwiz section 5: the longest consistent path
// is committed, the other branches are dropped, and the loop continues from
// the longer context.
//
// Committed rows are the root (flat node 0, whose key/value the verify pass
// produced) and the accepted nodes in path order.  Their tree keys/values are
// appended to the prefix cache at positions L .. L + a, the length becomes
// L + a + 1, and their LM-head inputs (the features) go to rows 0 .. a of a
// [depth + 1, hidden] block per request, the rows past a zero-filled.
//
// Grid (B, depth + 2): workgroup y == 0 copies the keys/values and owns the
// request's length (it alone reads and writes prefix_len[b], so the in-place
// update has no reader in another workgroup); workgroup y >= 1 writes feature
// row y - 1.  All copies are 16-byte vector loads/stores, several in flight
// per thread; the work is a few hundred KB per request and launch-bound.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kCommitBatch = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    int n, int hkv, int upr, int max_prefix, int hunits, int D, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accept_path, const uint4* __restrict__ kt, const uint4* __restrict__ vt,
    const uint4* __restrict__ x, uint4* __restrict__ kp, uint4* __restrict__ vp, int32_t* prefix_len,
    uint4* __restrict__ feat, int32_t* status) {
  __shared__ int s_nodes[EAGLE_MAX_DEPTH + 1];
  __shared__ int s_info[3];  // accepted count (-1: invalid path), L, room in the cache
  const int b = blockIdx.x;
  const int part = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const int a = accept_len[b];
    bool ok = a >= 0 && a <= D;
    s_nodes[0] = 0;
    for (int r = 0; ok && r < a; ++r) {
      const int u = accept_path[(size_t)b * D + r];
      ok = u >= 1 && u < n;
      s_nodes[r + 1] = u;
    }
    const int L = part == 0 ? prefix_len[b] : 0;
    const bool room = ok && L >= 0 && (int64_t)L + a + 1 <= max_prefix;
    s_info[0] = ok ? a : -1;
    s_info[1] = L;
    s_info[2] = room;
    if (part == 0) {
      if (!ok) set_status(status, EAGLE_STATUS_BAD_TREE);
      else if (!room) set_status(status, EAGLE_STATUS_CACHE_FULL);
    }
  }
  __syncthreads();
  const int a = s_info[0];
  if (part == 0) {
    if (a < 0 || !s_info[2]) return;
    const int L = s_info[1];
    const int row_units = hkv * upr;           // one node's keys (or values), all kv heads
    const int per = (a + 1) * row_units;       // keys of every committed row
    const int total = 2 * per;                 // + values
    for (int base = 0; base < total; base += kCommitThreads * kCommitBatch) {
      uint4 v[kCommitBatch];
      size_t dst[kCommitBatch];
#pragma unroll
      for (int j = 0; j < kCommitBatch; ++j) {
        const int e = base + j * kCommitThreads + tid;
        if (e < total) {
          const int t = e >= per;              // 0: keys, 1: values
          const int y = e - t * per;
          const int r = y / row_units;
          const int rem = y - r * row_units;
          const int g = rem / upr;
          const int c = rem - g * upr;
          const uint4* src = t ? vt : kt;
          v[j] = src[((size_t)b * n + s_nodes[r]) * row_units + rem];
          dst[j] = (((size_t)b * hkv + g) * max_prefix + L + r) * upr + c;
        }
      }
#pragma unroll
      for (int j = 0; j < kCommitBatch; ++j) {
        const int e = base + j * kCommitThreads + tid;
        if (e < total) (e >= per ? vp : kp)[dst[j]] = v[j];
      }
    }
    if (tid == 0) prefix_len[b] = L + a + 1;
  } else {
    const int r = part - 1;
    uint4* out = feat + ((size_t)b * (D + 1) + r) * hunits;
    if (a >= 0 && r <= a) {
      const uint4* src = x + ((size_t)b * n + s_nodes[r]) * hunits;
#pragma unroll 4
      for (int c = tid; c < hunits; c += kCommitThreads) out[c] = src[c];
    } else {
      const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll 4
      for (int c = tid; c < hunits; c += kCommitThreads) out[c] = zero;
    }
  }
}

}  // namespace

hipError_t launch_commit(int B, int n, int hkv, int head_dim, int max_prefix, int hidden, int D, int esz,
                         const int32_t* accept_len, const int32_t* accept_path, const void* kt, const void* vt,
                         const void* x, void* kp, void* vp, int32_t* prefix_len, void* feat, int32_t* status,
                         hipStream_t st) {
  const dim3 grid(B, D + 2);
  commit_kernel<<<grid, kCommitThreads, 0, st>>>(
      n, hkv, head_dim * esz / 16, max_prefix, hidden * esz / 16, D, accept_len, accept_path,
      static_cast<const uint4*>(kt), static_cast<const uint4*>(vt), static_cast<const uint4*>(x),
      static_cast<uint4*>(kp), static_cast<uint4*>(vp), prefix_len, static_cast<uint4*>(feat), status);
  return hipGetLastError();
}

}  // namespace eagle
