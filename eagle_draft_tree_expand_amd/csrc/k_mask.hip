// Ancestor-only tree mask (EAGLE-2 notes, "Tree Attention Mask": a flattened
// token sees only its ancestors, never another branch), the per-token row
// gather that supplies tree queries/keys/values, and a small fill kernel.
#include "common.h"
#include "kernels.h"

namespace eagle {

namespace {

constexpr int kMaxWords = (EAGLE_MAX_NODES + 63) / 64;

// grid B, one thread per node: walk the parent chain (depth <= D), set bits.
__global__ __launch_bounds__(256) void tree_mask_kernel(int n, int W, const int32_t* __restrict__ parent,
                                                        const int32_t* __restrict__ depth,
                                                        const int32_t* __restrict__ prefix_len,
                                                        uint64_t* __restrict__ mask, int32_t* __restrict__ pos,
                                                        int32_t* status) {
  const int b = blockIdx.x;
  const int32_t* par = parent + (size_t)b * n;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t words[kMaxWords];
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) words[w] = 0;
    bool bad = false;
    int j = i;
    for (int steps = 0; steps <= n; ++steps) {
      words[j >> 6] |= 1ull << (j & 63);
      const int pj = par[j];
      if (j == 0) { bad = pj != -1; break; }
      if (pj < 0 || pj >= j) { bad = true; break; }
      j = pj;
    }
    if (bad) {
#pragma unroll
      for (int w = 0; w < kMaxWords; ++w) words[w] = 0;
      words[i >> 6] = 1ull << (i & 63);
      set_status(status, EAGLE_STATUS_BAD_TREE);
    }
    for (int w = 0; w < W; ++w) mask[((size_t)b * n + i) * W + w] = words[w];
    pos[(size_t)b * n + i] = prefix_len[b] + depth[(size_t)b * n + i];
  }
}

// grid (x, n_tables): out_t[r, :] = table_t[idx[r], :] for every table t of
// the set (one launch for several tables sharing the ids).
template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(int n_rows, GatherSet gs, int table_rows,
                                                     const int32_t* __restrict__ idx, int32_t* status) {
  const int ti = blockIdx.y;
  const int row_vecs = gs.row_units[ti];
  const V* __restrict__ table = static_cast<const V*>(gs.table[ti]);
  V* __restrict__ out = static_cast<V*>(gs.out[ti]);
  const size_t total = (size_t)n_rows * row_vecs;
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < total; x += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(x / row_vecs);
    const int c = (int)(x - (size_t)r * row_vecs);
    const int t = idx[r];
    V v;
    if (t >= 0 && t < table_rows) {
      v = table[(size_t)t * row_vecs + c];
    } else {
      memset(&v, 0, sizeof(V));
      if (c == 0 && ti == 0) set_status(status, EAGLE_STATUS_TOKEN_RANGE);
    }
    out[x] = v;
  }
}

__global__ void zero_kernel(int32_t* p, size_t n) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) p[x] = 0;
}

}  // namespace

hipError_t launch_tree_mask(int B, int n, const int32_t* parent, const int32_t* depth, const int32_t* prefix_len,
                            uint64_t* mask, int32_t* pos, int32_t* status, hipStream_t st) {
  const int W = (n + 63) / 64;
  tree_mask_kernel<<<B, 256, 0, st>>>(n, W, parent, depth, prefix_len, mask, pos, status);
  return hipGetLastError();
}

hipError_t launch_gather(int n_rows, GatherSet gs, int table_rows, const int32_t* idx, int32_t* status,
                         hipStream_t st) {
  // gs.row_units holds row bytes on entry; the widest access every table allows is used for all
  if (n_rows == 0 || gs.n == 0) return hipSuccess;
  uintptr_t addr = 0;
  int common = 0, maxb = 0;
  for (int t = 0; t < gs.n; ++t) {
    addr |= (uintptr_t)gs.table[t] | (uintptr_t)gs.out[t];
    common |= gs.row_units[t];
    maxb = gs.row_units[t] > maxb ? gs.row_units[t] : maxb;
  }
  const int w = ((common % 16) == 0 && (addr & 15u) == 0) ? 16 : ((common % 4) == 0 && (addr & 3u) == 0) ? 4 : 2;
  for (int t = 0; t < gs.n; ++t) gs.row_units[t] /= w;
  const size_t total = (size_t)n_rows * (maxb / w);
  const int gx = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  const dim3 grid(gx, gs.n);
  if (w == 16) gather_kernel<uint4><<<grid, 256, 0, st>>>(n_rows, gs, table_rows, idx, status);
  else if (w == 4) gather_kernel<uint32_t><<<grid, 256, 0, st>>>(n_rows, gs, table_rows, idx, status);
  else gather_kernel<uint16_t><<<grid, 256, 0, st>>>(n_rows, gs, table_rows, idx, status);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  zero_kernel<<<grid, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

}  // namespace eagle
