// Ancestor-bitmask builder for draft trees.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "feat(activevln): grammar-trie tree speculation with
// exact acceptance" — all trie nodes are verified in one tree-attention
// forward, each seeing itself and its ancestors. The mask is built once per
// step and shared by every layer's attention call.
//
// One workgroup per sequence, one lane per tree row. Rows are topologically
// ordered (parent[i] < i), so the masks are produced level by level with the
// recurrence mask[i] = mask[parent[i]] | bit(i): every pass resolves every
// row whose parent is already resolved; the number of passes is the tree
// depth + 1 and is bounded by T.
#include "tv_common.h"

namespace {

constexpr int kMaxWords = TV_MAX_TREE / 32;

__global__ __launch_bounds__(TV_MAX_TREE) void build_tree_mask_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int W,
    uint32_t* __restrict__ mask, int32_t* __restrict__ depth, int32_t* __restrict__ row_status) {
  __shared__ uint32_t s_mask[TV_MAX_TREE][kMaxWords];
  __shared__ int32_t s_depth[TV_MAX_TREE];
  __shared__ int s_bad;

  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int n = n_nodes[b];
  const bool nn_ok = (n >= 0 && n <= T);

  if (i == 0) s_bad = nn_ok ? 0 : 1;
  __syncthreads();

  int p = -1;
  const bool live = nn_ok && i < n;
  if (live && i > 0) {
    p = parent[static_cast<int64_t>(b) * T + i];
    if (p < 0 || p >= i) atomicOr(&s_bad, 2);
  }
  for (int w = 0; w < kMaxWords; ++w) s_mask[i][w] = 0u;
  s_depth[i] = -1;
  if (live && i == 0) {
    s_mask[0][0] = 1u;
    s_depth[0] = 0;
  }
  __syncthreads();

  if (s_bad == 0) {
    // Level-synchronous resolution: a row resolves once its parent has. Each
    // pass ends in a barrier that also reports whether any row is unresolved.
    for (int pass = 0; pass < T; ++pass) {
      const bool resolve = live && i > 0 && s_depth[i] < 0 && s_depth[p] >= 0;
      uint32_t m[kMaxWords];
      int d = 0;
      if (resolve) {
        for (int w = 0; w < kMaxWords; ++w) m[w] = s_mask[p][w];
        m[i >> 5] |= 1u << (i & 31);
        d = s_depth[p] + 1;
      }
      __syncthreads();
      if (resolve) {
        for (int w = 0; w < kMaxWords; ++w) s_mask[i][w] = m[w];
        s_depth[i] = d;
      }
      const bool pending = live && i > 0 && !resolve && s_depth[i] < 0;
      if (!__syncthreads_or(pending)) break;
    }
  }
  __syncthreads();

  const int64_t row = static_cast<int64_t>(b) * T + i;
  if (i < T) {
    const bool ok = (s_bad == 0);
    for (int w = 0; w < W; ++w) mask[row * W + w] = ok ? s_mask[i][w] : 0u;
    depth[row] = ok ? s_depth[i] : -1;
  }
  if (i == 0) {
    row_status[b] = (s_bad & 1) ? TV_ROW_NNODES : (s_bad ? TV_ROW_BAD_PARENT : TV_ROW_OK);
  }
}

}  // namespace

extern "C" int tv_build_tree_mask(const int32_t* parent, const int32_t* n_nodes, int B, int T,
                                  uint32_t* mask, int32_t* depth, int32_t* row_status,
                                  hipStream_t stream) {
  if (!parent || !n_nodes || !mask || !depth || !row_status) return TV_ERR_NULL;
  if (B < 0 || T < 1 || T > TV_MAX_TREE) return TV_ERR_SHAPE;
  if (B == 0) return TV_OK;
  const int W = (T + 31) / 32;
  hipLaunchKernelGGL(build_tree_mask_kernel, dim3(B), dim3(TV_MAX_TREE), 0, stream, parent,
                     n_nodes, T, W, mask, depth, row_status);
  return tvh::launch_status();
}
