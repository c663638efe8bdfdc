// Visibility masks of the draft rows: ancestor bitmasks of draft trees, and
// causal or bidirectional masks of draft blocks.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "feat(activevln): grammar-trie tree speculation with
// exact acceptance" — all trie nodes are verified in one tree-attention
// forward, each seeing itself and its ancestors. The mask is built once per
// step and shared by every layer's attention call.
//
// One workgroup per sequence, one lane per tree row. Rows are topologically
// ordered (parent[i] < i, checked), so row i's mask is the set of rows met
// walking parent links from i to the root: each lane follows its own chain
// through the parent array held in LDS (at most i steps), with no barrier
// per tree level. depth[i] is the number of links walked.
#include "tv_common.h"

namespace {

constexpr int kMaxWords = TV_MAX_TREE / 32;

__global__ __launch_bounds__(TV_MAX_TREE) void build_tree_mask_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int W,
    uint32_t* __restrict__ mask, int32_t* __restrict__ depth, int32_t* __restrict__ row_status) {
  __shared__ int32_t s_par[TV_MAX_TREE];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int64_t row = static_cast<int64_t>(b) * T + i;
  // Both loads are issued together; neither address depends on the other.
  const int n = n_nodes[b];
  const int p = (i > 0 && i < T) ? parent[row] : -1;
  const bool nn_ok = (n >= 0 && n <= T);
  const bool live = nn_ok && i < n;
  const bool bad = live && i > 0 && (p < 0 || p >= i);
  s_par[i] = live ? p : -1;
  const bool any_bad = __syncthreads_or(bad) != 0;
  const bool ok = nn_ok && !any_bad;

  uint32_t m[kMaxWords];
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) m[w] = 0u;
  int d = -1;
  if (ok && live) {
    int cur = i;
    d = 0;
    for (;;) {
#pragma unroll
      for (int w = 0; w < kMaxWords; ++w) m[w] |= (cur >> 5) == w ? (1u << (cur & 31)) : 0u;
      if (cur == 0) break;
      cur = s_par[cur];
      ++d;
    }
  }
  if (i < T) {
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w < W) mask[row * W + w] = m[w];
    depth[row] = d;
  }
  if (i == 0) row_status[b] = !nn_ok ? TV_ROW_NNODES : (any_bad ? TV_ROW_BAD_PARENT : TV_ROW_OK);
}

// Draft blocks instead of trees (the FlashRT page "Alpamayo 1.5 on Thor:
// full-request engine with precision presets and FlashDrive streaming
// backend": the DFlash block rows attend over the context plus the block
// keys). Causal: row i sees block rows 0..i (a linear draft); bidirectional:
// every live row sees every live row. One lane per row writes its words.
__global__ __launch_bounds__(TV_MAX_TREE) void build_block_mask_kernel(
    const int32_t* __restrict__ n_nodes, int T, int W, int mode, uint32_t* __restrict__ mask,
    int32_t* __restrict__ position, int32_t* __restrict__ row_status) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  if (i >= T) return;
  const int64_t row = static_cast<int64_t>(b) * T + i;
  const int n = n_nodes[b];
  const bool nn_ok = (n >= 0 && n <= T);
  const bool live = nn_ok && i < n;
  // Bits 0..last of the row are set (none on padding rows).
  const int last = !live ? -1 : (mode == TV_BLOCK_CAUSAL ? i : n - 1);
  for (int w = 0; w < W; ++w) {
    const int lo = 32 * w;
    uint32_t m = 0u;
    if (last >= lo + 31)
      m = 0xFFFFFFFFu;
    else if (last >= lo)
      m = (2u << (last - lo)) - 1u;
    mask[row * W + w] = m;
  }
  position[row] = live ? i : -1;
  if (i == 0) row_status[b] = nn_ok ? TV_ROW_OK : TV_ROW_NNODES;
}

}  // namespace

extern "C" int tv_build_block_mask(const int32_t* n_nodes, int B, int T, int mode,
                                   uint32_t* mask, int32_t* position, int32_t* row_status,
                                   hipStream_t stream) {
  if (!n_nodes || !mask || !position || !row_status) return TV_ERR_NULL;
  if (B < 0 || T < 1 || T > TV_MAX_TREE) return TV_ERR_SHAPE;
  if (mode != TV_BLOCK_CAUSAL && mode != TV_BLOCK_BIDIRECTIONAL) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  const int W = (T + 31) / 32;
  hipLaunchKernelGGL(build_block_mask_kernel, dim3(B), dim3(TV_MAX_TREE), 0, stream, n_nodes, T,
                     W, mode, mask, position, row_status);
  return tvh::launch_status();
}

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
