// Adaptive draft budget: the number of draft nodes each sequence verifies in
// the next step, steered toward a target acceptance ratio, and the packed row
// table that step's ragged query rows use.
//
// Page: IluvatarLabs/vllm "Introduce SCV vectorized masking with
// graph/adaptive modes" — the adaptive mode adjusts the number of speculative
// tokens from recent acceptance ratios so as to hold a target ratio, and the
// follow-up commits remove the per-request device-to-host syncs of the
// acceptance bookkeeping. Here the controller never leaves the device: it
// reads the acceptance results where the verification left them and writes
// the next budgets and row starts where the next step reads them.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "perf(activevln): pack batched prefill turns back to
// back in CUDA graphs" — the packed rows of a batch are described by per-row
// starts; here row_start[b] is the exclusive prefix sum of the next step's
// row counts (budget + 1: the draft nodes and the root).
//
// Per sequence with n >= 2 verified rows, a valid accept length a and a good
// status: ratio = a / (n - 1); ema += alpha (ratio - ema); budget moves one
// step up if ema > target, one step down if ema < target, clamped to
// [n_min, n_max]. Every floating-point operation is a single fp32 operation
// rounded to nearest (no contraction), so the result is reproducible bit for
// bit by any IEEE fp32 evaluation in the same order.
#include "tv_common.h"

namespace {

constexpr int kThreadsBudget = 1024;

__global__ __launch_bounds__(kThreadsBudget) void adapt_budget_kernel(
    const int32_t* __restrict__ accept_len, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ status, int B, float target, float alpha, int n_min, int n_max,
    float* __restrict__ ema, int32_t* __restrict__ budget, int32_t* __restrict__ row_start,
    int32_t* __restrict__ rows_total) {
#pragma clang fp contract(off)
  __shared__ int s_wave[kThreadsBudget / tv::kWave];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  for (int b0 = 0; b0 < B; b0 += kThreadsBudget) {
    const int b = b0 + tid;
    int rows = 0;
    if (b < B) {
      const int n = n_nodes[b];
      const int a = accept_len[b];
      const bool ok = status == nullptr || status[b] == TV_ROW_OK;
      float e = ema[b];
      int nb = budget[b];
      if (ok && n >= 2 && a >= 0 && a <= n - 1) {
        const float ratio = static_cast<float>(a) / static_cast<float>(n - 1);
        const float diff = ratio - e;
        const float step = alpha * diff;
        e = e + step;
        nb += (e > target) ? 1 : ((e < target) ? -1 : 0);
        nb = min(max(nb, n_min), n_max);
        ema[b] = e;
        budget[b] = nb;
      } else {
        // Unchanged state; a budget outside the bounds is still clamped so
        // the row table below is always sized within them.
        nb = min(max(nb, n_min), n_max);
        budget[b] = nb;
      }
      rows = nb + 1;
    }
    // Exclusive prefix sum of rows over the block, plus the running carry.
    int inc = rows;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (b < B) row_start[b] = before + inc - rows;
    __syncthreads();
    if (tid == kThreadsBudget - 1) s_carry = before + inc;
    __syncthreads();
  }
  if (tid == 0) rows_total[0] = s_carry;
}

}  // namespace

extern "C" int tv_adapt_tree_budget(const int32_t* accept_len, const int32_t* n_nodes,
                                    const int32_t* row_status, int B, float target, float alpha,
                                    int n_min, int n_max, float* ratio_ema, int32_t* budget,
                                    int32_t* row_start, int32_t* rows_total,
                                    hipStream_t stream) {
  if (!rows_total) return TV_ERR_NULL;
  if (B < 0) return TV_ERR_SHAPE;
  if (B > 0 && (!accept_len || !n_nodes || !ratio_ema || !budget || !row_start))
    return TV_ERR_NULL;
  if (!(target >= 0.f && target <= 1.f) || !(alpha > 0.f && alpha <= 1.f)) return TV_ERR_SHAPE;
  if (n_min < 1 || n_max < n_min || n_max > TV_MAX_TREE - 1) return TV_ERR_SHAPE;
  if (static_cast<int64_t>(B) * TV_MAX_TREE > INT32_MAX) return TV_ERR_SHAPE;
  hipLaunchKernelGGL(adapt_budget_kernel, dim3(1), dim3(kThreadsBudget), 0, stream, accept_len,
                     n_nodes, row_status, B, target, alpha, n_min, n_max, ratio_ema, budget,
                     row_start, rows_total);
  return tvh::launch_status();
}
