// Accepted-path KV commit: after acceptance the keys and values of the
// accepted tree rows become contiguous committed context.
//
// Pages: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "perf(activevln): lossless batched replay throughput
// options", item incremental_kv_commit (only the new turn is copied into the
// owned KV buffers); IluvatarLabs/vllm "Introduce SCV vectorized masking with
// graph/adaptive modes" (a commit kernel for accepted drafts over NHD and
// HND cache layouts).
//
// Slot ctx_len + k takes what slot ctx_len + path[k] held, k = 1..accept_len
// (slot ctx_len holds the root already). A path leaves the root through
// strictly increasing node indices, so path[k] >= k: walking k upwards and
// reading every source before writing its destination never reads a slot
// that was already overwritten, which lets the copy run in place.
//
// MI355X: one wave per (layer, sequence, KV head); lane j owns the 16-byte
// column j of the K rows (j < C) or of the V rows (C <= j < 2C), C = row
// bytes / 16. A lane touches only its own column, so no two lanes depend on
// each other and the wave needs no barrier. Up to 16 rows are loaded before
// their stores are issued.
#include "tv_common.h"

namespace {

constexpr int kBatch = 16;

struct CommitParams {
  char* k;
  char* v;
  int64_t layer_stride, kv_sb, kv_sh, kv_ss;  // bytes
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const int32_t* accept_len;
  const int32_t* path;
  int B, T, Hkv, row_chunks, kv_capacity;
  int32_t* new_ctx_len;
  int32_t* row_status;
};

__global__ __launch_bounds__(64) void commit_kv_kernel(CommitParams p) {
  const int lane = threadIdx.x;
  const int bg = blockIdx.x;
  const int layer = blockIdx.y;
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  // Lengths and the whole path row in one round trip: lane j holds path[j]
  // in pv0 and path[64 + j] in pv1 (T <= 128; indices past T re-read the
  // last entry and are never used).
  const int32_t* pr = p.path + static_cast<int64_t>(b) * p.T;
  const int n = p.n_nodes[b];
  const int L = p.ctx_len[b];
  const int a = p.accept_len[b];
  const int pv0 = pr[min(lane, p.T - 1)];
  const int pv1 = pr[min(lane + 64, p.T - 1)];
  int st = TV_ROW_OK;
  if (n < 0 || n > p.T) {
    st = TV_ROW_NNODES;
  } else if (n > 0) {
    if (L < 0 || static_cast<int64_t>(L) + n > p.kv_capacity) {
      st = TV_ROW_CTX_BOUND;
    } else if (a < 0 || a > n - 1) {
      st = TV_ROW_BAD_PATH;
    } else {
      // path[0] = 0 and path[k-1] < path[k] < n for k = 1..a (lane k checks k
      // and, in the second half, 64 + k).
      const int prev0 = __shfl_up(pv0, 1);
      const int last0 = __shfl(pv0, 63);
      const int up1 = __shfl_up(pv1, 1);
      const int prev1 = lane == 0 ? last0 : up1;
      bool ok = true;
      if (lane <= a) ok = lane == 0 ? pv0 == 0 : (prev0 < pv0 && pv0 < n);
      if (lane + 64 <= a) ok = ok && prev1 < pv1 && pv1 < n;
      if (!__all(ok)) st = TV_ROW_BAD_PATH;
    }
  }
  if (layer == 0 && g == 0 && lane == 0) {
    p.row_status[b] = st;
    p.new_ctx_len[b] = (st == TV_ROW_OK && n > 0) ? L + a + 1 : L;
  }
  if (st != TV_ROW_OK || n == 0 || a == 0) return;
  const int C = p.row_chunks;
  if (lane >= 2 * C) return;
  char* base = (lane < C ? p.k : p.v) + layer * p.layer_stride + b * p.kv_sb + g * p.kv_sh +
               static_cast<int64_t>(lane < C ? lane : lane - C) * 16;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  for (int k0 = 1; k0 <= a; k0 += kBatch) {
    u32x4_t row[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int kk = k0 + j;
      if (kk <= a) {
        const int src = kk < 64 ? __builtin_amdgcn_readlane(pv0, kk)
                                : __builtin_amdgcn_readlane(pv1, kk - 64);
        row[j] = *reinterpret_cast<const u32x4_t*>(base + (L + src) * p.kv_ss);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int kk = k0 + j;
      if (kk <= a) *reinterpret_cast<u32x4_t*>(base + (L + kk) * p.kv_ss) = row[j];
    }
  }
}

}  // namespace

extern "C" int tv_commit_accepted_kv(void* k, void* v, int64_t layer_stride, int64_t kv_sb,
                                     int64_t kv_sh, int64_t kv_ss, const int32_t* ctx_len,
                                     const int32_t* n_nodes, const int32_t* accept_len,
                                     const int32_t* path, int B, int T, int Hkv, int D,
                                     int elem_bytes, int layers, int kv_capacity,
                                     int32_t* new_ctx_len, int32_t* row_status,
                                     hipStream_t stream) {
  if (!k || !v || !ctx_len || !n_nodes || !accept_len || !path || !new_ctx_len || !row_status)
    return TV_ERR_NULL;
  if (elem_bytes != 2 && elem_bytes != 4) return TV_ERR_DTYPE;
  if (B < 0 || T < 1 || T > TV_MAX_TREE || Hkv < 1 || D < 1 || layers < 1 || kv_capacity < 1)
    return TV_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(D) * elem_bytes;
  if (row_bytes % 16 || row_bytes / 16 > 32) return TV_ERR_UNSUPPORTED;
  if (!tvh::aligned16(k) || !tvh::aligned16(v)) return TV_ERR_ALIGN;
  const int64_t strides[4] = {layer_stride, kv_sb, kv_sh, kv_ss};
  for (const int64_t s : strides)
    if (s < 0 || (s * elem_bytes) % 16) return TV_ERR_ALIGN;
  if (static_cast<const void*>(new_ctx_len) == static_cast<const void*>(ctx_len))
    return TV_ERR_SHAPE;
  if (B == 0) return TV_OK;
  if (static_cast<int64_t>(B) * Hkv > INT32_MAX || layers > 65535) return TV_ERR_SHAPE;
  CommitParams p;
  p.k = static_cast<char*>(k);
  p.v = static_cast<char*>(v);
  p.layer_stride = layer_stride * elem_bytes;
  p.kv_sb = kv_sb * elem_bytes;
  p.kv_sh = kv_sh * elem_bytes;
  p.kv_ss = kv_ss * elem_bytes;
  p.ctx_len = ctx_len;
  p.n_nodes = n_nodes;
  p.accept_len = accept_len;
  p.path = path;
  p.B = B;
  p.T = T;
  p.Hkv = Hkv;
  p.row_chunks = static_cast<int>(row_bytes / 16);
  p.kv_capacity = kv_capacity;
  p.new_ctx_len = new_ctx_len;
  p.row_status = row_status;
  hipLaunchKernelGGL(commit_kv_kernel, dim3(B * Hkv, layers), dim3(64), 0, stream, p);
  return tvh::launch_status();
}
