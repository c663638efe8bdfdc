// Exact acceptance of a verified draft tree: greedy argmax walk and
// SpecInfer-style rejection sampling.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "feat(activevln): grammar-trie tree speculation with
// exact acceptance": greedy decoding keeps the argmax path, sampling runs
// standard rejection sampling against the draft so the output distribution
// is unchanged (the page's summary calls it exact SpecInfer-style
// acceptance). The accept-mask output is the vectorised accepted-token mask
// of the IluvatarLabs/vllm page "Introduce SCV vectorized masking with
// graph/adaptive modes".
//
// Both modes are two launches:
//   1. a data-parallel pass over the live logits rows, split along the
//      vocabulary so the whole chip streams the rows once (16-byte loads):
//      greedy keeps a (max, lowest index) pair per slice; sampling keeps the
//      slice max and the float64 sum of exp((l - max) / tau);
//   2. one workgroup per sequence merges the slices and walks the tree.
// Sequences with n_nodes == 0 read nothing.
#include <limits.h>

#include "tv_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 16384;   // vocabulary entries per slice
constexpr int kMaxSplits = 64;
constexpr int kWalkThreads = 1024;

struct ArgBest {
  float v;
  int i;
};

int num_splits(int V) {
  int s = (V + kSlice - 1) / kSlice;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return s;
}

// Slice [lo, hi) of split s.
__device__ __forceinline__ void slice_bounds(int V, int S, int s, int& lo, int& hi) {
  int span = (V + S - 1) / S;
  span = (span + 3) & ~3;
  lo = s * span;
  hi = min(V, lo + span);
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ bool live_row(const int32_t* n_nodes, int T, int b, int j) {
  const int n = n_nodes[b];
  return n > 0 && n <= T && j < n;
}

// ------------------------------------------------------------- greedy ---

__global__ __launch_bounds__(kThreads) void argmax_slices_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ n_nodes, int T,
    int V, int S, ArgBest* __restrict__ part) {
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  if (!live_row(n_nodes, T, b, j)) return;
  int lo, hi;
  slice_bounds(V, S, s, lo, hi);
  const float* row = logits + (static_cast<int64_t>(b) * T + j) * stride;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const int tid = threadIdx.x;
  // Rows need not be 16-byte aligned: up to 3 leading elements are read as
  // scalars, the body with 16-byte loads, the last < 4 elements as scalars.
  // Every thread sees its elements in increasing index order (head, body,
  // tail), so a strict comparison keeps the lowest index among its equal
  // maxima.
  const int mis = static_cast<int>((reinterpret_cast<uintptr_t>(row + lo) >> 2) & 3);
  const int lo_al = min(hi, lo + ((4 - mis) & 3));
  if (lo + tid < lo_al) {
    bv = row[lo + tid];
    bi = lo + tid;
  }
  int v0 = lo_al + 4 * tid;
  const int hi4 = lo_al + ((hi - lo_al) & ~3);
  for (; v0 + 4 * kThreads * 3 < hi4; v0 += 4 * kThreads * 4) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(row + v0 + 4 * kThreads * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int base = v0 + 4 * kThreads * u;
      if (x[u].x > bv || bi == INT_MAX) { bv = x[u].x; bi = base; }
      if (x[u].y > bv) { bv = x[u].y; bi = base + 1; }
      if (x[u].z > bv) { bv = x[u].z; bi = base + 2; }
      if (x[u].w > bv) { bv = x[u].w; bi = base + 3; }
    }
  }
  for (; v0 < hi4; v0 += 4 * kThreads) {
    const float4 x = *reinterpret_cast<const float4*>(row + v0);
    if (x.x > bv || bi == INT_MAX) { bv = x.x; bi = v0; }
    if (x.y > bv) { bv = x.y; bi = v0 + 1; }
    if (x.z > bv) { bv = x.z; bi = v0 + 2; }
    if (x.w > bv) { bv = x.w; bi = v0 + 3; }
  }
  const int tv = hi4 + tid;
  if (tv < hi) {
    const float x = row[tv];
    if (x > bv || bi == INT_MAX) { bv = x; bi = tv; }
  }
  // Reduce (max value, lowest index) over the workgroup.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    part[(static_cast<int64_t>(b) * T + j) * S + s] = ArgBest{bv, bi};
  }
}

// Per-sequence validation shared by both walks; returns the row status.
__device__ int validate_seq(const int32_t* parent, const int32_t* tokens, int n, int T, int V,
                            int b, int* s_flags) {
  const int tid = threadIdx.x;
  if (tid == 0) *s_flags = 0;
  __syncthreads();
  if (n < 0 || n > T) return TV_ROW_NNODES;
  for (int i = tid; i < n; i += blockDim.x) {
    if (i == 0) continue;
    const int p = parent[static_cast<int64_t>(b) * T + i];
    if (p < 0 || p >= i) atomicOr(s_flags, 1);
    const int t = tokens[static_cast<int64_t>(b) * T + i];
    if (t < 0 || t >= V) atomicOr(s_flags, 2);
  }
  __syncthreads();
  const int f = *s_flags;
  if (f & 1) return TV_ROW_BAD_PARENT;
  if (f & 2) return TV_ROW_BAD_TOKEN;
  return TV_ROW_OK;
}

// One workgroup per sequence (one thread per tree row). Every global load is
// issued up front (no load waits on another); the row argmaxes are merged
// from their slice partials eight at a time; the walk itself runs in wave 0,
// which finds the lowest-index child carrying the argmax token of the current
// node with two ballots (rows lane and lane + 64) per step.
__global__ __launch_bounds__(TV_MAX_TREE) void greedy_walk_kernel(
    const ArgBest* __restrict__ part, int S, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int V,
    int32_t* accept_len, int32_t* path, int32_t* bonus, uint8_t* accept_mask,
    int32_t* row_status) {
  __shared__ int s_flags;
  __shared__ int s_arg[TV_MAX_TREE];
  __shared__ int s_par[TV_MAX_TREE];
  __shared__ int s_tok[TV_MAX_TREE];
  __shared__ int s_path[TV_MAX_TREE];
  __shared__ int s_on[TV_MAX_TREE];
  __shared__ int s_len, s_bonus;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int64_t row = static_cast<int64_t>(b) * T + i;
  const bool in_t = i < T;
  const int n = n_nodes[b];
  const int pr = in_t ? parent[row] : -1;
  const int tk = in_t ? tokens[row] : 0;
  ArgBest best{-INFINITY, 0x7fffffff};
  if (in_t) {
    // Rows past n were never written by the slice pass: read (in bounds) but
    // unused. Clamped duplicates of the last slice never win a strict test.
    const ArgBest* pp = part + row * S;
    best = pp[0];
    for (int s0 = 1; s0 < S; s0 += 8) {
      ArgBest o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = pp[min(s0 + u, S - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (better(o[u].v, o[u].i, best.v, best.i)) best = o[u];
    }
  }
  if (i == 0) s_flags = 0;
  __syncthreads();
  const bool n_ok = n >= 0 && n <= T;
  const bool live = n_ok && i < n;
  int f = 0;
  if (live && i > 0) {
    if (pr < 0 || pr >= i) f |= 1;
    if (tk < 0 || tk >= V) f |= 2;
  }
  if (f) atomicOr(&s_flags, f);
  if (in_t) {
    s_arg[i] = best.i;
    s_par[i] = (live && i > 0) ? pr : -1;
    s_tok[i] = tk;
    s_path[i] = -1;
    s_on[i] = 0;
  }
  __syncthreads();
  const int flags = s_flags;
  const int st = !n_ok ? TV_ROW_NNODES
                       : ((flags & 1) ? TV_ROW_BAD_PARENT
                                      : ((flags & 2) ? TV_ROW_BAD_TOKEN : TV_ROW_OK));
  if (st != TV_ROW_OK || n == 0) {
    if (in_t) {
      path[row] = -1;
      accept_mask[row] = 0;
    }
    if (i == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
      row_status[b] = st;
    }
    return;
  }
  if (i < tv::kWave) {
    const int c1 = i, c2 = i + tv::kWave;  // candidate child rows of this lane
    int cur = 0, len = 0;
    if (i == 0) {
      s_path[0] = 0;
      s_on[0] = 1;
    }
    for (;;) {
      const int a = s_arg[cur];
      const bool m1 = c1 > cur && c1 < n && s_par[c1] == cur && s_tok[c1] == a;
      const bool m2 = c2 > cur && c2 < n && s_par[c2] == cur && s_tok[c2] == a;
      const uint64_t b1 = __ballot(m1);
      const uint64_t b2 = __ballot(m2);
      if (b1 == 0 && b2 == 0) {
        if (i == 0) s_bonus = a;
        break;
      }
      cur = b1 ? __builtin_ctzll(b1) : tv::kWave + __builtin_ctzll(b2);
      ++len;
      if (i == 0) {
        s_path[len] = cur;
        s_on[cur] = 1;
      }
    }
    if (i == 0) s_len = len;
  }
  __syncthreads();
  if (in_t) {
    path[row] = s_path[i];
    accept_mask[row] = static_cast<uint8_t>(s_on[i]);
  }
  if (i == 0) {
    accept_len[b] = s_len;
    bonus[b] = s_bonus;
    row_status[b] = TV_ROW_OK;
  }
}

// ----------------------------------------------------------- sampling ---

struct StatPart {
  double m;  // slice max of the logits (a float32 value)
  double z;  // sum over the slice of exp((l - m) / tau)
};

__global__ __launch_bounds__(kThreads) void softmax_slices_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ n_nodes, int T,
    int V, int S, double tau, StatPart* __restrict__ part) {
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  if (!live_row(n_nodes, T, b, j)) return;
  int lo, hi;
  slice_bounds(V, S, s, lo, hi);
  const float* row = logits + (static_cast<int64_t>(b) * T + j) * stride;
  const int tid = threadIdx.x;
  __shared__ float smax[kThreads / 64];
  __shared__ double ssum[kThreads / 64];
  float m = -INFINITY;
  for (int v = lo + tid; v < hi; v += kThreads) m = fmaxf(m, row[v]);
  m = tv::wave_max(m);
  if ((tid & 63) == 0) smax[tid >> 6] = m;
  __syncthreads();
  m = smax[0];
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, smax[w]);
  const double md = static_cast<double>(m);
  double z = 0.0;
  for (int v = lo + tid; v < hi; v += kThreads) z += exp((static_cast<double>(row[v]) - md) / tau);
  z = tv::wave_sum_f64(z);
  if ((tid & 63) == 0) ssum[tid >> 6] = z;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += ssum[w];
    part[(static_cast<int64_t>(b) * T + j) * S + s] = StatPart{md, t};
  }
}

// Block-wide float64 sum for kWalkThreads threads; every thread gets it.
__device__ double block_sum_f64(double x, double* s_red) {
  x = tv::wave_sum_f64(x);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) s_red[tid >> 6] = x;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kWalkThreads / 64; ++w) t += s_red[w];
  return t;
}

__global__ __launch_bounds__(kWalkThreads) void sample_walk_kernel(
    const StatPart* __restrict__ part, int S, const float* __restrict__ logits,
    int64_t lstride, const float* __restrict__ q, int64_t qstride,
    const float* __restrict__ u, double tau, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int V,
    double* __restrict__ resid, int32_t* accept_len, int32_t* path, int32_t* bonus,
    uint8_t* accept_mask, int8_t* decision, int32_t* row_status) {
  __shared__ int s_flags;
  __shared__ double s_m[TV_MAX_TREE], s_z[TV_MAX_TREE];
  __shared__ int s_par[TV_MAX_TREE], s_tok[TV_MAX_TREE], s_path[TV_MAX_TREE];
  __shared__ double s_red[kWalkThreads / 64];
  __shared__ int s_accept;
  __shared__ int s_cand;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = n_nodes[b];
  const int st = validate_seq(parent, tokens, n, T, V, b, &s_flags);
  const int64_t rbase = static_cast<int64_t>(b) * T;
  if (st != TV_ROW_OK || n == 0) {
    if (tid < T) {
      path[rbase + tid] = -1;
      accept_mask[rbase + tid] = 0;
      decision[rbase + tid] = -1;
    }
    if (tid == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
      row_status[b] = st;
    }
    return;
  }
  if (tid < n) {
    const StatPart* pp = part + (rbase + tid) * S;
    double M = pp[0].m;
    for (int s = 1; s < S; ++s) M = fmax(M, pp[s].m);
    double Z = 0.0;
    for (int s = 0; s < S; ++s) Z += pp[s].z * exp((pp[s].m - M) / tau);
    s_m[tid] = M;
    s_z[tid] = Z;
    s_par[tid] = tid == 0 ? -1 : parent[rbase + tid];
    s_tok[tid] = tokens[rbase + tid];
  }
  if (tid < T) {
    s_path[tid] = -1;
    decision[rbase + tid] = -1;
  }
  __syncthreads();

  // The residual r is either p_cur (implicit: recomputed from the logits
  // row) or held, normalised, in one of two float64 buffers of V entries.
  double* buf[2] = {resid + static_cast<int64_t>(b) * 2 * V,
                    resid + static_cast<int64_t>(b) * 2 * V + V};
  int cur = 0, len = 0, held = -1;  // held: index of the buffer holding r, -1 = implicit
  if (tid == 0) s_path[0] = 0;

  auto r_at = [&](int x) -> double {
    if (held < 0) {
      const double l = static_cast<double>(logits[(rbase + cur) * lstride + x]);
      return exp((l - s_m[cur]) / tau) / s_z[cur];
    }
    return buf[held][x];
  };

  for (;;) {
    bool accepted = false;
    for (int c = cur + 1; c < n; ++c) {
      if (s_par[c] != cur) continue;
      const int x = s_tok[c];
      if (tid == 0) {
        const double rx = r_at(x);
        const double qx = static_cast<double>(q[(rbase + c) * qstride + x]);
        double ratio;
        if (rx == 0.0)
          ratio = 0.0;
        else if (qx == 0.0)
          ratio = INFINITY;
        else
          ratio = rx / qx;
        const int acc = static_cast<double>(u[rbase + c]) < ratio ? 1 : 0;
        decision[rbase + c] = static_cast<int8_t>(acc);
        s_accept = acc;
      }
      __syncthreads();
      const int acc = s_accept;
      __syncthreads();
      if (acc) {
        ++len;  // uniform: every thread follows the same walk
        if (tid == 0) s_path[len] = c;
        cur = c;
        held = -1;
        accepted = true;
        break;
      }
      // Rejected: r <- max(r - q_c, 0) / sum, into the free buffer.
      const int dst = held == 0 ? 1 : 0;
      const float* qrow = q + (rbase + c) * qstride;
      double part_sum = 0.0;
      for (int v = tid; v < V; v += kWalkThreads) {
        const double res = fmax(r_at(v) - static_cast<double>(qrow[v]), 0.0);
        buf[dst][v] = res;
        part_sum += res;
      }
      const double tot = block_sum_f64(part_sum, s_red);
      if (tot > 0.0) {
        for (int v = tid; v < V; v += kWalkThreads) buf[dst][v] = buf[dst][v] / tot;
        __syncthreads();
        held = dst;
      }
    }
    if (!accepted) break;
  }
  __syncthreads();
  const int plen = len;

  // Bonus: smallest x with sum_{y<=x} r(y) > u0 * sum_y r(y). Each thread
  // owns a contiguous range of the vocabulary.
  const int per = (V + kWalkThreads - 1) / kWalkThreads;
  const int lo = min(V, tid * per);
  const int hi = min(V, lo + per);
  double mine = 0.0;
  for (int v = lo; v < hi; ++v) mine += r_at(v);
  // Exclusive prefix over threads: wave scan then across waves.
  double incl = mine;
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  double excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.0;
  __syncthreads();
  if (lane == 63) s_red[tid >> 6] = incl;
  __syncthreads();
  double wave_off = 0.0, total = 0.0;
  for (int w = 0; w < kWalkThreads / 64; ++w) {
    if (w < (tid >> 6)) wave_off += s_red[w];
    total += s_red[w];
  }
  const double u0 = static_cast<double>(u[rbase]);
  const double thr = u0 * total;
  double run = wave_off + excl;
  int cand = INT_MAX;
  for (int v = lo; v < hi; ++v) {
    run += r_at(v);
    if (run > thr) {
      cand = v;
      break;
    }
  }
  if (tid == 0) s_cand = INT_MAX;
  __syncthreads();
  if (cand != INT_MAX) atomicMin(&s_cand, cand);
  __syncthreads();
  int bon = s_cand;
  if (bon == INT_MAX) {
    // Rounding left the threshold above every running sum (u0 within an ulp
    // of 1): take the last token with positive mass.
    int lastpos = -1;
    for (int v = lo; v < hi; ++v)
      if (r_at(v) > 0.0) lastpos = v;
    if (tid == 0) s_cand = -1;
    __syncthreads();
    if (lastpos >= 0) atomicMax(&s_cand, lastpos);
    __syncthreads();
    bon = s_cand;
  }

  if (tid < T) {
    path[rbase + tid] = s_path[tid];
    bool on = false;
    for (int k = 0; k <= plen; ++k) on |= (s_path[k] == tid);
    accept_mask[rbase + tid] = on ? 1 : 0;
  }
  if (tid == 0) {
    accept_len[b] = plen;
    bonus[b] = bon;
    row_status[b] = TV_ROW_OK;
  }
}

bool accept_sizes_ok(int B, int T, int V) {
  return B >= 0 && T >= 1 && T <= TV_MAX_TREE && V >= 1;
}

size_t greedy_ws(int B, int T, int V) {
  return tvh::align_up(static_cast<size_t>(B) * T * num_splits(V) * sizeof(ArgBest), 256);
}

size_t sample_ws(int B, int T, int V) {
  return tvh::align_up(static_cast<size_t>(B) * T * num_splits(V) * sizeof(StatPart), 256) +
         tvh::align_up(static_cast<size_t>(B) * 2 * V * sizeof(double), 256);
}

}  // namespace

extern "C" size_t tv_accept_workspace_size(int B, int T, int V, int mode) {
  if (!accept_sizes_ok(B, T, V) || (mode != 0 && mode != 1)) return static_cast<size_t>(-1);
  return mode == 0 ? greedy_ws(B, T, V) : sample_ws(B, T, V);
}

extern "C" int tv_accept_greedy(const float* logits, int64_t logits_row_stride,
                                const int32_t* tokens, const int32_t* parent,
                                const int32_t* n_nodes, int B, int T, int V, int32_t* accept_len,
                                int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                                void* workspace, size_t ws_bytes, int32_t* row_status,
                                hipStream_t stream) {
  if (!logits || !tokens || !parent || !n_nodes || !accept_len || !path || !bonus ||
      !accept_mask || !row_status)
    return TV_ERR_NULL;
  if (!accept_sizes_ok(B, T, V) || logits_row_stride < V) return TV_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(logits) & 3u) return TV_ERR_ALIGN;
  if (B == 0) return TV_OK;
  if (!workspace || ws_bytes < greedy_ws(B, T, V) || !tvh::aligned256(workspace))
    return TV_ERR_WORKSPACE;
  const int S = num_splits(V);
  ArgBest* part = static_cast<ArgBest*>(workspace);
  hipLaunchKernelGGL(argmax_slices_kernel, dim3(S, T, B), dim3(kThreads), 0, stream, logits,
                     logits_row_stride, n_nodes, T, V, S, part);
  hipLaunchKernelGGL(greedy_walk_kernel, dim3(B), dim3(TV_MAX_TREE), 0, stream, part, S, tokens,
                     parent, n_nodes, T, V, accept_len, path, bonus, accept_mask, row_status);
  return tvh::launch_status();
}

extern "C" int tv_accept_sample(const float* logits, int64_t logits_row_stride,
                                float temperature, const float* q, int64_t q_row_stride,
                                const float* u, const int32_t* tokens, const int32_t* parent,
                                const int32_t* n_nodes, int B, int T, int V,
                                int32_t* accept_len, int32_t* path, int32_t* bonus,
                                uint8_t* accept_mask, int8_t* decision, void* workspace,
                                size_t ws_bytes, int32_t* row_status, hipStream_t stream) {
  if (!logits || !q || !u || !tokens || !parent || !n_nodes || !accept_len || !path || !bonus ||
      !accept_mask || !decision || !row_status)
    return TV_ERR_NULL;
  if (!accept_sizes_ok(B, T, V) || logits_row_stride < V || q_row_stride < V)
    return TV_ERR_SHAPE;
  if (!(temperature > 0.f)) return TV_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(q) & 3u))
    return TV_ERR_ALIGN;
  if (B == 0) return TV_OK;
  if (!workspace || ws_bytes < sample_ws(B, T, V) || !tvh::aligned256(workspace))
    return TV_ERR_WORKSPACE;
  const int S = num_splits(V);
  StatPart* part = static_cast<StatPart*>(workspace);
  double* resid = reinterpret_cast<double*>(
      static_cast<char*>(workspace) +
      tvh::align_up(static_cast<size_t>(B) * T * S * sizeof(StatPart), 256));
  const double tau = static_cast<double>(temperature);
  hipLaunchKernelGGL(softmax_slices_kernel, dim3(S, T, B), dim3(kThreads), 0, stream, logits,
                     logits_row_stride, n_nodes, T, V, S, tau, part);
  hipLaunchKernelGGL(sample_walk_kernel, dim3(B), dim3(kWalkThreads), 0, stream, part, S, logits,
                     logits_row_stride, q, q_row_stride, u, tau, tokens, parent, n_nodes, T, V,
                     resid, accept_len, path, bonus, accept_mask, decision, row_status);
  return tvh::launch_status();
}
