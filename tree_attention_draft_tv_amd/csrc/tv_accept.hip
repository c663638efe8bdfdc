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
// greedy: two launches. A data-parallel pass over the live logits rows,
//   split along the vocabulary so the whole chip streams the rows once
//   (16-byte loads), keeps a (max, lowest index) pair per slice; one
//   workgroup per sequence merges the slices and walks the tree.
// sampling, vocabularies up to 32768: two launches. One workgroup per live
//   tree node decides, from that node's rows held in registers, which child
//   the walk accepts there and which bonus it would draw there; one
//   workgroup per sequence then follows the accepted children from the
//   root. Larger vocabularies take a slice-statistics pass and a
//   per-sequence walk.
// Sequences with n_nodes == 0 read nothing.
#include <limits.h>

#include <mutex>

#include "tv_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 16384;   // vocabulary entries per slice
constexpr int kVec = kSlice / (4 * 256);  // 16-byte loads per argmax thread per round
constexpr int kMaxSplits = 64;
constexpr int kWalkThreads = 1024;
constexpr int kBatch = 8;        // entries per thread loaded together in the walk's passes

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct ArgBest {
  float v;
  int i;
};

// Sampling slices are smaller: every entry costs a float64 exp, so the
// statistics pass wants many short, independent workgroups.
constexpr int kSliceSample = 2048;
// Vocabulary entries per thread of the node-parallel sampling path: it
// covers V <= kRegSlots * kWalkThreads.
constexpr int kRegSlots = 32;
static_assert(kSliceSample % kWalkThreads == 0, "a walk block lies in one slice");

int num_splits(int V, int slice = kSlice) {
  int s = (V + slice - 1) / slice;
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
  // The body: kVec 16-byte loads per thread issued together (one round trip
  // covers a 16384-entry slice); addresses past the body are clamped to its
  // last vector and their values ignored, so no load sits behind a branch.
  // The logits are read once: non-temporal loads.
  const int hi4 = lo_al + ((hi - lo_al) & ~3);
  for (int v0 = lo_al + 4 * tid; v0 < hi4; v0 += 4 * kThreads * kVec) {
    f32x4_t x[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u)
      x[u] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(row + min(v0 + 4 * kThreads * u, hi4 - 4)));
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int base = v0 + 4 * kThreads * u;
      if (base < hi4) {
        if (x[u].x > bv || bi == INT_MAX) { bv = x[u].x; bi = base; }
        if (x[u].y > bv) { bv = x[u].y; bi = base + 1; }
        if (x[u].z > bv) { bv = x[u].z; bi = base + 2; }
        if (x[u].w > bv) { bv = x[u].w; bi = base + 3; }
      }
    }
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
  for (int i = tid; i < n; i += kWalkThreads) {  // the walk's workgroup size
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
    // unused. Sixteen slices per round (one round up to V = 16 slices of
    // 16384 entries, all requested together with the parent and token
    // loads); clamped duplicates of the last slice never win a strict test.
    const ArgBest* pp = part + row * S;
    for (int s0 = 0; s0 < S; s0 += 16) {
      ArgBest o[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) o[u] = pp[min(s0 + u, S - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u)
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

// Sampling slices: kSliceSample entries, widened (in steps of kWalkThreads)
// when the vocabulary needs more than kMaxSplits of them. A slice is always a
// whole number of kWalkThreads-wide blocks, so each block of a row lies in
// one slice.
__host__ __device__ inline int sample_span(int V) {
  int span = (V + kMaxSplits - 1) / kMaxSplits;
  if (span < kSliceSample) span = kSliceSample;
  return (span + kWalkThreads - 1) / kWalkThreads * kWalkThreads;
}

__host__ __device__ inline int sample_splits(int V) {
  const int span = sample_span(V);
  return (V + span - 1) / span;
}

// Per (sequence, row, slice): the slice max m_s of the logits, the float64
// sum of e(x) = exp((l(x) - m_s) / tau) over the slice, and every e(x) itself
// (stored, so the walk reads a row instead of re-evaluating V exps). A slice
// of at most kSliceSample entries is read once into registers (entry
// lo + j * kThreads + t for thread t); wider slices (vocabularies past
// kMaxSplits * kSliceSample) take a two-pass loop. The exponent is formed as
// (l - m_s) * (1 / tau).
__global__ __launch_bounds__(kThreads) void softmax_slices_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ n_nodes, int T,
    int V, int S, double inv_tau, StatPart* __restrict__ part, double* __restrict__ ebuf) {
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  if (!live_row(n_nodes, T, b, j)) return;
  const int span = sample_span(V);
  const int lo = s * span, hi = min(V, lo + span);
  const float* row = logits + (static_cast<int64_t>(b) * T + j) * stride;
  double* erow = ebuf + (static_cast<int64_t>(b) * T + j) * V;
  const int tid = threadIdx.x;
  __shared__ float smax[kThreads / 64];
  __shared__ double ssum[kThreads / 64];
  constexpr int kPer = kSliceSample / kThreads;
  const bool in_regs = hi - lo <= kSliceSample;  // uniform
  float lv[kPer];
  float m = -INFINITY;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = lo + k * kThreads + tid;
      lv[k] = v < hi ? row[v] : -INFINITY;
      m = fmaxf(m, lv[k]);
    }
  } else {
    for (int v = lo + tid; v < hi; v += kThreads) m = fmaxf(m, row[v]);
  }
  m = tv::wave_max(m);
  if ((tid & 63) == 0) smax[tid >> 6] = m;
  __syncthreads();
  m = smax[0];
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, smax[w]);
  const double md = static_cast<double>(m);
  double z = 0.0;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = lo + k * kThreads + tid;
      if (v < hi) {
        const double e = exp((static_cast<double>(lv[k]) - md) * inv_tau);
        erow[v] = e;
        z += e;
      }
    }
  } else {
    for (int v = lo + tid; v < hi; v += kThreads) {
      const double e = exp((static_cast<double>(row[v]) - md) * inv_tau);
      erow[v] = e;
      z += e;
    }
  }
  z = tv::wave_sum_f64(z);
  if ((tid & 63) == 0) ssum[tid >> 6] = z;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += ssum[w];
    part[(static_cast<int64_t>(b) * T + j) * S + s] = StatPart{md, t};
  }
}

// Cross-lane moves of float64 values on the vector ALU, with the DPP lane
// patterns of tv_common.h.
using tv::kDppHalfMirror;
using tv::kDppRowRor8;
using tv::kDppRowShr;
using tv::kDppXor1;
using tv::kDppXor2;

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), kCtrl, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Row-pair exchange (rows of 16 lanes): lanes with bit 4 clear get
// a(lane) + a(lane ^ 16), lanes with bit 4 set get b(lane ^ 16) + b(lane).
__device__ __forceinline__ double swap16_sum(double a, double b) {
  const auto lo = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(__double2loint(a)),
                                                   static_cast<unsigned>(__double2loint(b)),
                                                   false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(__double2hiint(a)),
                                                   static_cast<unsigned>(__double2hiint(b)),
                                                   false, false);
  return __hiloint2double(static_cast<int>(hi[0]), static_cast<int>(lo[0])) +
         __hiloint2double(static_cast<int>(hi[1]), static_cast<int>(lo[1]));
}

// Half-wave exchange: lanes below 32 get a(lane) + a(lane + 32), lanes from
// 32 up get b(lane - 32) + b(lane).
__device__ __forceinline__ double swap32_sum(double a, double b) {
  const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(__double2loint(a)),
                                                   static_cast<unsigned>(__double2loint(b)),
                                                   false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(__double2hiint(a)),
                                                   static_cast<unsigned>(__double2hiint(b)),
                                                   false, false);
  return __hiloint2double(static_cast<int>(hi[0]), static_cast<int>(lo[0])) +
         __hiloint2double(static_cast<int>(hi[1]), static_cast<int>(lo[1]));
}

// Sum over the wave, in every lane (each step adds a lane and its partner,
// so all lanes round alike and hold the same value).
__device__ __forceinline__ double wave_sum_valu(double x) {
  x += dpp_f64<kDppXor1>(x);
  x += dpp_f64<kDppXor2>(x);
  x += dpp_f64<kDppHalfMirror>(x);
  x += dpp_f64<kDppRowRor8>(x);
  x = swap16_sum(x, x);
  return swap32_sum(x, x);
}

__device__ __forceinline__ float wave_max_valu(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  const unsigned u = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const unsigned v = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// Inclusive prefix sum over the lanes of a wave: within each row of 16 by
// shifted adds, then the totals of the earlier rows.
__device__ __forceinline__ double wave_scan_valu(double x, int lane) {
  x += dpp_f64<kDppRowShr(1)>(x);
  x += dpp_f64<kDppRowShr(2)>(x);
  x += dpp_f64<kDppRowShr(4)>(x);
  x += dpp_f64<kDppRowShr(8)>(x);
  const auto row_total = [&](int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                            __builtin_amdgcn_readlane(__double2loint(x), l));
  };
  const double r0 = row_total(15), r1 = row_total(31), r2 = row_total(47);
  if (lane >= 16) x += r0;
  if (lane >= 32) x += r1;
  if (lane >= 48) x += r2;
  return x;
}

// Workgroup barrier that waits for this wave's LDS operations only, so that
// global loads and HBM -> LDS copies stay in flight across it.
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block-wide float64 sum for kWalkThreads threads; every thread gets it.
// kLdsOnly: the barriers order LDS only (callers that exchange nothing
// through global memory, and keep copies in flight across the sum).
template <bool kLdsOnly = false>
__device__ double block_sum_f64(double x, double* s_red) {
  x = wave_sum_valu(x);
  const int tid = threadIdx.x;
  if (kLdsOnly) lds_only_barrier(); else __syncthreads();
  if ((tid & 63) == 0) s_red[tid >> 6] = x;
  if (kLdsOnly) lds_only_barrier(); else __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kWalkThreads / 64; ++w) t += s_red[w];
  return t;
}

// Shared state of the two walk kernels (one workgroup per sequence).
struct WalkShared {
  int flags;
  int accept;
  int cand;
  int hit;
  double base, thr;
  double m[TV_MAX_TREE], z[TV_MAX_TREE];  // row max and sum of exp over the row
  double scale[kMaxSplits];  // exp((m_s - M) / tau) / Z of the current row, per slice
  int par[TV_MAX_TREE], tok[TV_MAX_TREE], path[TV_MAX_TREE];
  double red[kWalkThreads / 64];
};

// Validates the sequence and merges the slice statistics of its rows into
// (M, Z). Returns the row status; on a dead sequence the outputs are written.
__device__ int walk_prologue(WalkShared& sh, const StatPart* part, int S,
                             const int32_t* tokens, const int32_t* parent, int n, int T,
                             int V, double tau, int b, int32_t* accept_len, int32_t* path,
                             int32_t* bonus, uint8_t* accept_mask, int8_t* decision,
                             int32_t* row_status) {
  const int tid = threadIdx.x;
  const int st = validate_seq(parent, tokens, n, T, V, b, &sh.flags);
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
    return st == TV_ROW_OK ? -1 : st;
  }
  if (tid < n) {
    const StatPart* pp = part + (rbase + tid) * S;
    double M = pp[0].m;
    for (int s = 1; s < S; ++s) M = fmax(M, pp[s].m);
    double Z = 0.0;
    for (int s = 0; s < S; ++s) Z += pp[s].z * exp((pp[s].m - M) / tau);
    sh.m[tid] = M;
    sh.z[tid] = Z;
    sh.par[tid] = tid == 0 ? -1 : parent[rbase + tid];
    sh.tok[tid] = tokens[rbase + tid];
  }
  if (tid < T) {
    sh.path[tid] = -1;
    decision[rbase + tid] = -1;
  }
  if (tid == 0) sh.path[0] = 0;
  return TV_ROW_OK;
}

// Per-slice factors turning the stored exp terms of `row` into p_row.
__device__ void walk_set_row(WalkShared& sh, const StatPart* part, int S, int64_t rbase,
                             int row, double tau) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < S) {
    const StatPart ps = part[(rbase + row) * S + tid];
    sh.scale[tid] = exp((ps.m - sh.m[row]) / tau) / sh.z[row];
  } else if (tid < kMaxSplits) {
    sh.scale[tid] = 0.0;  // slots past the vocabulary read zeros times this
  }
  __syncthreads();
}

// ratio = r(x) / q(x) with the conventions 0 / q = 0 and r / 0 = +inf.
__device__ __forceinline__ int accept_test(double rx, float qx, float ux) {
  double ratio;
  if (rx == 0.0)
    ratio = 0.0;
  else if (qx == 0.f)
    ratio = INFINITY;
  else
    ratio = rx / static_cast<double>(qx);
  return static_cast<double>(ux) < ratio ? 1 : 0;
}

__device__ void walk_finish(const WalkShared& sh, int plen, int bon, int T, int b,
                            int32_t* accept_len, int32_t* path, int32_t* bonus,
                            uint8_t* accept_mask, int32_t* row_status) {
  const int tid = threadIdx.x;
  const int64_t rbase = static_cast<int64_t>(b) * T;
  if (tid < T) {
    path[rbase + tid] = sh.path[tid];
    bool on = false;
    for (int k = 0; k <= plen; ++k) on |= (sh.path[k] == tid);
    accept_mask[rbase + tid] = on ? 1 : 0;
  }
  if (tid == 0) {
    accept_len[b] = plen;
    bonus[b] = bon;
    row_status[b] = TV_ROW_OK;
  }
}

// Wave-major slot layout of the node-parallel sampling path: wave w of a
// workgroup owns the vocabulary range [w * kWaveSpan, (w + 1) * kWaveSpan),
// and slot k of its lane l is entry w * kWaveSpan + 64 k + l (a wave's slot
// is 64 consecutive entries: coalesced loads and conflict-free LDS access).
constexpr int kWaveSpan = kRegSlots * 64;

__device__ __forceinline__ int slot_entry(int t, int k) {
  return (t >> 6) * kWaveSpan + k * 64 + (t & 63);
}

// dst[k] = row[slot_entry(threadIdx.x, k)] for a row of V entries, with
// entries at or past V read as zero by the buffer's range check (no memory
// access), so the loads of a row need no per-lane predicate and are all in
// flight together. Slots K0 .. K1 - 1 only. The thread offset passes through
// an empty asm so that it is formed per call, next to its loads.
template <int K0 = 0, int K1 = kRegSlots, typename E>
__device__ __forceinline__ void load_blocks(const E* row, int V, E (&dst)[kRegSlots]) {
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(row), 0,
                                                    V * static_cast<int>(sizeof(E)), 0x00020000);
  int off = slot_entry(threadIdx.x, 0) * static_cast<int>(sizeof(E));
  asm volatile("" : "+v"(off));
#pragma unroll
  for (int k = K0; k < K1; ++k) {
    // The slot's byte offset goes in the scalar offset.
    const int so = k * 64 * static_cast<int>(sizeof(E));
    if constexpr (sizeof(E) == 8)
      dst[k] = __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b64(rs, off, so, 0));
    else
      dst[k] = __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b32(rs, off, so, 0));
  }
}

// --------------------------------------- sampling, one workgroup per node ---
// For V <= kRegSlots * kWalkThreads the walk is taken apart by tree node.
// Its result is fixed by two facts per node j: which child of j the walk
// accepts if it reaches j, and which bonus token it draws if it stops at j.
// Both depend on node j's rows alone (p_j, then the draft rows of j's
// children in ascending order), so one workgroup per (sequence, node) finds
// them for every live node at once, from registers, and a small second
// kernel follows the accepted children from the root. Nodes off the final
// path are evaluated too: every live logits row and every tested draft row
// is read once; nothing is written per vocabulary entry.

// exp(y ln 2 / 1024) for the row terms, table-driven: with y = N + f (N
// the nearest integer, |f| <= 1/2), exp = 2^floor(N / 1024) *
// 2^((N mod 1024) / 1024) * exp(f ln 2 / 1024); the last factor minus one
// is its Taylor series in f to the cube (|f ln 2 / 1024| <= ln 2 / 2048,
// truncation below 6e-16 relative), coefficients (ln 2 / 1024)^k / k!. N is
// read from the low word of y + 1.5 * 2^52 (|y| < 2^31); the power of two is
// applied by ldexp, which rounds subnormal results and underflows to 0;
// results past the range are +inf. Relative error a few units of 2^-52 for
// normal results.
constexpr int kExpTab = 1024;
constexpr double kExpScale = 1477.3197218702985;   // 1024 / ln 2
constexpr double kExpC1 = 0.0006769015435155716;   // ln 2 / 1024
constexpr double kExpC2 = 2.2909784980688164e-07;  // (ln 2 / 1024)^2 / 2
constexpr double kExpC3 = 5.1692229383458926e-11;  // (ln 2 / 1024)^3 / 6
constexpr double kExpRound = 6755399441055744.0;   // 1.5 * 2^52
// Logits more than this many tau below the reference give a term below
// 2^-1075 (0 after rounding); they are clamped there.
constexpr double kExpFloorTau = 752.0;

// The table-free part: the table index N (low word) and the polynomial
// factor.
__device__ __forceinline__ double exp_reduce(double y, int& nn) {
  const double yr = y + kExpRound;
  nn = __double2loint(yr);
  const double f = y - (yr - kExpRound);
  return f * fma(f, fma(f, kExpC3, kExpC2), kExpC1);
}

// The rest: table entry sc = 2^((N mod 1024) / 1024), power
// 2^floor(N / 1024).
__device__ __forceinline__ double exp_finish(double sc, double pr, int nn) {
  return __builtin_amdgcn_ldexp(fma(sc, pr, sc), nn >> 10);
}

// The thread index and V through an empty asm: per-slot indices formed from
// these copies are recomputed where they are used instead of being shared
// across the kernel (32 of them would stay in registers throughout).
__device__ __forceinline__ int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

struct NodeShared {
  double exp_tab[kExpTab];  // 2^(i / 1024)
  float mx[kWalkThreads / 64];
  double red[kWalkThreads / 64];
  double wtot[kWalkThreads / 64];  // per-wave sums of r (bonus draw)
  double ssum[kRegSlots];          // per-slot sums of r in one wave (bonus draw)
  int accept;
  int cand;
  int dec[TV_MAX_TREE];  // decisions on this node's children (-1: not reached)
};

// Inverse-CDF draw from r, given as this thread's slots (entry
// slot_entry(threadIdx.x, k) in rv[k], zero past V): the smallest x with
// sum_{y<=x} r(y) > u0 * sum_y r(y). In the wave-major layout index order
// is wave, then slot, then lane: (1) every thread finds, from the sixteen
// wave totals, the first wave whose running total passes the threshold;
// (2) that wave alone folds its slots into per-slot sums and finds the
// first slot to pass it; (3) it scans that slot's 64 entries. Where
// rounding leaves a finer level short of the threshold that a coarser
// level passed, the draw is the last positive entry of the coarser block
// (the threshold sits at its end). Every thread returns the token.
__device__ int inverse_cdf_draw(const double (&rv)[kRegSlots], double u0, NodeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double ts = 0.0;
#pragma unroll
  for (int k = 0; k < kRegSlots; ++k) ts += rv[k];
  ts = wave_sum_valu(ts);
  if (lane == 0) sh.wtot[wave] = ts;
  if (tid == 0) sh.cand = -1;
  lds_only_barrier();
  // (1) The same sums in the same order in every thread.
  double total = 0.0;
  for (int w = 0; w < kWalkThreads / 64; ++w) total += sh.wtot[w];
  const double thr = u0 * total;
  int ws = -1;
  double base = 0.0;
  {
    double run = 0.0;
    for (int w = 0; w < kWalkThreads / 64; ++w) {
      const double nx = run + sh.wtot[w];
      if (ws < 0 && nx > thr) {
        ws = w;
        base = run;
      }
      run = nx;
    }
  }
  // Last positive entry of this thread's slots in [k0, k1) (-1 if none).
  auto last_positive = [&](int k0, int k1) {
    int last = -1;
    const int t = opaque_v(tid);
#pragma unroll
    for (int k = 0; k < kRegSlots; ++k)
      if (k >= k0 && k < k1 && rv[k] > 0.0) last = slot_entry(t, k);
    return last;
  };
  if (ws < 0) {
    // Rounding left the threshold at the total (u0 within an ulp of 1):
    // the last token with positive mass.
    const int last = last_positive(0, kRegSlots);
    if (last >= 0) atomicMax(&sh.cand, last);
  } else if (wave == ws) {
    // (2) Per-slot sums of this wave, eight slots at a time: after the
    // exchanges across lane bits 5, 4 and 3 each lane holds a partial sum
    // of slot c0 + (lane >> 3), which three more exchanges complete.
#pragma unroll
    for (int c0 = 0; c0 < kRegSlots; c0 += 8) {
      double a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = swap32_sum(rv[c0 + i], rv[c0 + i + 4]);
      a[0] = swap16_sum(a[0], a[2]);
      a[1] = swap16_sum(a[1], a[3]);
      const bool up = (lane & 8) != 0;
      double t = (up ? a[1] : a[0]) + dpp_f64<kDppRowRor8>(up ? a[0] : a[1]);
      t += dpp_f64<kDppHalfMirror>(t);
      t += dpp_f64<kDppXor2>(t);
      t += dpp_f64<kDppXor1>(t);
      if ((lane & 7) == 0) sh.ssum[c0 + (lane >> 3)] = t;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes
    const double sv = lane < kRegSlots ? sh.ssum[lane] : 0.0;
    const double inc = wave_scan_valu(sv, lane);
    const unsigned long long hit = __ballot(lane < kRegSlots && base + inc > thr);
    int pick = -1;
    if (hit) {
      const int ks = __ffsll(hit) - 1;
      // This wave's running total before slot ks.
      const double ex = __shfl(inc, ks > 0 ? ks - 1 : 0);
      const double sbase = ks > 0 ? base + ex : base;
      double val = 0.0;
#pragma unroll
      for (int k = 0; k < kRegSlots; ++k) val = k == ks ? rv[k] : val;
      // (3) The lanes of slot ks.
      const double run = sbase + wave_scan_valu(val, lane);
      const unsigned long long m = __ballot(run > thr);
      if (m) {
        pick = slot_entry(ws * 64, ks) + __ffsll(m) - 1;
      } else {
        const unsigned long long pos = __ballot(val > 0.0);
        if (pos) pick = slot_entry(ws * 64, ks) + 63 - __clzll(pos);
      }
      if (lane == 0) sh.cand = pick;
    } else {
      const int last = last_positive(0, kRegSlots);
      if (last >= 0) atomicMax(&sh.cand, last);
    }
  }
  __syncthreads();
  return sh.cand;
}

// HBM -> LDS copy of a row: entry v lands at s_row[v] (thread t reads its
// slot k at s_row[slot_entry(t, k)]). Without register staging. Entries at or past V are not read (the buffer's range
// check); the caller waits with vmcnt(0) and a barrier before reading.
// x4: 16-byte copies (the row 16-byte aligned, V a multiple of 4), eight
// per wave, each filling 256 consecutive entries; otherwise 4-byte copies,
// thirty-two per wave, each filling one of the wave's own slots.
__device__ __forceinline__ void row_to_lds(const float* row, int V, float* s_row, bool x4) {
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, V * 4, 0x00020000);
  // The wave index as a scalar (the LDS address of each copy is
  // wave-uniform); the copy's byte offset goes in the scalar offset, so
  // the lane offset is the only vector register the copies need.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (x4) {
    constexpr int kWaves = kWalkThreads / 64;
    constexpr int kCopies = kRegSlots * kWalkThreads / (256 * kWaves);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int first = (i * kWaves + wave) * 256;  // first entry of this copy
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(s_row + first), 16, lane * 16, first * 4,
          0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRegSlots; ++k) {
      const int first = wave * kWaveSpan + k * 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(s_row + first), 4, lane * 4, first * 4, 0,
          0);
    }
  }
}

// Waits until at most n vector-memory operations of this wave are in
// flight (expcnt and lgkmcnt not waited on).
#define TV_ACCEPT_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14))
#define TV_ACCEPT_WAIT_VMCNT0() TV_ACCEPT_WAIT_VMCNT(0)


// One workgroup per sequence (one thread per tree row): validates the
// sequence, follows node_next from the root and writes the outputs. A
// child's decision is reported when its parent lies on the path (those are
// the tests the walk makes); every other entry is -1. Sequences with n
// outside [1, T] read nothing of the node arrays.
__global__ __launch_bounds__(TV_MAX_TREE) void sample_path_kernel(
    const int32_t* __restrict__ node_dec, const int32_t* __restrict__ node_next,
    const int32_t* __restrict__ node_bonus, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int V,
    int32_t* accept_len, int32_t* path, int32_t* bonus, uint8_t* accept_mask,
    int8_t* decision, int32_t* row_status) {
  __shared__ int s_flags[1], s_len[1], s_end[1];
  __shared__ int s_next[TV_MAX_TREE], s_path[TV_MAX_TREE], s_on[TV_MAX_TREE];
  __shared__ int s_bon[TV_MAX_TREE];
  const int b = blockIdx.x;
  const int n = n_nodes[b];
  const int i = threadIdx.x;
  const int64_t row = static_cast<int64_t>(b) * T + i;
  const bool in_t = i < T;
  const bool n_ok = n >= 0 && n <= T;
  const bool live = n_ok && i < n;
  // One round trip: every row's entries are requested together with
  // n_nodes (rows of [0, T) are in bounds; those past n are read but
  // unused).
  const int pr = in_t && i > 0 ? parent[row] : -1;
  const int tk = in_t && i > 0 ? tokens[row] : 0;
  const int nx = in_t ? node_next[row] : -1;
  const int dc = in_t && i > 0 ? node_dec[row] : -1;
  const int bn = in_t ? node_bonus[row] : -1;
  if (i == 0) *s_flags = 0;
  __syncthreads();
  int f = 0;
  if (live && i > 0) {
    if (pr < 0 || pr >= i) f |= 1;
    if (tk < 0 || tk >= V) f |= 2;
  }
  if (f) atomicOr(s_flags, f);
  if (in_t) {
    s_next[i] = nx;
    s_path[i] = -1;
    s_on[i] = 0;
    s_bon[i] = bn;
  }
  __syncthreads();
  const int flags = *s_flags;
  const int st = !n_ok ? TV_ROW_NNODES
                       : ((flags & 1) ? TV_ROW_BAD_PARENT
                                      : ((flags & 2) ? TV_ROW_BAD_TOKEN : TV_ROW_OK));
  if (st != TV_ROW_OK || n == 0) {
    if (in_t) {
      path[row] = -1;
      accept_mask[row] = 0;
      decision[row] = -1;
    }
    if (i == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
      row_status[b] = st;
    }
    return;
  }
  if (i == 0) {
    int cur = 0, len = 0;
    s_path[0] = 0;
    s_on[0] = 1;
    // An accepted child lies after its parent, so the walk ends within n.
    for (int c = s_next[0]; c > cur && c < n; c = s_next[cur]) {
      s_path[++len] = c;
      s_on[c] = 1;
      cur = c;
    }
    *s_len = len;
    *s_end = cur;
  }
  __syncthreads();
  if (in_t) {
    path[row] = s_path[i];
    accept_mask[row] = static_cast<uint8_t>(s_on[i]);
    decision[row] = static_cast<int8_t>(live && i > 0 && s_on[pr] ? dc : -1);
  }
  if (i == 0) {
    accept_len[b] = *s_len;
    bonus[b] = s_bon[*s_end];
    row_status[b] = TV_ROW_OK;
  }
}

// One workgroup per live (sequence b, node j); thread t owns the entries
// x = slot_entry(t, k) (slot k) of every row it touches. p_j is formed in
// registers as e(x) = exp((l(x) - max l) / tau) with the factor 1 / sum e;
// the children of j are then tested in ascending index exactly as the walk
// tests them at j. The residual stays in registers as r = rv * inv (rv
// unnormalised): a test is one lookup by the owner of x, a rejection copies
// q_c's row into LDS, sums max(r - q_c, 0) in one pass and keeps it in a
// second once the sum is known to be positive (a zero sum keeps r
// unchanged). Outputs per node: node_next (the accepted child, -1 if none),
// node_dec for each child of j (+1, 0, or -1 when never reached) and, when
// no child is accepted, node_bonus (the draw from the final r with u[b][0]).
__global__ __launch_bounds__(kWalkThreads) void sample_node_kernel(
    const float* __restrict__ logits, int64_t stride, double inv_tau,
    const float* __restrict__ q, int64_t qstride, bool q_x4, const float* __restrict__ u,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ n_nodes, int T, int V, int32_t* __restrict__ node_dec,
    int32_t* __restrict__ node_next, int32_t* __restrict__ node_bonus) {
  __shared__ NodeShared sh;
  // The logits row, then the draft row of the child under test (slot
  // layout). Entries at or past V are zeroed once and never written by the
  // row copies.
  __shared__ float s_row[kRegSlots * kWalkThreads];
  const int j = blockIdx.x, b = blockIdx.y;
  if (!live_row(n_nodes, T, b, j)) return;
  const int n = n_nodes[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rbase = static_cast<int64_t>(b) * T;
  // Parents of rows lane and lane + 64 (-2 where there is no such child).
  static_assert(TV_MAX_TREE <= 128, "two parent words per lane");
  const int par_lo = lane >= 1 && lane < n ? parent[rbase + lane] : -2;
  const int par_hi = lane + 64 < n ? parent[rbase + lane + 64] : -2;
  // First child of j at index >= from (n when there is none).
  auto next_child = [&](int from) {
    const unsigned long long lo = __ballot(par_lo == j && lane >= from);
    if (lo) return __ffsll(lo) - 1;
    const unsigned long long hi = __ballot(par_hi == j && lane + 64 >= from);
    return hi ? 64 + __ffsll(hi) - 1 : n;
  };
  // The test of child c needs only q_c(x_c): its owner requests that one
  // value ahead; q_c's row is read only after c is rejected.
  auto token_of = [&](int cc) { return cc < n ? tokens[rbase + cc] : -1; };
  // Owner of entry xx: lane xx mod 64 of wave xx / kWaveSpan (slot
  // (xx mod kWaveSpan) / 64).
  auto owner_of = [&](int xx) {
    return xx >= 0 && xx < V ? (xx / kWaveSpan) * 64 + (xx & 63) : 0;
  };
  auto probe = [&](int cc, int xx) {
    return cc < n && xx >= 0 && xx < V && tid == owner_of(xx)
               ? q[(rbase + cc) * qstride + xx]
               : 0.f;
  };
  int c = next_child(1);
  int x = token_of(c);
  float qx = probe(c, x);
  const float u0 = u[rbase];  // the bonus draw's uniform, requested early
  if (tid < TV_MAX_TREE) sh.dec[tid] = -1;
  const float* lrow = logits + (rbase + j) * stride;
  sh.exp_tab[tid] = exp2(tid * (1.0 / kExpTab));
  static_assert(kExpTab == kWalkThreads, "one table entry per thread");
  {
    const int t = opaque_v(tid), vv = opaque_s(V);
    const int wb = (tid >> 6) * kWaveSpan;  // first entry of this wave
#pragma unroll
    for (int k = 0; k < kRegSlots; ++k)
      if (wb + k * 64 + 64 > vv && slot_entry(t, k) >= vv) s_row[slot_entry(t, k)] = 0.f;
  }
  // The terms are formed against a reference m0 known before the whole row
  // has arrived: the largest logit of slot 0. Every ratio the walk uses is
  // of two terms of one row (p_j = e / sum e), so the common factor
  // exp((max - m0) / tau) cancels. Logits are clamped to
  // [m0 - 752 tau, m0 + 1e5 tau] (both rounded down): below, the term is 0
  // in any case; above, the term overflows like every logit more than
  // ~710 tau above m0, the sum is not finite and the row goes round again
  // with its maximum as reference (also when m0 + 1e5 tau rounds to m0).
  const double ky = inv_tau * kExpScale;
  const double tau = 1.0 / inv_tau;
  double rv[kRegSlots];
  double z = 0.0;
  float m0 = -INFINITY;
#pragma nounroll
  for (int round = 0; round < 2; ++round) {
    // The whole row is requested at once; the reference and the first
    // half's terms wait only for the first half (loads into registers
    // complete in issue order), so the second half's transfer overlaps them.
    float lv[kRegSlots];
    load_blocks<0, kRegSlots>(lrow, V, lv);
    TV_ACCEPT_WAIT_VMCNT(kRegSlots / 2);
    float mr = slot_entry(tid, 0) < V ? lv[0] : -INFINITY;
    if (round == 1)  // the row maximum (a separate pass over the row)
      for (int v = tid; v < V; v += kWalkThreads) mr = fmaxf(mr, lrow[v]);
    // Barriers on LDS only: the second half is still in flight.
    mr = wave_max_valu(mr);
    if (lane == 0) sh.mx[wave] = mr;
    lds_only_barrier();
    m0 = sh.mx[0];
    for (int w = 1; w < kWalkThreads / 64; ++w) m0 = fmaxf(m0, sh.mx[w]);
    lds_only_barrier();  // sh.mx is written again below
    const float lo = __double2float_rd(static_cast<double>(m0) - kExpFloorTau * tau);
    const float hi = __double2float_rd(static_cast<double>(m0) + 1e5 * tau);
    // y = (l - m0) / tau * 1024 / ln 2 as one fused step.
    const double nky = -static_cast<double>(m0) * ky;
    const int t = opaque_v(tid), vv = opaque_s(V);
    const int wb = __builtin_amdgcn_readfirstlane((tid >> 6) * kWaveSpan);
    z = 0.0;
    // Logit of slot k, clamped; entries past V (only in the slots that
    // reach V, a wave-uniform test) read as the lower bound, whose term is
    // 0.
    auto logit = [&](int k) {
      float l = __builtin_amdgcn_fmed3f(lv[k], lo, hi);
      if (__builtin_expect(wb + k * 64 + 64 > vv, 0)) {
        if (slot_entry(t, k) >= vv) l = lo;
      }
      return static_cast<double>(l);
    };
    // Two-stage pipeline over the slots: the table read of slot k + 1 is
    // in flight while slot k is finished.
    int nn_n;
    double pr_n = exp_reduce(fma(logit(0), ky, nky), nn_n);
    double sc_n = sh.exp_tab[nn_n & (kExpTab - 1)];
#pragma unroll
    for (int k = 0; k < kRegSlots; ++k) {
      const int nn = nn_n;
      const double pr = pr_n, sc = sc_n;
      if (k + 1 < kRegSlots) {
        pr_n = exp_reduce(fma(logit(k + 1), ky, nky), nn_n);
        sc_n = sh.exp_tab[nn_n & (kExpTab - 1)];
      }
      const double e = exp_finish(sc, pr, nn);
      rv[k] = e;
      z += e;
      // Settle this slot's sum here: left to the compiler, the rest of each
      // term's evaluation sinks below the loop and every slot's
      // intermediates stay alive until then.
      asm volatile("" : "+v"(z));
    }
    const bool again = __syncthreads_or(!(z < INFINITY) || !(hi > m0));
    if (!again || round == 1) break;
  }
  // The first child's draft row goes to LDS while the sum and the first
  // test run (it is read only if that child is rejected). Issued after the
  // logits, so that the waits for the logits never wait for it.
  if (c < n) row_to_lds(q + (rbase + c) * qstride, V, s_row, q_x4);
  double inv = 1.0 / block_sum_f64<true>(z, sh.red);

  int accepted = -1;
  bool first = true;  // c is the first child: its row is in LDS already
  while (c < n) {
    const bool x_ok = x >= 0 && x < V;
    if (tid == owner_of(x)) {
      int acc = 0;
      if (x_ok) {
        const int ks = (x % kWaveSpan) / 64;
        double rx = 0.0;
#pragma unroll
        for (int k = 0; k < kRegSlots; ++k) rx = k == ks ? rv[k] : rx;
        acc = accept_test(rx * inv, qx, u[rbase + c]);
      }
      sh.dec[c] = acc;
      sh.accept = acc;
    }
    // This barrier also ends every read of s_row before the copy below
    // overwrites it (LDS only: a copy in flight stays in flight).
    lds_only_barrier();
    // Every thread reads sh.accept before the barrier inside block_sum_f64,
    // which the next test's write comes after.
    if (sh.accept) {
      accepted = c;
      break;
    }
    if (!first) row_to_lds(q + (rbase + c) * qstride, V, s_row, q_x4);
    first = false;
    const int cn = next_child(c + 1);
    x = token_of(cn);
    qx = probe(cn, x);
    TV_ACCEPT_WAIT_VMCNT0();
    __syncthreads();
    double part_sum = 0.0;
#pragma unroll
    for (int k = 0; k < kRegSlots; ++k)
      part_sum += fmax(fma(rv[k], inv, -static_cast<double>(s_row[slot_entry(tid, k)])), 0.0);
    const double tot = block_sum_f64<true>(part_sum, sh.red);
    if (tot > 0.0) {
#pragma unroll
      for (int k = 0; k < kRegSlots; ++k)
        rv[k] = fmax(fma(rv[k], inv, -static_cast<double>(s_row[slot_entry(tid, k)])), 0.0);
      inv = 1.0 / tot;
    }
    c = cn;
  }
  int bon = -1;
  if (accepted >= 0) {
    // The first child's row copy may still be in flight: it must land
    // before the LDS is reused.
    TV_ACCEPT_WAIT_VMCNT0();
  } else {
    bon = inverse_cdf_draw(rv, static_cast<double>(u0), sh);
  }
  __syncthreads();  // sh.dec complete
  // Wave 0 stores this node's results: the decisions on the node's children
  // (found from the parent words it holds), the accepted child and the
  // bonus.
  if (wave == 0) {
    if (par_lo == j) node_dec[rbase + lane] = sh.dec[lane];
    if (par_hi == j) node_dec[rbase + lane + 64] = sh.dec[lane + 64];
    if (lane == 0) {
      node_next[rbase + j] = accepted;
      if (accepted < 0) node_bonus[rbase + j] = bon;
    }
  }
}


// Walk for larger vocabularies: the residual r lives in one of two float64
// buffers of V entries per sequence, or stays implicit as p_cur (the stored
// exp terms times the per-slice factors) until the first rejection.
__global__ __launch_bounds__(kWalkThreads) void sample_walk_kernel(
    const StatPart* __restrict__ part, int S, const float* __restrict__ q, int64_t qstride,
    const float* __restrict__ u, double tau, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int T, int V,
    const double* __restrict__ ebuf, double* __restrict__ resid, int32_t* accept_len,
    int32_t* path, int32_t* bonus, uint8_t* accept_mask, int8_t* decision,
    int32_t* row_status) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = n_nodes[b];
  if (walk_prologue(sh, part, S, tokens, parent, n, T, V, tau, b, accept_len, path, bonus,
                    accept_mask, decision, row_status) != TV_ROW_OK)
    return;
  const int64_t rbase = static_cast<int64_t>(b) * T;
  double* buf[2] = {resid + static_cast<int64_t>(b) * 2 * V,
                    resid + static_cast<int64_t>(b) * 2 * V + V};
  int cur = 0, len = 0, held = -1;  // held: index of the buffer holding r, -1 = implicit
  const int span = sample_span(V);
  walk_set_row(sh, part, S, rbase, 0, tau);
  const double* erow = ebuf + rbase * V;  // + cur * V
  auto r_at = [&](int x) -> double {
    if (held < 0) return erow[static_cast<int64_t>(cur) * V + x] * sh.scale[x / span];
    return buf[held][x];
  };

  for (;;) {
    bool accepted = false;
    for (int c = cur + 1; c < n; ++c) {
      if (sh.par[c] != cur) continue;
      const int x = sh.tok[c];
      if (tid == 0) {
        const int acc = accept_test(r_at(x), q[(rbase + c) * qstride + x], u[rbase + c]);
        decision[rbase + c] = static_cast<int8_t>(acc);
        sh.accept = acc;
      }
      __syncthreads();
      if (sh.accept) {
        ++len;
        if (tid == 0) sh.path[len] = c;
        cur = c;
        held = -1;
        walk_set_row(sh, part, S, rbase, c, tau);
        accepted = true;
        break;
      }
      // Rejected: r <- max(r - q_c, 0) / sum, into the free buffer. Each
      // thread loads kBatch entries before storing any, so the loads are in
      // flight together.
      const int dst = held == 0 ? 1 : 0;
      const float* qrow = q + (rbase + c) * qstride;
      double part_sum = 0.0;
      for (int v0 = tid; v0 < V; v0 += kWalkThreads * kBatch) {
        double rv[kBatch], qv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int v = min(v0 + k * kWalkThreads, V - 1);
          rv[k] = r_at(v);
          qv[k] = static_cast<double>(qrow[v]);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int v = v0 + k * kWalkThreads;
          if (v < V) {
            const double res = fmax(rv[k] - qv[k], 0.0);
            buf[dst][v] = res;
            part_sum += res;
          }
        }
      }
      const double tot = block_sum_f64(part_sum, sh.red);
      if (tot > 0.0) {
        for (int v0 = tid; v0 < V; v0 += kWalkThreads * kBatch) {
          double rv[kBatch];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) rv[k] = buf[dst][min(v0 + k * kWalkThreads, V - 1)];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const int v = v0 + k * kWalkThreads;
            if (v < V) buf[dst][v] = rv[k] / tot;
          }
        }
        __syncthreads();
        held = dst;
      }
    }
    if (!accepted) break;
  }
  __syncthreads();

  // Bonus: smallest x with sum_{y<=x} r(y) > u0 * sum_y r(y). Each thread
  // owns a contiguous range of the vocabulary.
  const int per = (V + kWalkThreads - 1) / kWalkThreads;
  const int lo = min(V, tid * per);
  const int hi = min(V, lo + per);
  if (held < 0) {
    // Materialise p_cur once (each thread writes and later reads only its
    // own range).
    for (int v0 = lo; v0 < hi; v0 += kBatch) {
      double rv[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) rv[k] = r_at(min(v0 + k, V - 1));
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (v0 + k < hi) buf[0][v0 + k] = rv[k];
    }
    held = 0;
  }
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
  if (lane == 63) sh.red[tid >> 6] = incl;
  __syncthreads();
  double wave_off = 0.0, total = 0.0;
  for (int w = 0; w < kWalkThreads / 64; ++w) {
    if (w < (tid >> 6)) wave_off += sh.red[w];
    total += sh.red[w];
  }
  const double thr = static_cast<double>(u[rbase]) * total;
  double run = wave_off + excl;
  int cand = INT_MAX;
  for (int v0 = lo; v0 < hi && cand == INT_MAX; v0 += kBatch) {
    double rv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) rv[k] = r_at(min(v0 + k, V - 1));
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (cand == INT_MAX && v0 + k < hi) {
        run += rv[k];
        if (run > thr) cand = v0 + k;
      }
    }
  }
  if (tid == 0) sh.cand = INT_MAX;
  __syncthreads();
  if (cand != INT_MAX) atomicMin(&sh.cand, cand);
  __syncthreads();
  int bon = sh.cand;
  if (bon == INT_MAX) {
    // Rounding left the threshold above every running sum (u0 within an ulp
    // of 1): take the last token with positive mass.
    int lastpos = -1;
    for (int v = lo; v < hi; ++v)
      if (r_at(v) > 0.0) lastpos = v;
    __syncthreads();
    if (tid == 0) sh.cand = -1;
    __syncthreads();
    if (lastpos >= 0) atomicMax(&sh.cand, lastpos);
    __syncthreads();
    bon = sh.cand;
  }
  walk_finish(sh, len, bon, T, b, accept_len, path, bonus, accept_mask, row_status);
}

bool accept_sizes_ok(int B, int T, int V) {
  return B >= 0 && T >= 1 && T <= TV_MAX_TREE && V >= 1;
}

size_t greedy_ws(int B, int T, int V) {
  return tvh::align_up(static_cast<size_t>(B) * T * num_splits(V) * sizeof(ArgBest), 256);
}

// Vocabularies the one-round-trip walk covers.
bool sample_one_pass(int V) { return V <= kRegSlots * kWalkThreads; }

// Sampling workspace. Vocabularies of the node-parallel path: per node the
// accepted child, the bonus draw and the decision (int32 each). Larger
// ones: slice statistics, the stored exp terms of every row (float64, B T V)
// and two float64 residual buffers per sequence.
size_t node_ws(int B, int T) {
  return 3 * tvh::align_up(static_cast<size_t>(B) * T * sizeof(int32_t), 256);
}

size_t sample_ws(int B, int T, int V) {
  if (sample_one_pass(V)) return node_ws(B, T);
  return tvh::align_up(static_cast<size_t>(B) * T * sample_splits(V) * sizeof(StatPart), 256) +
         tvh::align_up(static_cast<size_t>(B) * T * V * sizeof(double), 256) +
         tvh::align_up(static_cast<size_t>(B) * 2 * V * sizeof(double), 256);
}

}  // namespace

extern "C" size_t tv_accept_workspace_size(int B, int T, int V, int mode) {
  if (!accept_sizes_ok(B, T, V) || (mode != 0 && mode != 1)) return static_cast<size_t>(-1);
  return mode == 0 ? greedy_ws(B, T, V) : sample_ws(B, T, V);
}

namespace {

// ---------------------------------------------- greedy without allocation ---
// tv_accept_greedy_noalloc keeps the per-slice argmax partials in this
// file-scope array instead of a caller workspace: one copy per device, held
// until the process ends. Every call on a device shares it (calls that
// overlap on one device race). The argmax kernel writes every partial the
// walk reads, so nothing in it needs clearing between calls.
constexpr size_t kStaticScratchBytes = size_t(2) << 20;  // 2 MiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of this device's `scratch`, looked up once per device (the
// array's name is only a host-side handle: kernels must get the address).
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();  // do not leave the failure for the next call to report
      return TV_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TV_OK;
}

int greedy_launch(const float* logits, int64_t logits_row_stride, const int32_t* tokens,
                  const int32_t* parent, const int32_t* n_nodes, int B, int T, int V,
                  int32_t* accept_len, int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                  ArgBest* part, int32_t* row_status, hipStream_t stream) {
  const int S = num_splits(V);
  hipLaunchKernelGGL(argmax_slices_kernel, dim3(S, T, B), dim3(kThreads), 0, stream, logits,
                     logits_row_stride, n_nodes, T, V, S, part);
  hipLaunchKernelGGL(greedy_walk_kernel, dim3(B), dim3(TV_MAX_TREE), 0, stream, part, S, tokens,
                     parent, n_nodes, T, V, accept_len, path, bonus, accept_mask, row_status);
  return tvh::launch_status();
}

int greedy_args(const float* logits, int64_t logits_row_stride, const int32_t* tokens,
                const int32_t* parent, const int32_t* n_nodes, int B, int T, int V,
                int32_t* accept_len, int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                int32_t* row_status) {
  if (!logits || !tokens || !parent || !n_nodes || !accept_len || !path || !bonus ||
      !accept_mask || !row_status)
    return TV_ERR_NULL;
  // B is a grid dimension of the argmax launch (at most 65535).
  if (!accept_sizes_ok(B, T, V) || B > 65535 || logits_row_stride < V) return TV_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(logits) & 3u) return TV_ERR_ALIGN;
  return TV_OK;
}

}  // namespace

extern "C" int tv_accept_greedy_noalloc(const float* logits, int64_t logits_row_stride,
                                        const int32_t* tokens, const int32_t* parent,
                                        const int32_t* n_nodes, int B, int T, int V,
                                        int32_t* accept_len, int32_t* path, int32_t* bonus,
                                        uint8_t* accept_mask, int32_t* row_status,
                                        hipStream_t stream) {
  const int st = greedy_args(logits, logits_row_stride, tokens, parent, n_nodes, B, T, V,
                             accept_len, path, bonus, accept_mask, row_status);
  if (st != TV_OK) return st;
  if (B == 0) return TV_OK;
  if (greedy_ws(B, T, V) > kStaticScratchBytes) return TV_ERR_WORKSPACE;
  void* ptr = nullptr;
  const int sp = scratch_ptr(&ptr);
  if (sp != TV_OK) return sp;
  return greedy_launch(logits, logits_row_stride, tokens, parent, n_nodes, B, T, V, accept_len,
                       path, bonus, accept_mask, static_cast<ArgBest*>(ptr), row_status, stream);
}

extern "C" int tv_accept_greedy(const float* logits, int64_t logits_row_stride,
                                const int32_t* tokens, const int32_t* parent,
                                const int32_t* n_nodes, int B, int T, int V, int32_t* accept_len,
                                int32_t* path, int32_t* bonus, uint8_t* accept_mask,
                                void* workspace, size_t ws_bytes, int32_t* row_status,
                                hipStream_t stream) {
  const int st = greedy_args(logits, logits_row_stride, tokens, parent, n_nodes, B, T, V,
                             accept_len, path, bonus, accept_mask, row_status);
  if (st != TV_OK) return st;
  if (B == 0) return TV_OK;
  if (!workspace || ws_bytes < greedy_ws(B, T, V) || !tvh::aligned256(workspace))
    return TV_ERR_WORKSPACE;
  return greedy_launch(logits, logits_row_stride, tokens, parent, n_nodes, B, T, V, accept_len,
                       path, bonus, accept_mask, static_cast<ArgBest*>(workspace), row_status,
                       stream);
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
  // B is a grid dimension of every launch (at most 65535).
  if (!accept_sizes_ok(B, T, V) || B > 65535 || logits_row_stride < V || q_row_stride < V)
    return TV_ERR_SHAPE;
  if (!(temperature > 0.f)) return TV_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(q) & 3u))
    return TV_ERR_ALIGN;
  if (B == 0) return TV_OK;
  if (!workspace || ws_bytes < sample_ws(B, T, V) || !tvh::aligned256(workspace))
    return TV_ERR_WORKSPACE;
  const double tau = static_cast<double>(temperature);
  char* ws = static_cast<char*>(workspace);
  if (sample_one_pass(V)) {
    const size_t words = tvh::align_up(static_cast<size_t>(B) * T * sizeof(int32_t), 256);
    int32_t* node_next = reinterpret_cast<int32_t*>(ws);
    int32_t* node_bonus = reinterpret_cast<int32_t*>(ws + words);
    int32_t* node_dec = reinterpret_cast<int32_t*>(ws + 2 * words);
    // Draft rows copied 16 bytes at a time when every row is 16-byte aligned.
    const bool q_x4 = (V & 3) == 0 && (q_row_stride & 3) == 0 && tvh::aligned16(q);
    hipLaunchKernelGGL(sample_node_kernel, dim3(T, B), dim3(kWalkThreads), 0, stream, logits,
                       logits_row_stride, 1.0 / tau, q, q_row_stride, q_x4, u, tokens, parent,
                       n_nodes, T, V, node_dec, node_next, node_bonus);
    hipLaunchKernelGGL(sample_path_kernel, dim3(B), dim3(TV_MAX_TREE), 0, stream, node_dec,
                       node_next, node_bonus, tokens, parent, n_nodes, T, V, accept_len, path,
                       bonus, accept_mask, decision, row_status);
    return tvh::launch_status();
  }
  const int S = sample_splits(V);
  StatPart* part = static_cast<StatPart*>(workspace);
  char* base = ws + tvh::align_up(static_cast<size_t>(B) * T * S * sizeof(StatPart), 256);
  double* ebuf = reinterpret_cast<double*>(base);
  hipLaunchKernelGGL(softmax_slices_kernel, dim3(S, T, B), dim3(kThreads), 0, stream, logits,
                     logits_row_stride, n_nodes, T, V, S, 1.0 / tau, part, ebuf);
  double* resid = reinterpret_cast<double*>(
      base + tvh::align_up(static_cast<size_t>(B) * T * V * sizeof(double), 256));
  hipLaunchKernelGGL(sample_walk_kernel, dim3(B), dim3(kWalkThreads), 0, stream, part, S, q,
                     q_row_stride, u, tau, tokens, parent, n_nodes, T, V, ebuf, resid,
                     accept_len, path, bonus, accept_mask, decision, row_status);
  return tvh::launch_status();
}
