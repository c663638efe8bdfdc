// Tree-masked, split-KV, grouped-query attention for draft-tree verification.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput".
//   - commit "feat(activevln): grammar-trie tree speculation with exact
//     acceptance": every draft node is verified in one tree-attention
//     forward; a node sees the committed context and its own ancestors;
//   - commit "perf(activevln): lossless batched replay throughput options":
//     attention_kernel="gqa" splits the keys into partitions and packs the
//     query heads sharing a KV head into one program; probability_parts
//     keeps the probabilities fp32-faithful in the P.V product;
//     skip_padded_queries: programs with only padding rows do no KV work;
//   - commit "fix(attention): never read KV slots past a row's live
//     queries": slots at or past ctx_len + n_nodes are never loaded.
//
// MI355X design (gfx950, wave64, 160 KB LDS, bf16 MFMA):
//   * One workgroup (4 waves) per (key chunk, row group, sequence, KV head).
//     The G query heads of a KV head times the T tree rows form R = G*T
//     packed rows (row r = node * G + head-in-group); a workgroup holds up
//     to 256 of them, 64 per wave, so every key and value read from HBM is
//     used by all G heads and all T nodes at once: the contraction over D
//     and over keys is dense, so it runs on MFMA (v_mfma_f32_16x16x32_bf16).
//   * Keys are cut into fixed chunks of C keys (split-KV). The last chunk of
//     a sequence also covers the tree block [L, L + n), so tree masking
//     only happens there; partial (m, l, O) go to a workspace and a second
//     kernel merges them with a log-sum-exp combine. A sequence with one
//     chunk is written directly.
//   * K and V tiles of 64 keys are double-buffered through LDS: registers
//     hold the next tile's loads while the waves compute on the current one.
//     K is stored row-major with an XOR swizzle of its 16-byte chunks; V is
//     stored transposed (V^T, padded rows) so that the P.V operand reads
//     eight consecutive keys per lane with one 16-byte LDS load.
//   * S^T = K Q^T is computed so that a lane's accumulators always belong to
//     one packed row: the per-row softmax max needs only two cross-lane
//     steps, and P^T lands directly in the MFMA B-operand layout.
//   * Online softmax in the log2 domain with a lazy rescale: the running
//     max only moves when a row's block max exceeds it by more than 8, so
//     P stays below 2^8 and the O rescale is rare.
#include "tv_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKB = 64;            // keys per LDS stage
constexpr int kThreads = 256;      // 4 waves
constexpr int kRowsWave = 64;      // packed rows per wave (4 tiles of 16)
constexpr int kRT = 4;             // row tiles per wave
constexpr int kRowsWG = kRowsWave * (kThreads / tv::kWave);
constexpr int kVtStride = kKB + 8; // bf16 per V^T row: 144 bytes
constexpr int kRowsWGf32 = 64;     // packed rows per fp32 workgroup (4 lanes each)
constexpr int kKBf32 = 32;         // keys per fp32 LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;   // lazy-rescale threshold (log2 units)

struct AttnParams {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_sh, kv_ss;
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const uint32_t* mask;
  int B, T, Hq, Hkv, G, R, W, max_ctx, kv_capacity, chunk, nchunk, parts;
  float scale_log2;
  float* out;
  float* lse;
  float* part_o;    // [B*Hkv][nchunk][R][D], un-normalised
  float2* part_ml;  // [B*Hkv][nchunk][R]: (running max in log2 units, sum)
  int32_t* row_status;
};

// Status of sequence b: TV_ROW_OK (live), -1 (padded: n == 0) or an error.
__device__ __forceinline__ int seq_check(const AttnParams& p, int b, int& n, int& L) {
  n = p.n_nodes[b];
  L = p.ctx_len[b];
  if (n < 0 || n > p.T) return TV_ROW_NNODES;
  if (n == 0) return -1;
  if (L < 0 || L > p.max_ctx || static_cast<int64_t>(L) + n > p.kv_capacity)
    return TV_ROW_CTX_BOUND;
  return TV_ROW_OK;
}

__device__ __forceinline__ int num_chunks(int L, int chunk) {
  return L == 0 ? 1 : (L + chunk - 1) / chunk;
}

// Output rows of (b, kvh) in [r_lo, r_hi) set to the padding values.
template <int D>
__device__ void zero_rows(const AttnParams& p, int b, int kvh, int r_lo, int r_hi, int tid,
                          int nthreads) {
  constexpr int D4 = D / 4;
  const int rows = r_hi - r_lo;
  for (int idx = tid; idx < rows * D4; idx += nthreads) {
    const int r = r_lo + idx / D4;
    const int d4 = idx % D4;
    const int i = r / p.G;
    const int h = kvh * p.G + (r - i * p.G);
    const int64_t orow = (static_cast<int64_t>(b) * p.T + i) * p.Hq + h;
    reinterpret_cast<float4*>(p.out + orow * D)[d4] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d4 == 0) p.lse[orow] = -INFINITY;
  }
}

// Handles sequences that are padded or invalid; returns true if the caller
// must stop. Also publishes the per-sequence status exactly once.
template <int D>
__device__ bool handle_non_live(const AttnParams& p, int st, int b, int kvh, int c, int rg,
                                int rows_wg, int tid, int nthreads) {
  if (c == 0 && rg == 0 && kvh == 0 && tid == 0)
    p.row_status[b] = (st == -1) ? TV_ROW_OK : st;
  if (st == TV_ROW_OK) return false;
  if (c == 0) {
    const int r_lo = rg * rows_wg;
    const int r_hi = min(p.R, r_lo + rows_wg);
    zero_rows<D>(p, b, kvh, r_lo, r_hi, tid, nthreads);
  }
  return true;
}

__device__ __forceinline__ bool tree_visible(const uint32_t* s_mask, int W, int node, int j) {
  return (s_mask[node * W + (j >> 5)] >> (j & 31)) & 1u;
}

// ------------------------------------------------------------ bf16 MFMA ---

template <int D>
__device__ __forceinline__ int k_swz(int key) {
  constexpr int DCH = D / 8;
  return ((key & 3) | (((key >> 3) & 3) << 2)) & (DCH - 1);
}

template <int D, int PARTS>
__global__ __launch_bounds__(kThreads) void attn_split_bf16_kernel(AttnParams p) {
  constexpr int DCH = D / 8;               // 16-byte chunks per key row
  constexpr int KS = D / 32;               // MFMA k-steps along D
  constexpr int DT = D / 16;               // 16-wide d tiles of O
  constexpr int KLOADS = kKB * DCH / kThreads;   // K chunks per thread per tile
  constexpr int VITEMS = (kKB / 4) * DCH;        // V (4 keys x 8 d) items per tile

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][D * kVtStride];
  __shared__ uint32_t sMask[TV_MAX_TREE * (TV_MAX_TREE / 32)];

  const int c = blockIdx.x;
  const int rg = blockIdx.y;
  const int bk = blockIdx.z;
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int n, L;
  const int st = seq_check(p, b, n, L);
  if (handle_non_live<D>(p, st, b, kvh, c, rg, kRowsWG, tid, kThreads)) return;
  const int nch = num_chunks(L, p.chunk);
  if (c >= nch) return;
  const bool last = (c == nch - 1);
  const int kbeg = c * p.chunk;
  const int kend = last ? L + n : min(kbeg + p.chunk, L);

  if (last) {
    const uint32_t* mrow = p.mask + static_cast<int64_t>(b) * p.T * p.W;
    for (int idx = tid; idx < n * p.W; idx += kThreads) sMask[idx] = mrow[idx];
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + b * p.kv_sb + kvh * p.kv_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + b * p.kv_sb + kvh * p.kv_sh;

  // ---- Q fragments (MFMA B operand of S^T = K Q^T) ----
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int row0 = rg * kRowsWG + wave * kRowsWave;
  const int rows_here = min(p.R - row0, kRowsWave);
  const int ntile = rows_here <= 0 ? 0 : (rows_here + 15) / 16;
  bf16x8_t qf[kRT][KS];
  int node_rt[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = row0 + rt * 16 + l16;
    int node = -1;
    if (r < p.R) {
      const int i = r / p.G;
      if (i < n) node = i;
    }
    node_rt[rt] = node;
    if (node >= 0) {
      const int h = kvh * p.G + (r - node * p.G);
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + b * p.q_sb + node * p.q_st +
                             h * p.q_sh;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[rt][s] = __builtin_bit_cast(bf16x8_t,
                                       *reinterpret_cast<const u16x8_t*>(qrow + 32 * s + 8 * g));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[rt][s] = __builtin_bit_cast(bf16x8_t, u16x8_t(0));
    }
  }

  f32x4_t o[DT][kRT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) o[dt][rt] = f32x4_t(0.f);
  float m_run[kRT], l_run[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }

  // ---- tile loads: global -> registers -> LDS ----
  u16x8_t kreg[KLOADS];
  u16x8_t vreg[4];
  const int vkq = tid & 15;       // V item: keys 4*vkq .. 4*vkq+3
  const int vdq = tid >> 4;       //         d   8*vdq .. 8*vdq+7
  const bool v_item = tid < VITEMS;

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int it = 0; it < KLOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / DCH;
      const int ch = idx - key * DCH;
      const int s = key0 + key;
      kreg[it] = (s < kend)
                     ? *reinterpret_cast<const u16x8_t*>(kbase + s * p.kv_ss + ch * 8)
                     : u16x8_t(0);
    }
    if (v_item) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = key0 + 4 * vkq + j;
        vreg[j] = (s < kend)
                      ? *reinterpret_cast<const u16x8_t*>(vbase + s * p.kv_ss + vdq * 8)
                      : u16x8_t(0);
      }
    }
  };
  auto store_tile = [&](int stg) {
#pragma unroll
    for (int it = 0; it < KLOADS; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx / DCH;
      const int ch = idx - key * DCH;
      *reinterpret_cast<u16x8_t*>(&sK[stg][key * D + ((ch ^ k_swz<D>(key)) * 8)]) = kreg[it];
    }
    if (v_item) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = static_cast<uint32_t>(vreg[0][e]) |
                            (static_cast<uint32_t>(vreg[1][e]) << 16);
        const uint32_t hi = static_cast<uint32_t>(vreg[2][e]) |
                            (static_cast<uint32_t>(vreg[3][e]) << 16);
        *reinterpret_cast<uint2*>(&sVt[stg][(8 * vdq + e) * kVtStride + 4 * vkq]) =
            make_uint2(lo, hi);
      }
    }
  };

  const int nblk = (kend - kbeg + kKB - 1) / kKB;
  const int vis_all_end = min(L, kend);  // keys below this are visible to every row

  load_tile(kbeg);
  store_tile(0);
  __syncthreads();

  for (int blk = 0; blk < nblk; ++blk) {
    const int stg = blk & 1;
    const int key0 = kbeg + blk * kKB;
    if (blk + 1 < nblk) load_tile(key0 + kKB);

    if (ntile > 0) {
#pragma unroll
      for (int sb = 0; sb < kKB / 32; ++sb) {
        const int skey0 = key0 + 32 * sb;
        if (skey0 >= kend) break;
        // S^T for 32 keys: two 16-key tiles; tile t row m holds key
        // 8*(m/4) + 4*t + m%4 so that lane group g ends up with keys 8g..8g+7.
        f32x4_t sacc[2][kRT];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) sacc[t][rt] = f32x4_t(0.f);
          const int krow = 32 * sb + 8 * (l16 >> 2) + 4 * t + (l16 & 3);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const int ch = 4 * s + g;
            const bf16x8_t a = __builtin_bit_cast(
                bf16x8_t,
                *reinterpret_cast<const u16x8_t*>(&sK[stg][krow * D + ((ch ^ k_swz<D>(krow)) * 8)]));
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt)
              if (rt < ntile)
                sacc[t][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][s], sacc[t][rt], 0,
                                                                      0, 0);
          }
        }
        // ---- scale, mask, online softmax ----
        const bool full = (skey0 + 32 <= vis_all_end);
        float x[kRT][8];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = sacc[t][rt][e] * p.scale_log2;
              if (!full) {
                const int key = skey0 + 8 * g + 4 * t + e;
                bool vis = key < vis_all_end;
                if (!vis && key >= L && key < kend) {
                  const int node = node_rt[rt];
                  vis = node >= 0 && tree_visible(sMask, p.W, node, key - L);
                }
                if (!vis) v = -INFINITY;
              }
              x[rt][4 * t + e] = v;
            }
        }
        float mx[kRT];
        bool need_any = false;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          float m = x[rt][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) m = fmaxf(m, x[rt][e]);
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          mx[rt] = m;
          need_any |= (m > m_run[rt] + kRescale);
        }
        if (__any(need_any)) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            const bool need = mx[rt] > m_run[rt] + kRescale;
            const float m_new = need ? mx[rt] : m_run[rt];
            const float alpha = need ? exp2f(m_run[rt] - m_new) : 1.f;
            l_run[rt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
            m_run[rt] = m_new;
          }
        }
        bf16x8_t pb[kRT], pb2[kRT], pb3[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const float mu = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];
          u16x8_t h1, h2, h3;
          float lsum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pr = exp2f(x[rt][e] - mu);
            lsum += pr;
            const uint16_t b1 = tv::f32_to_bf16_rne(pr);
            h1[e] = b1;
            if (PARTS > 1) {
              const float r1 = pr - tv::bf16_to_f32(b1);
              const uint16_t b2 = tv::f32_to_bf16_rne(r1);
              h2[e] = b2;
              h3[e] = tv::f32_to_bf16_rne(r1 - tv::bf16_to_f32(b2));
            }
          }
          l_run[rt] += lsum;
          pb[rt] = __builtin_bit_cast(bf16x8_t, h1);
          if (PARTS > 1) {
            pb2[rt] = __builtin_bit_cast(bf16x8_t, h2);
            pb3[rt] = __builtin_bit_cast(bf16x8_t, h3);
          }
        }
        // ---- O^T += V^T P^T over these 32 keys ----
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u16x8_t*>(
                            &sVt[stg][(16 * dt + l16) * kVtStride + 32 * sb + 8 * g]));
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            if (rt < ntile) {
              o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], o[dt][rt], 0, 0, 0);
              if (PARTS > 1)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb2[rt], o[dt][rt], 0, 0, 0);
              if (PARTS > 2)
                o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb3[rt], o[dt][rt], 0, 0, 0);
            }
          }
        }
      }
    }

    if (blk + 1 < nblk) store_tile(stg ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  float l_tot[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_tot[rt] = l;
  }
  const bool direct = (nch == 1);
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if (rt >= ntile) continue;
    const int r = row0 + rt * 16 + l16;
    if (r >= p.R) continue;
    if (direct) {
      const int i = r / p.G;
      const int h = kvh * p.G + (r - i * p.G);
      const int64_t orow = (static_cast<int64_t>(b) * p.T + i) * p.Hq + h;
      float* dst = p.out + orow * D;
      const bool live = node_rt[rt] >= 0;
      const float inv = live ? 1.f / l_tot[rt] : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t v = o[dt][rt] * inv;
        *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) p.lse[orow] = live ? (m_run[rt] + __log2f(l_tot[rt])) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = (static_cast<int64_t>(bk) * p.nchunk + c) * p.R + r;
      float* dst = p.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t v = o[dt][rt];
        *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) p.part_ml[prow] = make_float2(m_run[rt], l_tot[rt]);
    }
  }
}

// ---------------------------------------------------------- fp32 (VALU) ---
// fp32 inputs are kept fp32 end to end (a bf16 round trip of the inputs
// alone would move the log-sum-exp by ~1e-3). Four lanes share a packed row,
// each holding a quarter of D; keys are staged through LDS 32 at a time.

template <int D>
__global__ __launch_bounds__(kThreads) void attn_split_f32_kernel(AttnParams p) {
  constexpr int DQ = D / 4;
  constexpr int D4 = D / 4;  // float4 per key row
  __shared__ __attribute__((aligned(16))) float sK[kKBf32 * D];
  __shared__ __attribute__((aligned(16))) float sV[kKBf32 * D];
  __shared__ uint32_t sMask[TV_MAX_TREE * (TV_MAX_TREE / 32)];

  const int c = blockIdx.x;
  const int rg = blockIdx.y;
  const int bk = blockIdx.z;
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int tid = threadIdx.x;

  int n, L;
  const int st = seq_check(p, b, n, L);
  if (handle_non_live<D>(p, st, b, kvh, c, rg, kRowsWGf32, tid, kThreads)) return;
  const int nch = num_chunks(L, p.chunk);
  if (c >= nch) return;
  const bool last = (c == nch - 1);
  const int kbeg = c * p.chunk;
  const int kend = last ? L + n : min(kbeg + p.chunk, L);
  if (last) {
    const uint32_t* mrow = p.mask + static_cast<int64_t>(b) * p.T * p.W;
    for (int idx = tid; idx < n * p.W; idx += kThreads) sMask[idx] = mrow[idx];
  }

  const float* kbase = static_cast<const float*>(p.k) + b * p.kv_sb + kvh * p.kv_sh;
  const float* vbase = static_cast<const float*>(p.v) + b * p.kv_sb + kvh * p.kv_sh;

  const int quarter = tid & 3;
  const int r = rg * kRowsWGf32 + (tid >> 2);
  int node = -1;
  int h = 0;
  if (r < p.R) {
    const int i = r / p.G;
    h = kvh * p.G + (r - i * p.G);
    if (i < n) node = i;
  }
  float qv[DQ];
  float ov[DQ];
  if (node >= 0) {
    const float* qrow = static_cast<const float*>(p.q) + b * p.q_sb + node * p.q_st + h * p.q_sh;
#pragma unroll
    for (int d = 0; d < DQ; ++d) qv[d] = qrow[quarter * DQ + d];
  } else {
#pragma unroll
    for (int d = 0; d < DQ; ++d) qv[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DQ; ++d) ov[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int vis_all_end = min(L, kend);

  for (int key0 = kbeg; key0 < kend; key0 += kKBf32) {
    __syncthreads();
    for (int idx = tid; idx < kKBf32 * D4; idx += kThreads) {
      const int key = idx / D4;
      const int d4 = idx - key * D4;
      const int s = key0 + key;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (s < kend) {
        kk = reinterpret_cast<const float4*>(kbase + s * p.kv_ss)[d4];
        vv = reinterpret_cast<const float4*>(vbase + s * p.kv_ss)[d4];
      }
      reinterpret_cast<float4*>(sK)[idx] = kk;
      reinterpret_cast<float4*>(sV)[idx] = vv;
    }
    __syncthreads();
    const int nk = min(kKBf32, kend - key0);
    for (int j = 0; j < nk; ++j) {
      const float* kr = sK + j * D + quarter * DQ;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DQ; ++d) s = fmaf(qv[d], kr[d], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      const int key = key0 + j;
      bool vis = key < vis_all_end;
      if (!vis && key >= L) vis = node >= 0 && tree_visible(sMask, p.W, node, key - L);
      if (!vis) continue;
      const float x = s * p.scale_log2;
      const float m_new = fmaxf(m_run, x);
      const float alpha = exp2f(m_run - m_new);
      const float pr = exp2f(x - m_new);
      l_run = l_run * alpha + pr;
      const float* vr = sV + j * D + quarter * DQ;
#pragma unroll
      for (int d = 0; d < DQ; ++d) ov[d] = fmaf(pr, vr[d], ov[d] * alpha);
      m_run = m_new;
    }
  }

  if (r >= p.R) return;
  const int i = r / p.G;
  if (nch == 1) {
    const int64_t orow = (static_cast<int64_t>(b) * p.T + i) * p.Hq + h;
    const bool live = node >= 0;
    const float inv = live ? 1.f / l_run : 0.f;
#pragma unroll
    for (int d = 0; d < DQ; ++d) p.out[orow * D + quarter * DQ + d] = live ? ov[d] * inv : 0.f;
    if (quarter == 0) p.lse[orow] = live ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t prow = (static_cast<int64_t>(bk) * p.nchunk + c) * p.R + r;
#pragma unroll
    for (int d = 0; d < DQ; ++d) p.part_o[prow * D + quarter * DQ + d] = ov[d];
    if (quarter == 0) p.part_ml[prow] = make_float2(m_run, l_run);
  }
}

// ----------------------------------------------------- log-sum-exp merge ---
// One wave per packed row: merges the chunk partials of sequences with more
// than one chunk: m* = max m_c, l* = sum l_c 2^(m_c - m*),
// O = sum O_c 2^(m_c - m*) / l*, lse = (m* + log2 l*) ln 2.

template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnParams p) {
  constexpr int PER = D / tv::kWave;
  const int bk = blockIdx.y;
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kThreads / tv::kWave) + (threadIdx.x >> 6);
  if (r >= p.R) return;
  int n, L;
  if (seq_check(p, b, n, L) != TV_ROW_OK) return;
  const int nch = num_chunks(L, p.chunk);
  if (nch == 1) return;
  const int i = r / p.G;
  const int h = kvh * p.G + (r - i * p.G);
  const int64_t orow = (static_cast<int64_t>(b) * p.T + i) * p.Hq + h;
  float* dst = p.out + orow * D;
  if (i >= n) {
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[lane + e * tv::kWave] = 0.f;
    if (lane == 0) p.lse[orow] = -INFINITY;
    return;
  }
  const int64_t base = static_cast<int64_t>(bk) * p.nchunk * p.R + r;
  float mstar = -INFINITY;
  for (int cc = 0; cc < nch; ++cc) mstar = fmaxf(mstar, p.part_ml[base + cc * p.R].x);
  float lstar = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int cc = 0; cc < nch; ++cc) {
    const float2 ml = p.part_ml[base + cc * p.R];
    const float w = exp2f(ml.x - mstar);
    lstar += ml.y * w;
    const float* src = p.part_o + (base + cc * p.R) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(src[lane + e * tv::kWave], w, acc[e]);
  }
  const float inv = 1.f / lstar;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[lane + e * tv::kWave] = acc[e] * inv;
  if (lane == 0) p.lse[orow] = (mstar + __log2f(lstar)) * kLn2;
}

int auto_chunk(int B, int T, int Hq, int Hkv, int max_ctx) {
  const int64_t R = static_cast<int64_t>(Hq / Hkv) * T;
  const int64_t rg = (R + kRowsWG - 1) / kRowsWG;
  const int64_t units = static_cast<int64_t>(B) * Hkv * rg;
  const int64_t keys = units * (max_ctx > 0 ? max_ctx : 1);
  const int64_t target = 512;  // about two workgroups per compute unit
  int64_t ch = (keys + target - 1) / target;
  ch = (ch + 63) / 64 * 64;
  if (ch < 256) ch = 256;
  if (ch > 8192) ch = 8192;
  return static_cast<int>(ch);
}

bool valid_sizes(int B, int T, int Hq, int Hkv, int D, int max_ctx, int chunk_keys) {
  if (B < 0 || T < 1 || T > TV_MAX_TREE || Hq < 1 || Hkv < 1 || Hq % Hkv) return false;
  if (Hq / Hkv > TV_MAX_GROUP || max_ctx < 0) return false;
  if (chunk_keys != 0 && (chunk_keys < 64 || chunk_keys > 65536 || chunk_keys % 64)) return false;
  (void)D;
  return true;
}

size_t workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_ctx, int chunk) {
  const int64_t nchunk = max_ctx == 0 ? 1 : (max_ctx + chunk - 1) / chunk;
  if (nchunk <= 1) return 0;
  const int64_t R = static_cast<int64_t>(Hq / Hkv) * T;
  const int64_t rows = static_cast<int64_t>(B) * Hkv * nchunk * R;
  const size_t o_bytes = tvh::align_up(static_cast<size_t>(rows) * D * sizeof(float), 256);
  const size_t ml_bytes = tvh::align_up(static_cast<size_t>(rows) * sizeof(float2), 256);
  return o_bytes + ml_bytes;
}

template <int D>
void launch_all(const AttnParams& p, int in_dtype, int rowgroups, hipStream_t stream) {
  const dim3 grid(p.nchunk, rowgroups, p.B * p.Hkv);
  if (in_dtype == TV_BF16) {
    if (p.parts == 1)
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 1>), grid, dim3(kThreads), 0, stream, p);
    else if (p.parts == 2)
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 3>), grid, dim3(kThreads), 0, stream, p);
  } else
    hipLaunchKernelGGL(attn_split_f32_kernel<D>, grid, dim3(kThreads), 0, stream, p);
  if (p.nchunk > 1) {
    const dim3 cgrid((p.R + 3) / 4, p.B * p.Hkv);
    hipLaunchKernelGGL(attn_combine_kernel<D>, cgrid, dim3(kThreads), 0, stream, p);
  }
}

}  // namespace

extern "C" int tv_tree_attention_auto_chunk(int B, int T, int Hq, int Hkv, int max_ctx) {
  if (!valid_sizes(B, T, Hq, Hkv, 128, max_ctx, 0)) return -1;
  return auto_chunk(B, T, Hq, Hkv, max_ctx);
}

extern "C" size_t tv_tree_attention_workspace_size(int B, int T, int Hq, int Hkv, int D,
                                                   int max_ctx, int chunk_keys) {
  if (!valid_sizes(B, T, Hq, Hkv, D, max_ctx, chunk_keys)) return static_cast<size_t>(-1);
  const int chunk = chunk_keys ? chunk_keys : auto_chunk(B, T, Hq, Hkv, max_ctx);
  return workspace_bytes(B, T, Hq, Hkv, D, max_ctx, chunk);
}

extern "C" int tv_tree_attention(const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                                 const void* k, const void* v, int64_t kv_sb, int64_t kv_sh,
                                 int64_t kv_ss, const int32_t* ctx_len, const int32_t* n_nodes,
                                 const uint32_t* mask, int B, int T, int Hq, int Hkv, int D,
                                 int max_ctx, int kv_capacity, float scale, int in_dtype,
                                 int probability_parts, int chunk_keys, float* out, float* lse,
                                 void* workspace, size_t ws_bytes, int32_t* row_status,
                                 hipStream_t stream) {
  if (!q || !k || !v || !ctx_len || !n_nodes || !mask || !out || !lse || !row_status)
    return TV_ERR_NULL;
  if (in_dtype != TV_F32 && in_dtype != TV_BF16) return TV_ERR_DTYPE;
  if (!valid_sizes(B, T, Hq, Hkv, D, max_ctx, chunk_keys) || kv_capacity < 1)
    return TV_ERR_SHAPE;
  if (probability_parts < 1 || probability_parts > 3) return TV_ERR_SHAPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  const int64_t elem_align = in_dtype == TV_BF16 ? 8 : 4;  // 16 bytes
  if (!tvh::aligned16(q) || !tvh::aligned16(k) || !tvh::aligned16(v) || !tvh::aligned16(out) ||
      !tvh::aligned16(lse))
    return TV_ERR_ALIGN;
  if (q_sb % elem_align || q_st % elem_align || q_sh % elem_align || kv_sb % elem_align ||
      kv_sh % elem_align || kv_ss % elem_align)
    return TV_ERR_ALIGN;
  if (B == 0) return TV_OK;
  const int chunk = chunk_keys ? chunk_keys : auto_chunk(B, T, Hq, Hkv, max_ctx);
  const size_t need = workspace_bytes(B, T, Hq, Hkv, D, max_ctx, chunk);
  if (need > 0 && (!workspace || ws_bytes < need || !tvh::aligned256(workspace)))
    return TV_ERR_WORKSPACE;

  AttnParams p;
  p.q = q;
  p.q_sb = q_sb;
  p.q_st = q_st;
  p.q_sh = q_sh;
  p.k = k;
  p.v = v;
  p.kv_sb = kv_sb;
  p.kv_sh = kv_sh;
  p.kv_ss = kv_ss;
  p.ctx_len = ctx_len;
  p.n_nodes = n_nodes;
  p.mask = mask;
  p.B = B;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.R = p.G * T;
  p.W = (T + 31) / 32;
  p.max_ctx = max_ctx;
  p.kv_capacity = kv_capacity;
  p.chunk = chunk;
  p.nchunk = max_ctx == 0 ? 1 : (max_ctx + chunk - 1) / chunk;
  p.parts = probability_parts;
  p.scale_log2 = scale * kLog2e;
  p.out = out;
  p.lse = lse;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (need > 0) {
    const int64_t rows = static_cast<int64_t>(B) * Hkv * p.nchunk * p.R;
    p.part_o = static_cast<float*>(workspace);
    p.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                          tvh::align_up(rows * D * sizeof(float), 256));
  }
  p.row_status = row_status;
  const int rows_wg = in_dtype == TV_BF16 ? kRowsWG : kRowsWGf32;
  const int rowgroups = (p.R + rows_wg - 1) / rows_wg;
  if (rowgroups > 65535 || static_cast<int64_t>(B) * Hkv > 65535) return TV_ERR_SHAPE;
  if (D == 128)
    launch_all<128>(p, in_dtype, rowgroups, stream);
  else
    launch_all<64>(p, in_dtype, rowgroups, stream);
  return tvh::launch_status();
}
