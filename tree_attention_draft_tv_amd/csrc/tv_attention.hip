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
//   * A persistent grid of one workgroup (8 waves, two per SIMD) per compute
//     unit. The G query heads of a KV head times the T tree rows form
//     R = G*T packed rows (row r = node * G + head-in-group); a workgroup
//     holds up to 256 of them, 32 per wave, so every key and value read from
//     HBM is used by all G heads and all T nodes at once: the contraction
//     over D and over keys is dense, so it runs on MFMA
//     (v_mfma_f32_16x16x32_bf16).
//   * The keys of every live (sequence, KV head, row group) pair are cut into
//     units (split-KV); each workgroup derives the unit size and its own
//     units from ctx_len / n_nodes on the device, balancing the launch. The
//     last unit of a pair also covers the tree block [L, L + n), so tree
//     masking only happens there; partial (m, l, O) go to a workspace and a
//     second kernel merges them with a log-sum-exp combine. A pair with one
//     unit is written directly.
//   * K and V tiles of 64 keys are copied HBM -> LDS with
//     global_load_lds_dwordx4 (no register staging) into a ring of four
//     stages, two tiles ahead of the one being read. K is stored with an
//     XOR swizzle of its 16-byte chunks; V is read transposed with
//     ds_read_b64_tr_b16, so P.V needs no shuffle.
//   * S^T = K Q^T is computed so that a lane's accumulators always belong to
//     one packed row and P^T lands directly in the MFMA B-operand layout.
//   * Softmax in the log2 domain against a fixed per-row reference (the
//     max of the unit's first 32 scores): O is never rescaled, the per-key
//     work is one FMA, one exp2, one add and half a bf16 pack, and a pass
//     whose row sums exceed 2^32 is redone with the exact unit max.
//   * The loop is software-pipelined over 32-key sub-blocks: the S^T MFMAs
//     of sub-block j+1 are issued together with the softmax of sub-block j,
//     so matrix cores and VALU work side by side within a wave.
#include <algorithm>
#include <type_traits>

#include "tv_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKB = 64;            // keys per LDS tile
constexpr int kThreads = 512;      // 8 waves, two per SIMD
constexpr int kRowsWave = 32;      // packed rows per wave (2 tiles of 16)
constexpr int kRT = 2;             // row tiles per wave
constexpr int kRing = 4;           // LDS tiles: one finishing, one current, two in flight
constexpr int kRowsWG = kRowsWave * (kThreads / tv::kWave);
constexpr int kThreadsF32 = 256;   // fp32 kernel: 4 lanes per packed row
constexpr int kThreadsCombine = 256;
constexpr int kRowsWGf32 = 64;     // packed rows per fp32 workgroup (4 lanes each)
constexpr int kKBf32 = 32;         // keys per fp32 LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRowSumLimit = 4294967296.0f;  // 2^32: a row sum above it means P ran away
constexpr float kRowSumFloor = 2.3283064365386963e-10f;  // 2^-32

// Reference max of a row: 0 when the row saw no key (-inf).
__device__ __forceinline__ float finite_ref(float m) { return m == -INFINITY ? 0.f : m; }

struct AttnParams {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_sh, kv_ss;
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const uint32_t* mask;
  const int32_t* row_start;  // packed rows: first row of sequence b (null: row b T + i)
  int rows_total;            // packed rows: rows of q / out / lse
  int B, T, Hq, Hkv, G, R, W, max_ctx, kv_capacity, parts;
  uint32_t g_mul;  // ceil(2^16 / G): packed row r -> tree row (r * g_mul) >> 16
  int kunit;    // keys per unit if fixed by the caller, 0 = balanced on the device
  int rows_wg;  // packed rows per workgroup (one row group)
  int RG;       // row groups per (sequence, KV head)
  int nw;       // workgroups launched (a multiple of 8)
  float scale_log2;
  void* out;        // [rows][Hq][D] fp32, or bf16 when out_bf16
  int out_bf16;
  float* lse;
  int32_t* sched;   // table for the combine (see write_sched)
  float* part_o;    // [unit][rows_wg][D], un-normalised: fp32 in d order, or int16 fixed
                    // point (q16) with each row as [g][dt][e] (d = 16 dt + 4 g + e)
  float4* part_ml;  // per pair [rows_wg][unit of the pair]: (reference max in log2 units, sum,
                    // int16 scale, 0)
  int32_t* row_status;
};

// The kernels' parameter type: the packed-row layout is a compile-time
// choice, so the padded kernels carry none of its address arithmetic.
template <bool PK>
struct AttnParamsT : AttnParams {
  static constexpr bool kPacked = PK;
};

// Status of a sequence with n live rows, L committed keys and (packed rows
// only) first row start: TV_ROW_OK (live), -1 (padded: n == 0) or an error.
template <class P>
__device__ __forceinline__ int seq_status(const P& p, int n, int L, int start) {
  if (n < 0 || n > p.T) return TV_ROW_NNODES;
  if (n == 0) return -1;
  if (P::kPacked && (start < 0 || start > p.rows_total - n)) return TV_ROW_BAD_START;
  if (L < 0 || L > p.max_ctx || static_cast<int64_t>(L) + n > p.kv_capacity)
    return TV_ROW_CTX_BOUND;
  return TV_ROW_OK;
}

// First output row of sequence b: its packed start, else b T.
template <class P>
__device__ __forceinline__ int64_t seq_row0(const P& p, int b, int start) {
  return P::kPacked ? static_cast<int64_t>(start) : static_cast<int64_t>(b) * p.T;
}

// Four consecutive output entries starting at entry `off` of out: fp32, or
// bf16 rounded to nearest even.
__device__ __forceinline__ void store_out4(const AttnParams& p, int64_t off, float a, float b,
                                           float c, float d) {
  if (p.out_bf16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t h;
    h[0] = static_cast<__bf16>(a);
    h[1] = static_cast<__bf16>(b);
    h[2] = static_cast<__bf16>(c);
    h[3] = static_cast<__bf16>(d);
    *reinterpret_cast<bf16x4_t*>(static_cast<uint16_t*>(p.out) + off) = h;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) = make_float4(a, b, c, d);
  }
}

// a / b for 0 <= a, 1 <= b (exact). Below 2^22 the float quotient through
// the hardware reciprocal is within 1 of the true one and one correction
// step finishes it (a few instructions instead of a long integer division
// sequence); larger dividends divide exactly.
__device__ __forceinline__ int div_fast(int a, int b) {
  if (a >= (1 << 22)) return a / b;
  int q = static_cast<int>(static_cast<float>(a) * __builtin_amdgcn_rcpf(static_cast<float>(b)));
  const int r = a - q * b;
  q += static_cast<int>(r >= b) - static_cast<int>(r < 0);
  return q;
}
// a / b for 0 <= a < 2^52, 1 <= b < 2^31 (exact): the correctly rounded
// double quotient is within 1 of the true one; one correction step. (A
// 64-bit integer division is a long instruction sequence.)
__device__ __forceinline__ int64_t div64_fast(int64_t a, int64_t b) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
  const int64_t r = a - q * b;
  q += static_cast<int64_t>(r >= b) - static_cast<int64_t>(r < 0);
  return q;
}

// Packed row r -> tree row r / G with the host's multiplier ceil(2^16 / G):
// exact for r < 2048 and G <= 32, which TV_MAX_TREE * TV_MAX_GROUP keeps.
__device__ __forceinline__ int row_node(const AttnParams& p, int r) {
  return static_cast<int>((static_cast<uint32_t>(r) * p.g_mul) >> 16);
}

// Status of sequence b (see seq_status); also returns its n, L and packed
// start (0 without packed rows).
template <class P>
__device__ __forceinline__ int seq_check(const P& p, int b, int& n, int& L, int& start) {
  n = p.n_nodes[b];
  L = p.ctx_len[b];
  start = P::kPacked ? p.row_start[b] : 0;
  return seq_status(p, n, L, start);
}


// Padded (n == 0) and invalid sequences: every output row gets the padding
// values (O = 0, lse = -inf) and every sequence its status, spread over the
// whole grid. With packed rows a sequence owns only its n rows, written when
// n and its start are valid (a bounds error writes nothing). st0 holds the statuses of the first 64 sequences (lane b:
// sequence b); later blocks of 64 are read in one round before their stores
// (a load placed after the stores would wait for them: the compiler cannot
// rule out that they alias the length arrays). THREADS is the workgroup
// size and the grid is p.nw workgroups (reading blockDim would cost a memory
// round trip at the start of every workgroup).
template <int D, int THREADS, class P>
__device__ void finish_non_live(const P& p, int st0, int n0, int s0) {
  constexpr int D4 = D / 4;
  const int nthreads = p.nw * THREADS;
  const int gtid = blockIdx.x * THREADS + threadIdx.x;
  const int lane = threadIdx.x & 63;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const bool has = b0 + lane < p.B;
    int st = st0, n = n0, L, start = s0;
    if (b0 > 0 && has) st = seq_check(p, b0 + lane, n, L, start);
    if (gtid < 64 && has) p.row_status[b0 + lane] = (st == -1) ? TV_ROW_OK : st;
    // Rows to clear: all T in the padded layout, the sequence's own n rows
    // when packed (none if n or the start is out of bounds).
    const int nclr = !P::kPacked ? p.T
                     : (st == TV_ROW_CTX_BOUND ? n : 0);
    for (uint64_t m = __ballot(has && st != TV_ROW_OK && nclr > 0); m; m &= m - 1) {
      const int bl = __builtin_ctzll(m);
      const int b = b0 + bl;
      const int rows = __builtin_amdgcn_readlane(nclr, bl);
      const int64_t r0 = seq_row0(p, b, __builtin_amdgcn_readlane(start, bl));
      const int64_t o0 = r0 * p.Hq * D;
      float* l = p.lse + r0 * p.Hq;
      const int per_seq = rows * p.Hq * D4;
      for (int idx = gtid; idx < per_seq; idx += nthreads) {
        store_out4(p, o0 + 4 * static_cast<int64_t>(idx), 0.f, 0.f, 0.f, 0.f);
        if (idx % D4 == 0) l[idx / D4] = -INFINITY;
      }
    }
  }
}

// ------------------------------------------------------------ schedule ---
// The keys of every live (sequence, KV head, row group) pair are processed
// as pieces, one workgroup per piece at a time, under one of two partitions:
//  * units (a caller-fixed chunk_keys, or one unit per pair when the caller
//    passed no workspace for partials): a pair's keys cut into units of K
//    keys, numbered pair-major; workgroup w takes units w', w' + nw, ...
//    With a fixed chunk a row's result does not depend on the other
//    sequences of the batch.
//    With chunk_keys == 0 (balanced, the default) K is the smallest size
//    that gives at most one unit per workgroup: units then split each pair
//    evenly and never straddle pairs.
//  * stream-K (balanced, when the live pairs P outnumber the workgroups):
//    every workgroup takes floor(P / nw) whole pairs (written directly),
//    and the other P mod nw pairs, laid on a line of tiles (below), are
//    shared out equally over the workgroups, which cuts them into pieces
//    (whole pairs alone left a second pass to a few workgroups). Units are
//    kept while they fit: a piece costs its own start and epilogue.
// Every wave derives the partition from ctx_len / n_nodes by itself (no host
// sync, no communication between workgroups); the combine kernel reads the
// table workgroup 0 writes.

constexpr int kMinUnit = 128;  // smallest balanced unit (keys)

// Committed length of sequence b if it is live, else -1.
template <class P>
__device__ __forceinline__ int live_len(const P& p, int b) {
  int n, L, start;
  return seq_check(p, b, n, L, start) == TV_ROW_OK ? L : -1;
}

// Every wave loads the committed lengths of the first 64 sequences once
// (lane b holds sequence b, -1 if not live, its n in n0, packed start in s0
// and status in st0); longer batches re-read the rest from memory (L2) in
// each pass.
template <class P>
__device__ __forceinline__ int lane_len(const P& p, int& n0, int& s0, int& st0) {
  const int lane = threadIdx.x & 63;
  int L = -1;
  n0 = 0;
  s0 = 0;
  st0 = TV_ROW_OK;
  if (lane < p.B) {
    int n, start;
    st0 = seq_check(p, lane, n, L, start);
    if (st0 != TV_ROW_OK) L = -1;
    n0 = n;
    s0 = start;
  }
  return L;
}
// (n, L, first output row) of live sequence b: from the lane cache for b < 64.
template <class P>
__device__ __forceinline__ void unit_seq(const P& p, int b, int len0, int n0, int s0,
                                         int& n, int& L, int64_t& row0) {
  int start;
  if (b < 64) {
    n = __builtin_amdgcn_readlane(n0, b);
    L = __builtin_amdgcn_readlane(len0, b);
    start = __builtin_amdgcn_readlane(s0, b);
  } else {
    seq_check(p, b, n, L, start);
  }
  row0 = seq_row0(p, b, start);
}
template <class P>
__device__ __forceinline__ int block_len(const P& p, int b0, int len0) {
  const int b = b0 + (threadIdx.x & 63);
  return b0 == 0 ? len0 : (b < p.B ? live_len(p, b) : -1);
}
// Balanced units: the tree block (masked, unpipelined) costs about as much as
// this many committed keys, so the last unit of a pair, which holds it, gets
// that many fewer committed keys (half a unit at most: tree_extra(K)).
constexpr int kTreeExtra = 128;
__device__ __forceinline__ int tree_extra(int K) { return min(kTreeExtra, K >> 1); }

// Units of a pair with L committed keys and K keys per unit.
__device__ __forceinline__ int pair_units(const AttnParams& p, int L, int K) {
  const int x = p.kunit > 0 ? 0 : tree_extra(K);
  return L == 0 ? 1 : div_fast(L + x + K - 1, K);
}
// First committed key of unit c of a pair: c K for fixed chunks; in balanced
// mode the units split L + x evenly (x = tree_extra(K)), boundaries rounded
// down to whole 64-key tiles. Since K >= 2 x, the last unit keeps at least
// one committed key (no boundary passes L) and every unit at most K + 63 keys.
__device__ __forceinline__ int unit_start(const AttnParams& p, int L, int K, int nch, int c) {
  if (p.kunit > 0) return min(c * K, L);
  const int x = tree_extra(K);
  // c <= nch <= 1024 units per pair, so below 2^22 the product fits 32 bits.
  if (L < (1 << 22) - kTreeExtra)
    return static_cast<int>(static_cast<uint32_t>(c) * static_cast<uint32_t>(L + x) /
                            static_cast<uint32_t>(nch)) & ~63;
  return static_cast<int>(div64_fast(static_cast<int64_t>(c) * (L + x), nch)) & ~63;
}

__device__ __forceinline__ int units_of(const AttnParams& p, int L, int K) {
  return L < 0 ? 0 : pair_units(p, L, K) * p.Hkv * p.RG;
}

// Committed length of sequence b (live): from the lane cache for b < 64.
template <class P>
__device__ __forceinline__ int seq_len(const P& p, int b, int len0) {
  return b < 64 ? __builtin_amdgcn_readlane(len0, b) : live_len(p, b);
}

// Units of the whole launch (wave-uniform; every lane must call).
template <class P>
__device__ int total_units(const P& p, int len0, int K) {
  int acc = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) acc += units_of(p, block_len(p, b0, len0), K);
  return tv::wave_sum_i32(acc);
}

// Keys per unit: the caller's fixed chunk; else the smallest multiple of 64
// (at least kMinUnit) that cuts the launch into at most nw units, so that a
// single pass of the nw workgroups covers it with the least work per unit;
// else (more pairs than workgroups, or no workspace for partials) one unit
// per pair: L + kTreeExtra <= K for every sequence. `stream_k` tells whether
// the balanced partition leaves more units than workgroups (the stream-K
// line then takes over); the search has counted them already.
template <class P>
__device__ int choose_unit(const P& p, int len0, bool& stream_k) {
  stream_k = false;
  if (p.kunit > 0) return p.kunit;
  // Sequences in lanes (the first 64 from len0, later blocks from memory),
  // reduced across the wave.
  int maxl = 0, keys = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int L = block_len(p, b0, len0);
    maxl = max(maxl, L);
    keys += max(L, 0);
  }
  maxl = tv::wave_max_i32(maxl);
  keys = tv::wave_sum_i32(keys);
  const int hi = max(kMinUnit, (maxl + kTreeExtra + 63) / 64 * 64);
  if (p.part_o == nullptr) return hi;
  // Lower bound: the committed keys of all pairs spread evenly over nw
  // units; rounding each pair up adds at most one unit per pair, so a few
  // steps of 64 usually reach the answer.
  const int64_t pair_keys = static_cast<int64_t>(keys) * p.Hkv * p.RG;
  int lo = static_cast<int>(div64_fast(pair_keys + p.nw - 1, p.nw));
  lo = max(kMinUnit, (lo + 63) / 64 * 64);
  if (lo >= hi) {
    stream_k = total_units(p, len0, hi) > p.nw;
    return hi;
  }
  // Each candidate's unit count is one wave reduction over the sequences'
  // lanes (no memory for the first 64): a few steps of 64 from the bound,
  // then a bisection.
  for (int step = 0; step < 4 && lo < hi; ++step, lo += 64)
    if (total_units(p, len0, lo) <= p.nw) return lo;
  if (total_units(p, len0, hi) > p.nw) {
    stream_k = true;
    return hi;
  }
  int bad = lo - 64;  // units(bad) > nw >= units(hi)
  int good = hi;
  while (good - bad > 64) {
    const int mid = (bad / 64 + good / 64) / 2 * 64;
    if (total_units(p, len0, mid) <= p.nw)
      good = mid;
    else
      bad = mid;
  }
  return good;
}

// ---- stream-K line. Every live pair is a run of pair_tiles(L) tiles:
// ceil(L / 64) of committed keys, then kTreeTiles standing for its masked
// tree block (about what it costs); pairs lie pair-major along the line
// (the pairs of a sequence consecutive, KV head major, then row group).
// The first p0 = nw floor(P / nw) pairs are whole-pair units; the rest of
// the line, from tile off, holds W tiles. Active workgroup v < nwa takes
// tiles off + [sk_start(v), sk_start(v + 1)), sk_start(v) = floor(v W /
// nwa), nwa = min(nw, W): equal shares of at least one tile. The piece of
// pair p that workgroup v holds keeps its partial rows in slot (p - p0) +
// v: slots increase along the line, so the slots of a pair are consecutive
// from (p - p0) + v_lo and there are fewer than P + nw of them.
constexpr int kTreeTiles = kTreeExtra / kKB;

struct SkLine {
  int W;    // tiles of the shared part of the line (the host keeps the line below 2^31)
  int nwa;  // active workgroups of the shared part, 0 when it is empty
  int off;  // line tiles before it
  int p0;   // pairs before it (whole-pair units)
};

__device__ __forceinline__ int pair_tiles(int L) { return (L + kKB - 1) / kKB + kTreeTiles; }

__device__ __forceinline__ int sk_start(const SkLine& s, int v) {
  return v >= s.nwa ? s.W : static_cast<int>(div64_fast(static_cast<int64_t>(v) * s.W, s.nwa));
}

// The workgroup whose share holds tile x of the shared part (0 <= x < W):
// the largest v with sk_start(v) <= x.
__device__ __forceinline__ int sk_owner(const SkLine& s, int x) {
  return static_cast<int>(div64_fast(static_cast<int64_t>(x + 1) * s.nwa - 1, s.W));
}

// The live sequence b whose tiles hold line tile `key` (by_pair: whose
// pairs hold pair index `key`), with the tiles (sb) and pairs (pb) before it
// on the line: lane scans of the per-sequence tiles and live flags, 64
// sequences a block, and a ballot (wave-uniform; b = -1 past the line).
template <class P>
__device__ void sk_locate(const P& p, int len0, int key, bool by_pair, int& b, int& sb, int& pb) {
  const int lane = threadIdx.x & 63;
  const int per = p.Hkv * p.RG;
  int base = 0, pbase = 0;
  b = -1;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int L = block_len(p, b0, len0);
    const int live = L < 0 ? 0 : 1;
    const int work = live * per * pair_tiles(max(L, 0));
    const int inc = tv::wave_scan_i32(work, lane);
    const int linc = tv::wave_scan_i32(live, lane);
    const int tot = __builtin_amdgcn_readlane(inc, 63);
    const int ltot = __builtin_amdgcn_readlane(linc, 63);
    if (by_pair ? key < pbase + per * ltot : key < base + tot) {
      const int l = __builtin_ctzll(__ballot(by_pair ? pbase + per * linc > key : base + inc > key));
      b = b0 + l;
      sb = base + __builtin_amdgcn_readlane(inc - work, l);
      pb = pbase + per * __builtin_amdgcn_readlane(linc - live, l);
      return;
    }
    base += tot;
    pbase += per * ltot;
  }
}

// The shared part of the line (wave-uniform; every lane calls).
template <class P>
__device__ SkLine sk_line(const P& p, int len0) {
  const int per = p.Hkv * p.RG;
  int w = 0, live = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int L = block_len(p, b0, len0);
    w += L < 0 ? 0 : per * pair_tiles(L);
    live += L < 0 ? 0 : 1;
  }
  const int total = tv::wave_sum_i32(w);
  const int pairs = per * tv::wave_sum_i32(live);
  SkLine s;
  s.p0 = div_fast(pairs, p.nw) * p.nw;
  s.off = total;
  if (s.p0 < pairs) {
    int b, sb, pb;
    sk_locate(p, len0, s.p0, true, b, sb, pb);
    s.off = sb + (s.p0 - pb) * pair_tiles(seq_len(p, b, len0));
  }
  s.W = total - s.off;
  s.nwa = min(p.nw, s.W);
  return s;
}

// The pieces of the pair whose tiles start at sp (wp tiles, first pair index
// pidx on the line): first slot, piece count and the index of the first
// empty piece. Pieces jt .. np - 2 hold only tree-cost tiles without the
// pair's end, so no keys: they are skipped by the split and the combine.
struct SkPair {
  int base, np, jt, v_lo;
};
__device__ __forceinline__ SkPair sk_pair(const SkLine& s, int sp, int wp, int pidx) {
  SkPair r;
  r.v_lo = sk_owner(s, sp);
  r.np = sk_owner(s, sp + wp - 1) - r.v_lo + 1;
  r.base = pidx + r.v_lo;
  const int ct = wp - kTreeTiles;  // committed tiles
  r.jt = ct > 0 ? sk_owner(s, sp + ct - 1) - r.v_lo + 1 : 0;
  return r;
}

// Unit u -> (b, kvh, rg, c) and the pair's unit count nch; false past the
// last unit (wave-uniform; every lane must call). An inclusive scan of the
// per-sequence unit counts over the lanes, 64 sequences per block, and a
// ballot for the first sequence whose units reach past u.
template <class P>
__device__ bool decode_unit(const P& p, int len0, int K, int u, int& b, int& kvh, int& rg,
                            int& c, int& nch) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int cnt = units_of(p, block_len(p, b0, len0), K);
    const int inc = tv::wave_scan_i32(cnt, lane);
    const int tot = __builtin_amdgcn_readlane(inc, 63);
    if (u < base + tot) {
      const uint64_t hit = __ballot(base + inc > u);
      const int l = __builtin_ctzll(hit);
      b = b0 + l;
      const int cnt_l = __builtin_amdgcn_readlane(cnt, l);
      const int per_pair = div_fast(cnt_l, p.Hkv * p.RG);
      const int local = u - base - (__builtin_amdgcn_readlane(inc, l) - cnt_l);
      nch = per_pair;
      const int pair = div_fast(local, per_pair);
      c = local - pair * per_pair;
      kvh = div_fast(pair, p.RG);
      rg = pair - kvh * p.RG;
      return true;
    }
    base += tot;
  }
  return false;
}

// Table for the combine kernel. Unit mode: [0] = K, [1] = -1, [4 + 2 b] =
// first unit of sequence b. Stream-K: [0] = W, [1] = nwa, [2] = off, [3] =
// p0, [4 + 2 b] = line tiles before sequence b, [5 + 2 b] = pairs before it.
template <class P>
__device__ void write_sched(const P& p, int len0, int K, const SkLine& s, bool stream_k) {
  const int lane = threadIdx.x & 63;
  const int per = p.Hkv * p.RG;
  if (lane == 0) {
    p.sched[0] = stream_k ? s.W : K;
    p.sched[1] = stream_k ? s.nwa : -1;
    p.sched[2] = s.off;
    p.sched[3] = s.p0;
  }
  int base = 0, pbase = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int L = block_len(p, b0, len0);
    const int live = L < 0 ? 0 : 1;
    const int cnt = stream_k ? live * per * pair_tiles(max(L, 0)) : units_of(p, L, K);
    const int inc = tv::wave_scan_i32(cnt, lane);
    const int linc = tv::wave_scan_i32(live, lane);
    if (b0 + lane < p.B) {
      p.sched[4 + 2 * (b0 + lane)] = base + inc - cnt;
      p.sched[5 + 2 * (b0 + lane)] = pbase + per * (linc - live);
    }
    base += __builtin_amdgcn_readlane(inc, 63);
    pbase += per * __builtin_amdgcn_readlane(linc, 63);
  }
}

// First unit of workgroup w: the nw / 8 workgroups that share w mod 8 (the
// XCD that hardware dispatch gives them) take one contiguous run of units,
// so the units of a pair mostly share an L2.
__device__ __forceinline__ int first_unit(const AttnParams& p) {
  const int w = blockIdx.x;
  return (w & 7) * (p.nw >> 3) + (w >> 3);
}

// One piece of work: pair (b, kvh, rg), keys from kbeg: to kcut, or with
// `last` (it holds the tree block) through the committed keys and the tree
// block (to L + n). Partial rows in slot `slot`, the (m, l) records of the
// pair's np pieces from slot `base` (this one is piece j); np == 1: the piece
// is the whole pair and is written directly.
struct Piece {
  int b, kvh, rg;
  int kbeg, kcut;
  bool last;
  int slot, base, np, j;
};

// Unit mode: unit u as a piece; false past the last unit (wave-uniform).
template <class P>
__device__ bool unit_piece(const P& p, int len0, int K, int u, Piece& pc) {
  int b, kvh, rg, c, nch;
  if (!decode_unit(p, len0, K, u, b, kvh, rg, c, nch)) return false;
  const int L = seq_len(p, b, len0);
  pc.b = b;
  pc.kvh = kvh;
  pc.rg = rg;
  pc.last = c == nch - 1;
  pc.kbeg = unit_start(p, L, K, nch, c);
  pc.kcut = pc.last ? L : unit_start(p, L, K, nch, c + 1);
  pc.slot = u;
  pc.base = u - c;
  pc.np = nch;
  pc.j = c;
  return true;
}

// Stream-K: the next non-empty piece of workgroup v's share from line tile
// x on; next_x is the tile after it. False when the share holds no more.
template <class P>
__device__ bool sk_piece(const P& p, int len0, const SkLine& s, int v, int x, Piece& pc,
                         int& next_x) {
  const int e = s.off + sk_start(s, v + 1);
  while (x < e) {
    int b, sb, pb;
    sk_locate(p, len0, x, false, b, sb, pb);
    if (b < 0) return false;
    const int L = seq_len(p, b, len0);
    const int wp = pair_tiles(L);
    const int q = div_fast(x - sb, wp);
    const int sp = sb + q * wp;
    const int x1 = min(e - sp, wp);
    next_x = sp + x1;
    const bool last = x1 == wp;
    const int kbeg = min((x - sp) * kKB, L);
    const int kcut = last ? L : min(x1 * kKB, L);
    if (!last && kbeg >= kcut) {  // tree-cost tiles only, without the pair's end
      x = next_x;
      continue;
    }
    const SkPair pr = sk_pair(s, sp - s.off, wp, pb + q - s.p0);
    pc.b = b;
    pc.kvh = div_fast(q, p.RG);
    pc.rg = q - pc.kvh * p.RG;
    pc.kbeg = kbeg;
    pc.kcut = kcut;
    pc.last = last;
    pc.np = pr.np;
    pc.base = pr.base;
    pc.j = v - pr.v_lo;
    pc.slot = pr.base + pc.j;
    return true;
  }
  return false;
}

// Runs run(piece) for every piece of this workgroup, with a barrier between
// pieces (the previous piece's LDS reads are done). Unit mode: units
// first_unit(blockIdx) + k nw. Stream-K: the whole pairs first_unit(blockIdx)
// + k nw below p0, then share v = (blockIdx mod 8) c + blockIdx / 8 (c =
// ceil(nwa / 8)) if v < nwa and blockIdx / 8 < c, so that neighbouring
// shares (which cut the same pairs) run on one XCD under round-robin
// dispatch.
template <class P, class Run>
__device__ __forceinline__ void for_each_piece(const P& p, int len0, int K, const SkLine& s,
                                               bool stream_k, Run run) {
  Piece pc;
  bool first = true;
  if (stream_k) {
    // Whole pairs first (units of one pair each: K fits every pair), then
    // this workgroup's share of the rest of the line.
    for (int u = first_unit(p); u < s.p0; u += p.nw) {
      unit_piece(p, len0, K, u, pc);
      if (!first) __syncthreads();
      first = false;
      run(pc);
    }
    const int per_xcd = (s.nwa + 7) >> 3;
    const int k = blockIdx.x >> 3;
    const int v = (blockIdx.x & 7) * per_xcd + k;
    if (k >= per_xcd || v >= s.nwa) return;
    int x = s.off + sk_start(s, v), nx;
    while (sk_piece(p, len0, s, v, x, pc, nx)) {
      if (!first) __syncthreads();
      first = false;
      run(pc);
      x = nx;
    }
  } else {
    for (int u = first_unit(p);; u += p.nw) {
      if (!unit_piece(p, len0, K, u, pc)) break;
      if (!first) __syncthreads();
      first = false;
      run(pc);
    }
  }
}


__device__ __forceinline__ bool tree_visible(const uint32_t* s_mask, int W, int node, int j) {
  return (s_mask[node * W + (j >> 5)] >> (j & 31)) & 1u;
}

// ------------------------------------------------------------ bf16 MFMA ---

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// LDS tiles hold 64 keys of K and V in [key][d] order, rows unpadded, with an
// XOR swizzle that depends only on the key's low bits:
//   K: 16-byte chunk c of key k sits at chunk c ^ (k mod D/8);
//   V: 32-byte chunk c of key k sits at chunk c ^ (k mod D/16 (max 8)).
// The S^T = K Q^T operand reads 16 consecutive keys at one chunk (distinct
// bank groups), the transposing V reads take 8 consecutive keys at one
// chunk (distinct 32-byte groups), and every lane's read addresses differ
// only by compile-time offsets from a few per-lane bases.
template <int D>
__device__ __forceinline__ int k_swz(int key) {
  return key & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int key) {
  return key & (D / 16 - 1);
}

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding).
#define TV_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14))

// Workgroup barrier for the LDS ring: waits for this wave's LDS operations
// only (lgkmcnt(0)), then s_barrier. __syncthreads() would also wait for
// every outstanding global load (vmcnt(0)), which drains the HBM->LDS copies
// of the tiles still in flight; the ring's explicit TV_WAIT_VMCNT waits
// already guarantee that the tile about to be read has landed.
// A 16-byte store at device scope (sc1): written through the XCD's L2 to
// memory instead of staying dirty there. Used for the fp32 split-KV
// partials, which only the combine reads: the end of the split kernel then
// has no L2 write-back of ~30 MB to wait for (-2 us per call at C3). The compiler does
// not see the store inside the asm, so the asm itself supplies the wait
// states that a VALU write to the data registers of a preceding store of
// more than 8 bytes needs (2 on gfx950; s_nop 2 gives 3): the registers are
// free for reuse right after the statement. (Two agent-scope atomic 8-byte
// stores, which the compiler does track, cost the C3 kernel 39 spilled
// registers, some inside the main loop.) V is a 16-byte vector type.
template <class V>
__device__ __forceinline__ void store_wt16(void* ptr, V v) {
  static_assert(sizeof(V) == 16, "16-byte stores");
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 2" ::"v"(ptr), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane i's bytes
// land at lds_base + 16 i, read from sbase + voff (a wave-uniform base in
// SGPRs plus a 32-bit byte offset per lane: one VGPR per address instead of
// a 64-bit pair, which keeps the kernel's VGPRs from spilling). Issued as
// inline assembly so that the compiler does not serialise it against
// unrelated LDS reads of other ring stages; completion is awaited explicitly
// with TV_WAIT_VMCNT before the barrier that publishes the tile.
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)lds_base));
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "{m0}"(lds)
      : "memory");
}

// A wave-uniform pointer, moved to SGPRs (the unit being processed is the
// same in every lane, but the compiler cannot prove it).
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int V>
using IC = std::integral_constant<int, V>;

// a (low half) and b (high half) rounded to bf16, nearest even.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t t;
  t[0] = static_cast<__bf16>(a);
  t[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, t);
}

// The high 16 bits of b and of a side by side: (b >> 16) << 16 | a >> 16,
// i.e. the bf16 truncations of a (low half) and b (high half).
__device__ __forceinline__ uint32_t high_halves(float b, float a) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Max over the four lanes l, l^16, l^32, l^48 (the four lane groups that
// hold the same packed row), with the gfx950 row-swap permutes (no LDS).
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int PARTS, bool PACKED>
__global__ __launch_bounds__(kThreads) void attn_split_bf16_kernel(AttnParamsT<PACKED> p) {
  constexpr int CH16 = D / 8;                    // 16-byte chunks per key row
  constexpr int KS = D / 32;                     // MFMA k-steps along D
  constexpr int DT = D / 16;                     // 16-wide d tiles of O
  constexpr int TILE = kKB * D;                  // elements per tensor per LDS tile
  constexpr int LOADS = kKB * CH16 / kThreads;   // 16-byte loads per thread per tensor
  constexpr int KEYS_PER_LOAD = kThreads / CH16; // keys covered by one load round

  __shared__ __attribute__((aligned(16))) uint16_t sK[kRing * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kRing * TILE];
  __shared__ uint32_t sMask[TV_MAX_TREE * (TV_MAX_TREE / 32)];
  __shared__ int sOvf;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int n0, s0, st0;
  const int len0 = lane_len(p, n0, s0, st0);
  bool stream_k;
  const int K = choose_unit(p, len0, stream_k);
  SkLine sk{0, 0, 0, 0};
  if (stream_k) sk = sk_line(p, len0);
  if (p.sched && blockIdx.x == 0 && wave == 0) write_sched(p, len0, K, sk, stream_k);

  // ---- one piece: keys [kbeg, kend) of (b, kvh), packed rows of row group rg ----
  auto run_unit = [&](const Piece& pc) __attribute__((always_inline)) {
  const int b = pc.b, kvh = pc.kvh, rg = pc.rg;
  int n, L;
  int64_t srow0;  // output row of tree row 0
  unit_seq(p, b, len0, n0, s0, n, L, srow0);
  const bool last = pc.last;
  const int kbeg = pc.kbeg;
  const int kend = last ? L + n : pc.kcut;
  const int ntile = (kend - kbeg + kKB - 1) / kKB;
  const int kv_ss = static_cast<int>(p.kv_ss);  // host checks capacity * stride < 2^31

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), loaded first ----
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int row0 = rg * kRowsWG + wave * kRowsWave;
  const bool wave_active = row0 < p.R;
  // Packed rows: q row of tree row 0 is the sequence's start (no batch stride).
  const int64_t qseq = PACKED ? srow0 * p.q_st : b * p.q_sb;
  bf16x8_t qf[kRT][KS];
  int node_rt[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = row0 + rt * 16 + l16;
    const int i = row_node(p, r);
    const int node = (r < p.R && i < n) ? i : -1;
    node_rt[rt] = node;
    const int h = kvh * p.G + (r - i * p.G);
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qseq +
                           (node < 0 ? 0 : node) * p.q_st + (node < 0 ? 0 : h) * p.q_sh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u16x8_t v = *reinterpret_cast<const u16x8_t*>(qrow + 32 * s + 8 * g);
      qf[rt][s] = __builtin_bit_cast(bf16x8_t, node < 0 ? u16x8_t(0) : v);
    }
  }
  if (last) {
    const uint32_t* mrow = p.mask + static_cast<int64_t>(b) * p.T * p.W;
    for (int idx = tid; idx < n * p.W; idx += kThreads) sMask[idx] = mrow[idx];
  }

  // ---- tile loads: HBM -> LDS directly (16 bytes per lane; lane i's bytes
  // land at base + 16 i). The swizzle is applied on the global side: the
  // lane filling LDS slot (key, chunk) fetches the chunk that belongs there.
  // A thread's chunk is the same in every load round. Keys at or past kend
  // are never read: their slots re-read key kend - 1 (finite data that the
  // softmax gives probability 0). Tile t lives in ring stage t mod kRing. ----
  const void* kbase =
      uniform_ptr(static_cast<const uint16_t*>(p.k) + b * p.kv_sb + kvh * p.kv_sh);
  const void* vbase =
      uniform_ptr(static_cast<const uint16_t*>(p.v) + b * p.kv_sb + kvh * p.kv_sh);
  const int ld_key = tid / CH16;
  const int ld_pch = tid - ld_key * CH16;
  const int ld_kch = ld_pch ^ k_swz<D>(ld_key);
  const int ld_vch = 2 * ((ld_pch >> 1) ^ v_swz<D>(ld_key)) + (ld_pch & 1);
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const int key0 = kbeg + t * kKB + ld_key;
    uint16_t* dK = sK + (t & (kRing - 1)) * TILE;
    uint16_t* dV = sV + (t & (kRing - 1)) * TILE;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      // Byte offsets below 2^32: the host bounds capacity * stride + D by 2^31 elements.
      const uint32_t row = static_cast<uint32_t>(min(key0 + it * KEYS_PER_LOAD, kend - 1)) *
                           static_cast<uint32_t>(kv_ss) * 2u;
      const int lds_off = (it * kThreads + wave * tv::kWave) * 8;
      lds_copy16(kbase, row + static_cast<uint32_t>(ld_kch * 16), dK + lds_off);
      lds_copy16(vbase, row + static_cast<uint32_t>(ld_vch * 16), dV + lds_off);
    }
  };
  // Max-only pass (rare): tile t becomes readable once every copy this
  // thread has in flight has landed (vmcnt(0), right whatever else is
  // outstanding); publish with a barrier, then reuse the stage of tile
  // t - 2, which every wave has finished reading, for tile t + 2. Tile t + 1
  // was issued a tile earlier, so it has usually landed by then anyway. The
  // main pass below counts its own copies instead and keeps tile t + 1 in
  // flight.
  auto enter_tile = [&](int t) __attribute__((always_inline)) {
    TV_WAIT_VMCNT(0);
    lds_barrier();
    if (t + 2 < ntile) issue_tile(t + 2);
  };

  f32x4_t o[DT][kRT];
  // Per row: mref = the reference max (log2 units) that P = 2^(s cs - mref)
  // is taken against; per lane: l_run = the partial sum; per row: l_tot =
  // the row sum after a pass.
  float mref[kRT], neg_m[kRT], l_run[kRT], l_tot[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) mref[rt] = 0.f;
  const float cs = p.scale_log2;          // > 0
  const int vis_all_end = min(L, kend);  // keys below this are visible to every row

  // Per-lane LDS read offsets (elements) within a stage. K operand: key
  // 16t + l16 of the sub-block, chunk (4s + g) ^ swizzle. V^T operand: key
  // 16hh + 4g + l16/4 of the sub-block, d 16 dt + 4 (l16 % 4).
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = l16 * D + (((4 * s + g) ^ k_swz<D>(l16)) * 8);
  const int vkey = 4 * g + (l16 >> 2);
  int v_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    v_off[dt] = vkey * D + ((dt ^ v_swz<D>(vkey)) * 16) + 4 * (l16 & 3);

  // S^T for the 32 keys of sub-block sb of tile t: two MFMA tiles of 16
  // consecutive keys. Lane (g, l16) ends up with S for packed row l16 and
  // keys 16u + 4g + (0..3): the P^T B-operand k-slot 4u + e of lane group g
  // is key 16u + 4g + e.
  auto s_block = [&](int t, int sb, f32x4_t (&sacc)[2][kRT]) __attribute__((always_inline)) {
    const uint16_t* tK = sK + (t & (kRing - 1)) * TILE + 32 * sb * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u16x8_t*>(tK + 16 * u * D + k_off[s]));
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          sacc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, qf[rt][s], s == 0 ? f32x4_t(0.f) : sacc[u][rt], 0, 0, 0);
      }
    }
  };
  // Tail sub-blocks: keys a row may not see (tree block, past the chunk end)
  // become -inf.
  auto mask_block = [&](int skey0, f32x4_t (&sacc)[2][kRT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int node = node_rt[rt] < 0 ? 0 : node_rt[rt];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = skey0 + 16 * u + 4 * g + e;
          const int j = key - L;
          const uint32_t in_tree = static_cast<uint32_t>(j >= 0) &
                                   static_cast<uint32_t>(key < kend) &
                                   static_cast<uint32_t>(node_rt[rt] >= 0);
          const int jj = in_tree ? j : 0;
          const uint32_t w = sMask[node * p.W + (jj >> 5)];
          const uint32_t vis = static_cast<uint32_t>(key < vis_all_end) |
                               (in_tree & (w >> (jj & 31)));
          sacc[u][rt][e] = (vis & 1u) ? sacc[u][rt][e] : -INFINITY;
        }
    }
  };
  // Row reference from the first scores of the chunk (one cross-lane max).
  auto take_reference = [&](const f32x4_t (&sacc)[2][kRT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const float m = fmaxf(fmaxf(fmaxf(sacc[0][rt][0], sacc[0][rt][1]),
                                  fmaxf(sacc[0][rt][2], sacc[0][rt][3])),
                            fmaxf(fmaxf(sacc[1][rt][0], sacc[1][rt][1]),
                                  fmaxf(sacc[1][rt][2], sacc[1][rt][3])));
      // A row that sees none of these keys (a caller-built mask without
      // them) takes 0 as its reference: the reference stored with the
      // partial is always the one P was computed against.
      mref[rt] = finite_ref(row_max4(m) * cs);
      neg_m[rt] = -mref[rt];
    }
  };
  // P = 2^(s cs - mref) as bf16 parts (the MFMA B operand P^T). No running
  // max is kept: a score far above the reference shows up in the row sum.
  // One part: P rounded to nearest even. Two parts: hi = P rounded to
  // nearest, mid = P - hi (exact in fp32) rounded to nearest. Three parts
  // are cut by truncation, which is exact: hi = the top 16 bits of P (a
  // bf16 value), r1 = P - hi (exact in fp32, at most 16 significant bits),
  // mid = the top 16 bits of r1, lo = r1 - mid (exact, at most 8
  // significant bits, so a bf16 value); P = hi + mid + lo exactly, and two
  // entries go into one register with one byte permute.
  auto softmax_block = [&](const f32x4_t (&sacc)[2][kRT], bf16x8_t (&pb)[PARTS][kRT])
                           __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float y[8], pr[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * u + e] = fmaf(sacc[u][rt][e], cs, neg_m[rt]);
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(y[e]);
      l_run[rt] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      if constexpr (PARTS == 1) {
        bf16x8_t h1;
#pragma unroll
        for (int e = 0; e < 8; ++e) h1[e] = static_cast<__bf16>(pr[e]);
        pb[0][rt] = h1;
      } else {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        u32x4_t w0, w1, w2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = pr[2 * k], b = pr[2 * k + 1];
          if constexpr (PARTS == 2) {
            // Both parts rounded to nearest: P - hi - mid <= 2^-16 P.
            w0[k] = bf16_pair(a, b);
            const float ra = a - __uint_as_float(w0[k] << 16);
            const float rb = b - __uint_as_float(w0[k] & 0xFFFF0000u);
            w1[k] = bf16_pair(ra, rb);
          } else {
            w0[k] = high_halves(b, a);
            const float ra = a - __uint_as_float(__float_as_uint(a) & 0xFFFF0000u);
            const float rb = b - __uint_as_float(__float_as_uint(b) & 0xFFFF0000u);
            w1[k] = high_halves(rb, ra);
            const float sa = ra - __uint_as_float(__float_as_uint(ra) & 0xFFFF0000u);
            const float sb = rb - __uint_as_float(__float_as_uint(rb) & 0xFFFF0000u);
            w2[k] = high_halves(sb, sa);
          }
        }
        pb[0][rt] = __builtin_bit_cast(bf16x8_t, w0);
        pb[1][rt] = __builtin_bit_cast(bf16x8_t, w1);
        if constexpr (PARTS > 2) pb[2][rt] = __builtin_bit_cast(bf16x8_t, w2);
      }
    }
  };
  // O^T += V^T P^T over sub-block sb of tile t. The V^T A operand needs, in
  // lane (g, j), V[key of k-slot 4hh + kk][d0 + j]; within each group of 16
  // lanes the transposing read hands lane j element j%4 of the 8 bytes
  // fetched by lanes 4kk + j/4, so lane (g, L) fetches d d0 + 4(L%4) .. +3
  // of key 16hh + 4g + L/4 of the sub-block.
  auto pv_block = [&](int t, int sb, const bf16x8_t (&pb)[PARTS][kRT])
                      __attribute__((always_inline)) {
    const uint16_t* tV = sV + (t & (kRing - 1)) * TILE + 32 * sb * D;
    auto read_v = [&](int dt) __attribute__((always_inline)) {
      const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tV + v_off[dt]));
      const s16x4_t h1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tV + 16 * D + v_off[dt]));
      return __builtin_bit_cast(bf16x8_t,
                                __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // The operands of d-tile dt + 1 are requested before the MFMAs of dt
    // (pinned below), so each slice's LDS latency hides behind the previous
    // slice's MFMAs; consecutive MFMAs go to different accumulators.
    bf16x8_t a = read_v(0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x8_t an = a;
      if (dt + 1 < DT) an = read_v(dt + 1);
#pragma unroll
      for (int q = 0; q < PARTS; ++q)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[q][rt], o[dt][rt], 0, 0, 0);
      a = an;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // reads of d-tiles 0, 1
      else if (dt + 1 < DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // d-tile dt + 1
      __builtin_amdgcn_sched_group_barrier(0x008, PARTS * kRT, 0);  // MFMAs of d-tile dt
    }
  };

  // ---- passes over the chunk. The first takes each row's reference from
  // the chunk's first 32 keys. If some row's sum l exceeds 2^32 (or is not
  // finite), a score rose far above that reference (P <= l): then a
  // max-only pass finds the exact chunk max per row and a second pass runs
  // with it as reference, where every P <= 1.
  //
  // A pass walks the chunk in 32-key sub-blocks j. Each step issues the
  // S^T MFMAs of sub-block j and the P.V MFMAs of sub-block j - 1 (whose
  // probabilities the previous step produced), then computes the
  // probabilities of sub-block j on the VALU. A workgroup barrier after
  // every second step publishes the next 64-key tile: tile t (sub-blocks
  // 2t, 2t + 1) is published before the step that reads its first keys, and
  // right after that barrier tile t + 2 is requested into the ring stage of
  // tile t - 2, which every wave has finished. Two tiles are in flight
  // while one is computed: the wait before the barrier leaves tile t + 1's
  // copies outstanding (vector-memory operations complete in issue order
  // for the counter, and these copies are the only ones issued inside the
  // loop). One barrier per tile: finer-grained phase barriers (one wave
  // group feeding the matrix cores while the other runs the softmax) were
  // measured slower once the HBM->LDS copies stream underneath.
  auto lds_barrier_pinned = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Waits until tile t has landed, leaving tile t + 1's copies in flight.
  constexpr int kTileOps = 2 * LOADS;  // copies per thread per tile (K and V)
  auto wait_tile = [&](int t) __attribute__((always_inline)) {
    if (t + 1 < ntile)
      TV_WAIT_VMCNT(kTileOps);
    else
      TV_WAIT_VMCNT(0);
  };
  const int nsub = (kend - kbeg + 31) / 32;  // 32-key sub-blocks of the chunk
  // Mask (tail sub-blocks only), reference (first sub-block of the first
  // pass), probabilities.
  auto s_phase = [&](int j, f32x4_t (&sacc)[2][kRT], bf16x8_t (&pb)[PARTS][kRT], bool need_ref)
                     __attribute__((always_inline)) {
    const int skey0 = kbeg + 32 * j;
    if (skey0 + 32 > vis_all_end) mask_block(skey0, sacc);
    if (need_ref) take_reference(sacc);
    softmax_block(sacc, pb);
  };
  auto run_pass = [&](const int attempt) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) o[dt][rt] = f32x4_t(0.f);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      l_run[rt] = 0.f;
      neg_m[rt] = -mref[rt];
    }
    if (tid == 0) sOvf = 0;
    issue_tile(0);
    if (ntile > 1) issue_tile(1);
    wait_tile(0);
    lds_barrier_pinned();  // tile 0 published
    if (ntile > 2) issue_tile(2);
    f32x4_t sacc[2][kRT];
    bf16x8_t pb[PARTS][kRT];
    bool need_ref = (attempt == 0);
#pragma unroll 1
    for (int j = 0; j <= nsub; ++j) {
      if (wave_active) {
        if (j < nsub) s_block(j >> 1, j & 1, sacc);
        if (j >= 1) pv_block((j - 1) >> 1, (j - 1) & 1, pb);
        if (j < nsub) s_phase(j, sacc, pb, need_ref);
      }
      need_ref = false;
      if (j & 1) {
        const int t = (j + 1) >> 1;  // the next tile
        if (t < ntile) {
          wait_tile(t);
          lds_barrier_pinned();
          if (t + 2 < ntile) issue_tile(t + 2);
        }
      }
    }
    // ---- end of pass: row sums and the runaway test (live rows only; a
    // sum below 2^-32 can only come from the zero reference of a row that
    // saw none of the unit's first keys) ----
    bool ovf = false;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      l_tot[rt] = row_sum4(l_run[rt]);
      ovf |= node_rt[rt] >= 0 && !(l_tot[rt] <= kRowSumLimit && l_tot[rt] >= kRowSumFloor);
    }
    if (wave_active && __any(ovf) && lane == 0) sOvf = 1;
    TV_WAIT_VMCNT(0);
    lds_barrier();
    const int again = sOvf;
    lds_barrier();
    return again;
  };
  // The common case is a single pass; the retry is a separate copy of the
  // pass (no loop around it), so the first pass's code and registers are
  // not shaped by a loop-carried second attempt.
  // Exact max of the visible scores of every row over the whole chunk.
  auto max_pass = [&]() {
    float lm[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) lm[rt] = -INFINITY;
    issue_tile(0);
    if (ntile > 1) issue_tile(1);
#pragma unroll 1
    for (int t = 0; t < ntile; ++t) {
      enter_tile(t);
#pragma unroll
      for (int sbk = 0; sbk < 2; ++sbk) {
        const int skey0 = kbeg + t * kKB + 32 * sbk;
        if (skey0 < kend) {
          f32x4_t sacc[2][kRT];
          s_block(t, sbk, sacc);
          if (skey0 + 32 > vis_all_end) mask_block(skey0, sacc);
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int e = 0; e < 4; ++e) lm[rt] = fmaxf(lm[rt], sacc[u][rt][e]);
        }
      }
    }
    TV_WAIT_VMCNT(0);
    lds_barrier();
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) mref[rt] = finite_ref(row_max4(lm[rt]) * cs);
  };
  if (run_pass(0)) {
    max_pass();
    run_pass(1);
  }

  // ---- epilogue ----
  if (!wave_active) return;
  const bool direct = (pc.np == 1);
  // With one probability part the unit partials are stored as 16-bit fixed
  // point against the row's largest |O| (error at most that / 65534 per
  // entry, i.e. max|v| / 65534 after normalisation); more parts keep fp32.
  constexpr bool kQ16 = (PARTS == 1);
  float amax[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float a = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a = fmaxf(a, fabsf(o[dt][rt][e]));
    amax[rt] = (kQ16 && !direct) ? row_max4(a) : 0.f;
  }
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int r = row0 + rt * 16 + l16;
    if (r >= p.R) continue;
    if (direct) {
      const bool live = node_rt[rt] >= 0;
      if (PACKED && !live) continue;  // packed: rows past n do not exist
      const int i = row_node(p, r);
      const int h = kvh * p.G + (r - i * p.G);
      const int64_t orow = (srow0 + i) * p.Hq + h;
      // A live row that saw no key at all (only possible with a caller-built
      // mask and no committed context) gets the padding values.
      const bool seen = live && l_tot[rt] > 0.f;
      const float inv = seen ? 1.f / l_tot[rt] : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t v = o[dt][rt] * inv;
        store_out4(p, orow * D + 16 * dt + 4 * g, v[0], v[1], v[2], v[3]);
      }
      if (g == 0) p.lse[orow] = seen ? (mref[rt] + __log2f(l_tot[rt])) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = static_cast<int64_t>(pc.slot) * p.rows_wg + (r - rg * kRowsWG);
      if constexpr (kQ16) {
        // Row layout [g][dt][e] (the lane's 4 DT entries contiguous: 16-byte
        // stores); entry (g, dt, e) is d = 16 dt + 4 g + e.
        int16_t* dst = reinterpret_cast<int16_t*>(p.part_o) + prow * D + g * (4 * DT);
        const float qs = amax[rt] > 0.f ? 32767.f / amax[rt] : 0.f;
        auto pack2 = [&](float a, float c) __attribute__((always_inline)) {
          return static_cast<uint32_t>(static_cast<uint16_t>(__float2int_rn(a * qs))) |
                 (static_cast<uint32_t>(static_cast<uint16_t>(__float2int_rn(c * qs))) << 16);
        };
#pragma unroll
        for (int dp = 0; dp < DT / 2; ++dp) {
          const f32x4_t v0 = o[2 * dp][rt];
          const f32x4_t v1 = o[2 * dp + 1][rt];
          // Plain stores here: written through at device scope, these
          // 16-byte pieces of a half-size row doubled the counted writes.
          *reinterpret_cast<uint4*>(dst + 8 * dp) =
              make_uint4(pack2(v0[0], v0[1]), pack2(v0[2], v0[3]), pack2(v1[0], v1[1]),
                         pack2(v1[2], v1[3]));
        }
      } else {
        float* dst = p.part_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          store_wt16(dst + 16 * dt + 4 * g, o[dt][rt]);
        }
      }
      if (g == 0)
        p.part_ml[static_cast<int64_t>(pc.base) * p.rows_wg + (r - rg * kRowsWG) * pc.np + pc.j] =
            make_float4(mref[rt], l_tot[rt], amax[rt], 0.f);
    }
  }
  };

  // Padding outputs first: their stores drain while the first tiles load.
  finish_non_live<D, kThreads>(p, st0, n0, s0);
  for_each_piece(p, len0, K, sk, stream_k, run_unit);
}

// ---------------------------------------------------------- fp32 (VALU) ---
// fp32 inputs are kept fp32 end to end (a bf16 round trip of the inputs
// alone would move the log-sum-exp by ~1e-3). Four lanes share a packed row,
// each holding a quarter of D; keys are staged through LDS 32 at a time.

template <int D, bool PACKED>
__global__ __launch_bounds__(kThreadsF32) void attn_split_f32_kernel(AttnParamsT<PACKED> p) {
  constexpr int DQ = D / 4;
  constexpr int D4 = D / 4;  // float4 per key row
  __shared__ __attribute__((aligned(16))) float sK[kKBf32 * D];
  __shared__ __attribute__((aligned(16))) float sV[kKBf32 * D];
  __shared__ uint32_t sMask[TV_MAX_TREE * (TV_MAX_TREE / 32)];

  const int tid = threadIdx.x;
  int n0, s0, st0;
  const int len0 = lane_len(p, n0, s0, st0);
  bool stream_k;
  const int K = choose_unit(p, len0, stream_k);
  SkLine sk{0, 0, 0, 0};
  if (stream_k) sk = sk_line(p, len0);
  if (p.sched && blockIdx.x == 0 && tid < tv::kWave) write_sched(p, len0, K, sk, stream_k);

  auto run_unit = [&](const Piece& pc) __attribute__((always_inline)) {
  const int b = pc.b, kvh = pc.kvh, rg = pc.rg;
  int n, L;
  int64_t srow0;  // output row of tree row 0
  unit_seq(p, b, len0, n0, s0, n, L, srow0);
  const bool last = pc.last;
  const int kbeg = pc.kbeg;
  const int kend = last ? L + n : pc.kcut;
  if (last) {
    const uint32_t* mrow = p.mask + static_cast<int64_t>(b) * p.T * p.W;
    for (int idx = tid; idx < n * p.W; idx += kThreadsF32) sMask[idx] = mrow[idx];
  }

  const float* kbase = static_cast<const float*>(p.k) + b * p.kv_sb + kvh * p.kv_sh;
  const float* vbase = static_cast<const float*>(p.v) + b * p.kv_sb + kvh * p.kv_sh;

  const int quarter = tid & 3;
  const int r = rg * kRowsWGf32 + (tid >> 2);
  int node = -1;
  int h = 0;
  if (r < p.R) {
    const int i = row_node(p, r);
    h = kvh * p.G + (r - i * p.G);
    if (i < n) node = i;
  }
  float qv[DQ];
  float ov[DQ];
  if (node >= 0) {
    const float* qrow = static_cast<const float*>(p.q) +
                        (PACKED ? srow0 * p.q_st : b * p.q_sb) + node * p.q_st + h * p.q_sh;
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
    for (int idx = tid; idx < kKBf32 * D4; idx += kThreadsF32) {
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
  const int i = row_node(p, r);
  if (pc.np == 1) {
    const bool live = node >= 0;
    if (PACKED && !live) return;  // packed: rows past n do not exist
    const int64_t orow = (srow0 + i) * p.Hq + h;
    const bool seen = live && l_run > 0.f;  // a live row that saw no key: padding values
    const float inv = seen ? 1.f / l_run : 0.f;
#pragma unroll
    for (int d = 0; d < DQ; d += 4)
      store_out4(p, orow * D + quarter * DQ + d, ov[d] * inv, ov[d + 1] * inv, ov[d + 2] * inv,
                 ov[d + 3] * inv);
    if (quarter == 0) p.lse[orow] = seen ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t prow = static_cast<int64_t>(pc.slot) * p.rows_wg + (r - rg * kRowsWGf32);
#pragma unroll
    for (int d = 0; d < DQ; ++d) p.part_o[prow * D + quarter * DQ + d] = ov[d];
    if (quarter == 0)
      p.part_ml[static_cast<int64_t>(pc.base) * p.rows_wg + (r - rg * kRowsWGf32) * pc.np + pc.j] =
          make_float4(m_run, l_run, 0.f, 0.f);
  }
  };

  // Padding outputs first: their stores drain while the first tiles load.
  finish_non_live<D, kThreadsF32>(p, st0, n0, s0);
  for_each_piece(p, len0, K, sk, stream_k, run_unit);
}

// ----------------------------------------------------- log-sum-exp merge ---
// Merges the unit partials of pairs with more than one unit:
// m* = max m_c, l* = sum l_c 2^(m_c - m*), O = sum O_c 2^(m_c - m*) / l*,
// lse = (m* + log2 l*) ln 2. The (m, l, scale) of a row's units are
// contiguous (the split kernel writes them as [row][unit] per pair); lane k
// of the row reads unit k's, the row max and the weighted sum of l are lane
// reductions, and each unit's weight is broadcast to the row's lanes by a
// shuffle. A lane holds eight entries of the row (one 16-byte load per unit)
// with 16-bit partials, four with fp32 ones. Up to 16 units per round are
// requested at once. Q16: the partial rows are int16 fixed point,
// entry = q * scale / 32767.

// Entries of a packed row per combine lane: eight 16-bit partials (one
// 16-byte load per unit), or four fp32 ones.
template <bool Q16>
constexpr int combine_epl() {
  return Q16 ? 8 : 4;
}
template <int D, bool Q16>
constexpr int combine_rows_per_block() {
  return kThreadsCombine / (D / combine_epl<Q16>());
}

// op-reduction over the LPR (8, 16, 32 or 64) lanes of an aligned lane
// group, in every lane of the group: DPP steps within groups of 8 and rows of
// 16, then the row-pair and half-wave swaps (vector ALU only; __shfl_xor
// would be an LDS round trip per step).
template <int LPR, class Op>
__device__ __forceinline__ float row_reduce(float x, Op op) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "lane groups of 8 to 64");
  auto dpp = [](float v, auto ctrl) __attribute__((always_inline)) {
    return __int_as_float(tv::dpp_i32<decltype(ctrl)::value>(__float_as_int(v)));
  };
  x = op(x, dpp(x, std::integral_constant<int, tv::kDppXor1>()));
  x = op(x, dpp(x, std::integral_constant<int, tv::kDppXor2>()));
  x = op(x, dpp(x, std::integral_constant<int, tv::kDppHalfMirror>()));
  if constexpr (LPR >= 16) x = op(x, dpp(x, std::integral_constant<int, tv::kDppRowRor8>()));
  if constexpr (LPR >= 32) {
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
    x = op(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  }
  if constexpr (LPR == 64) {
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
    x = op(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
  }
  return x;
}

template <int D, bool Q16, bool PACKED>
__global__ __launch_bounds__(kThreadsCombine) void attn_combine_kernel(AttnParamsT<PACKED> p) {
  constexpr int EPL = combine_epl<Q16>();                        // entries per lane
  constexpr int LPR = D / EPL;                                   // lanes per packed row
  constexpr int RPB = combine_rows_per_block<D, Q16>();          // packed rows per block
  constexpr int U = 16;                                          // units per round
  constexpr int MPL = U > LPR ? U / LPR : 1;                     // unit records per lane
  const int bk = blockIdx.y;
  const int b = bk / p.Hkv;
  const int kvh = bk - b * p.Hkv;
  const int sub = threadIdx.x & (LPR - 1);
  const int r = blockIdx.x * RPB + threadIdx.x / LPR;
  // Every scalar input in one round trip.
  const int n = p.n_nodes[b];
  const int L = p.ctx_len[b];
  const int t0 = p.sched[0];
  const int t1 = p.sched[1];
  const int t_off = p.sched[2];
  const int t_p0 = p.sched[3];
  const int t2 = p.sched[4 + 2 * b];
  const int t3 = p.sched[5 + 2 * b];
  const int start = PACKED ? p.row_start[b] : 0;
  // Keeps the loads ahead of the branches below (the compiler would
  // otherwise sink each one into the branch that first needs it and wait
  // for them one by one).
  asm volatile("" ::"s"(n), "s"(L), "s"(t0), "s"(t1), "s"(t_off), "s"(t_p0), "s"(t2), "s"(t3),
               "s"(start));
  if (r >= p.R) return;
  if (seq_status(p, n, L, start) != TV_ROW_OK) return;  // padded / invalid: done by the split
  const int rg = r / p.rows_wg;
  const int rl = r - rg * p.rows_wg;
  const int q = kvh * p.RG + rg;
  // The pair's pieces: first slot u0, count nch; pieces jt .. nch - 2 hold
  // no keys (stream-K only) and are skipped.
  int nch, u0, jt;
  if (t1 < 0) {  // unit mode: K = t0, first unit of the sequence = t2
    nch = pair_units(p, L, t0);
    u0 = t2 + q * nch;
    jt = nch;
  } else if (t3 + q < t_p0) {  // stream-K, a whole-pair unit
    nch = 1;
    u0 = jt = 0;
  } else {  // stream-K, shared part: line tiles and pairs before the sequence = t2, t3
    const int wp = pair_tiles(L);
    const SkPair pr =
        sk_pair(SkLine{t0, t1, t_off, t_p0}, t2 + q * wp - t_off, wp, t3 + q - t_p0);
    nch = pr.np;
    u0 = pr.base;
    jt = pr.jt;
  }
  if (nch == 1) return;  // written directly by the split
  const int i = row_node(p, r);
  const int h = kvh * p.G + (r - i * p.G);
  if (i >= n && PACKED) return;  // packed: rows past n do not exist
  const int64_t orow = (seq_row0(p, b, start) + i) * p.Hq + h;
  // Output entries of this lane, four per float4: with 16-bit partials the
  // lane's eight entries are (g, dt = 2 dp and 2 dp + 1, e) of the split's
  // row layout [g][dt][e], i.e. d = 16 dt + 4 g + e; fp32 partials are in
  // plain d order.
  int64_t dst[EPL / 4];  // entry offsets in out
  if constexpr (Q16) {
    constexpr int HALF = D / 32;  // dt pairs per g
    const int g = sub / HALF;
    const int dp = sub - g * HALF;
    dst[0] = orow * D + 32 * dp + 4 * g;
    dst[1] = orow * D + 32 * dp + 16 + 4 * g;
  } else {
    dst[0] = orow * D + EPL * sub;
  }
  if (i >= n) {
#pragma unroll
    for (int e = 0; e < EPL / 4; ++e) store_out4(p, dst[e], 0.f, 0.f, 0.f, 0.f);
    if (sub == 0) p.lse[orow] = -INFINITY;
    return;
  }
  const int64_t row_elem =
      (static_cast<int64_t>(u0) * p.rows_wg + rl) * D + EPL * sub;  // entry offset of piece 0
  const int64_t ustride = static_cast<int64_t>(p.rows_wg) * D;      // entries between pieces
  const float4* pml = p.part_ml + static_cast<int64_t>(u0) * p.rows_wg +
                      static_cast<int64_t>(rl) * nch;
  // Piece k holds keys: its record and partial row are read; an empty piece
  // reads the last one (which always holds the tree block) with weight 0.
  auto held = [&](int k) { return k < nch && (k < jt || k == nch - 1); };
  float mstar = -INFINITY, lstar = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += U) {
    // Lane k of the row loads the (m, l, scale) of unit c0 + k (and of
    // c0 + k + LPR ... when a round has more units than the row has lanes)
    // and computes its weight; the weights reach the other lanes by
    // shuffles. The partial rows of the round's pieces that hold keys are
    // requested together; the others count as zero rows with weight 0.
    float4 mine[MPL];
    bool valid[MPL];
#pragma unroll
    for (int j = 0; j < MPL; ++j) {
      const int kl = sub + j * LPR;
      valid[j] = kl < U && held(c0 + kl);
      mine[j] = pml[valid[j] ? c0 + kl : nch - 1];
    }
    using Raw = typename std::conditional<Q16, uint4, float4>::type;
    Raw v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t off = row_elem + (c0 + k) * ustride;
      v[k] = Raw{};
      if (held(c0 + k)) {
        if constexpr (Q16)
          v[k] = *reinterpret_cast<const uint4*>(reinterpret_cast<const int16_t*>(p.part_o) + off);
        else
          v[k] = *reinterpret_cast<const float4*>(p.part_o + off);
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MPL; ++j) m = fmaxf(m, valid[j] ? mine[j].x : -INFINITY);
    m = row_reduce<LPR>(m, [](float a, float b) { return fmaxf(a, b); });
    m = fmaxf(m, mstar);  // units with finite m only (a live row's reference always is)
    const float sc = mstar == -INFINITY ? 0.f : exp2f(mstar - m);
    float wo[MPL];
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < MPL; ++j) {
      const float wk = valid[j] ? exp2f(mine[j].x - m) : 0.f;
      ls = fmaf(mine[j].y, wk, ls);
      wo[j] = Q16 ? wk * (mine[j].z * (1.f / 32767.f)) : wk;
    }
    ls = row_reduce<LPR>(ls, [](float a, float b) { return a + b; });
    lstar = fmaf(lstar, sc, ls);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= sc;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float w = __shfl(wo[k / LPR], k % LPR, LPR);
      float x[EPL];
      if constexpr (Q16) {
        const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = static_cast<float>(static_cast<int16_t>(q[e] & 0xFFFFu));
          x[2 * e + 1] = static_cast<float>(static_cast<int16_t>(q[e] >> 16));
        }
      } else {
        x[0] = v[k].x;
        x[1] = v[k].y;
        x[2] = v[k].z;
        x[3] = v[k].w;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(x[e], w, acc[e]);
    }
    mstar = m;
  }
  const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
#pragma unroll
  for (int e = 0; e < EPL / 4; ++e)
    store_out4(p, dst[e], acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv,
               acc[4 * e + 3] * inv);
  if (sub == 0) p.lse[orow] = lstar > 0.f ? (mstar + __log2f(lstar)) * kLn2 : -INFINITY;
}

// Workgroups per launch: one per compute unit (a multiple of 8).
int grid_workgroups() { return tvh::grid_workgroups(); }

int host_chunks(int64_t L, int64_t K) { return L == 0 ? 1 : static_cast<int>((L + K - 1) / K); }

// Tiles on the stream-K line when every sequence is live with max_ctx
// committed keys, for the given packed rows per workgroup.
int64_t line_tiles(int B, int T, int Hq, int Hkv, int max_ctx, int rows_wg) {
  const int64_t R = static_cast<int64_t>(Hq / Hkv) * T;
  const int64_t pairs = static_cast<int64_t>(B) * Hkv * ((R + rows_wg - 1) / rows_wg);
  return pairs * ((static_cast<int64_t>(max_ctx) + kKB - 1) / kKB + kTreeTiles);
}

// The unit size the device picks when every sequence is live with max_ctx
// committed keys (bf16 row groups): the smallest multiple of 64, at least
// kMinUnit, that gives at most one unit per workgroup.
int auto_chunk(int B, int T, int Hq, int Hkv, int max_ctx) {
  const int64_t R = static_cast<int64_t>(Hq / Hkv) * T;
  const int64_t pairs = static_cast<int64_t>(B) * Hkv * ((R + kRowsWG - 1) / kRowsWG);
  const int64_t nw = grid_workgroups();
  // Units per pair as the device counts them: the tree block weighs
  // min(kTreeExtra, K / 2) committed keys.
  auto units = [&](int K) {
    return max_ctx == 0 ? pairs
                        : pairs * ((max_ctx + std::min(kTreeExtra, K / 2) + K - 1) / K);
  };
  int lo = kMinUnit;
  int hi = std::max(kMinUnit, (max_ctx + kTreeExtra + 63) / 64 * 64);
  if (units(lo) <= nw) return lo;
  if (units(hi) > nw) return hi;
  while (hi - lo > 64) {
    const int mid = (lo / 64 + hi / 64) / 2 * 64;
    if (units(mid) <= nw)
      hi = mid;
    else
      lo = mid;
  }
  return hi;
}

bool valid_sizes(int B, int T, int Hq, int Hkv, int D, int max_ctx, int chunk_keys) {
  if (B < 0 || T < 1 || T > TV_MAX_TREE || Hq < 1 || Hkv < 1 || Hq % Hkv) return false;
  if (Hq / Hkv > TV_MAX_GROUP || max_ctx < 0) return false;
  if (chunk_keys != 0 && (chunk_keys < 64 || chunk_keys > 65536 || chunk_keys % 64)) return false;
  (void)D;
  return true;
}

// Workspace layout: the schedule table ((4 + 2 B) int32), then partial O
// [slot][rows_wg][D] (fp32, or int16 fixed point in the same space, each
// row in the split lanes' order), then (m, l, scale, 0) per pair as
// [rows_wg][piece of the pair] from the pair's first slot. Fixed chunks use
// one slot per unit; the balanced (stream-K) partition at most pairs + nw.
// Sized for the larger of the bf16 (256 rows per workgroup) and fp32 (64)
// kernels. No workspace when every pair is a single unit (written directly):
// max_ctx <= chunk_keys, or max_ctx + kTreeExtra <= kMinUnit when balanced
// (the kernels then take one unit per pair).
struct WsLayout {
  size_t sched = 0, part_o = 0, part_ml = 0, total = 0;
};

WsLayout workspace_layout(int B, int T, int Hq, int Hkv, int D, int max_ctx, int chunk_keys) {
  WsLayout w;
  const int64_t R = static_cast<int64_t>(Hq / Hkv) * T;
  const int64_t nw = grid_workgroups();
  int64_t rows_max = 0;
  for (const int rows_wg : {kRowsWG, kRowsWGf32}) {
    const int64_t pairs = static_cast<int64_t>(B) * Hkv * ((R + rows_wg - 1) / rows_wg);
    int64_t units = 0;
    if (chunk_keys > 0) {
      const int64_t nch = host_chunks(max_ctx, chunk_keys);
      units = nch > 1 ? pairs * nch : 0;
    } else {
      units = max_ctx + kTreeExtra > kMinUnit ? pairs + nw : 0;
    }
    rows_max = std::max(rows_max, units * rows_wg);
  }
  if (rows_max == 0) return w;
  w.sched = 0;
  w.part_o = tvh::align_up(static_cast<size_t>(4 + 2 * static_cast<int64_t>(B)) * sizeof(int32_t), 256);
  w.part_ml = w.part_o + tvh::align_up(static_cast<size_t>(rows_max) * D * sizeof(float), 256);
  w.total = w.part_ml + tvh::align_up(static_cast<size_t>(rows_max) * sizeof(float4), 256);
  return w;
}

template <int D, bool PACKED>
void launch_all(const AttnParams& p0, int in_dtype, bool combine, hipStream_t stream) {
  AttnParamsT<PACKED> p;
  static_cast<AttnParams&>(p) = p0;
  const dim3 grid(p.nw);
  if (in_dtype == TV_BF16) {
    if (p.parts == 1)
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 1, PACKED>), grid, dim3(kThreads), 0, stream, p);
    else if (p.parts == 2)
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 2, PACKED>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_split_bf16_kernel<D, 3, PACKED>), grid, dim3(kThreads), 0, stream, p);
  } else
    hipLaunchKernelGGL((attn_split_f32_kernel<D, PACKED>), grid, dim3(kThreadsF32), 0, stream, p);
  if (combine) {
    if (in_dtype == TV_BF16 && p.parts == 1) {
      constexpr int rpb = combine_rows_per_block<D, true>();
      hipLaunchKernelGGL((attn_combine_kernel<D, true, PACKED>),
                         dim3((p.R + rpb - 1) / rpb, p.B * p.Hkv), dim3(kThreadsCombine), 0,
                         stream, p);
    } else {
      constexpr int rpb = combine_rows_per_block<D, false>();
      hipLaunchKernelGGL((attn_combine_kernel<D, false, PACKED>),
                         dim3((p.R + rpb - 1) / rpb, p.B * p.Hkv), dim3(kThreadsCombine), 0,
                         stream, p);
    }
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
  return workspace_layout(B, T, Hq, Hkv, D, max_ctx, chunk_keys).total;
}

namespace {

// Both layouts: row_start == nullptr is the padded [B][T] layout.
int attention_call(const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh, const void* k,
                   const void* v, int64_t kv_sb, int64_t kv_sh, int64_t kv_ss,
                   const int32_t* ctx_len, const int32_t* n_nodes, const uint32_t* mask,
                   const int32_t* row_start, int rows_total, int B, int T, int Hq, int Hkv, int D,
                   int max_ctx, int kv_capacity, float scale, int in_dtype, int out_dtype,
                   int probability_parts, int chunk_keys, void* out, float* lse, void* workspace,
                   size_t ws_bytes, int32_t* row_status, hipStream_t stream) {
  if (!q || !k || !v || !ctx_len || !n_nodes || !mask || !out || !lse || !row_status)
    return TV_ERR_NULL;
  if (in_dtype != TV_F32 && in_dtype != TV_BF16) return TV_ERR_DTYPE;
  if (out_dtype != TV_F32 && out_dtype != TV_BF16) return TV_ERR_DTYPE;
  if (!valid_sizes(B, T, Hq, Hkv, D, max_ctx, chunk_keys) || kv_capacity < 1)
    return TV_ERR_SHAPE;
  if (probability_parts < 1 || probability_parts > 3) return TV_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < INFINITY)) return TV_ERR_SHAPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  const int64_t elem_align = in_dtype == TV_BF16 ? 8 : 4;  // 16 bytes
  if (!tvh::aligned16(q) || !tvh::aligned16(k) || !tvh::aligned16(v) || !tvh::aligned16(out) ||
      !tvh::aligned16(lse))
    return TV_ERR_ALIGN;
  if (q_sb % elem_align || q_st % elem_align || q_sh % elem_align || kv_sb % elem_align ||
      kv_sh % elem_align || kv_ss % elem_align)
    return TV_ERR_ALIGN;
  if (kv_ss < 0 || static_cast<int64_t>(kv_capacity) * kv_ss + D > INT32_MAX) return TV_ERR_SHAPE;
  if (B == 0) return TV_OK;
  if (static_cast<int64_t>(B) * Hkv > 65535) return TV_ERR_SHAPE;
  // The stream-K line is indexed with 32-bit tiles.
  if (line_tiles(B, T, Hq, Hkv, max_ctx, kRowsWGf32) >= INT32_MAX) return TV_ERR_SHAPE;
  const WsLayout ws = workspace_layout(B, T, Hq, Hkv, D, max_ctx, chunk_keys);
  if (ws.total > 0 && (!workspace || ws_bytes < ws.total || !tvh::aligned256(workspace)))
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
  p.row_start = row_start;
  p.rows_total = rows_total;
  p.B = B;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.g_mul = (65536u + static_cast<uint32_t>(p.G) - 1u) / static_cast<uint32_t>(p.G);
  p.R = p.G * T;
  p.W = (T + 31) / 32;
  p.max_ctx = max_ctx;
  p.kv_capacity = kv_capacity;
  p.parts = probability_parts;
  p.kunit = chunk_keys;
  p.rows_wg = in_dtype == TV_BF16 ? kRowsWG : kRowsWGf32;
  p.RG = (p.R + p.rows_wg - 1) / p.rows_wg;
  p.nw = grid_workgroups();
  p.scale_log2 = scale * kLog2e;
  p.out = out;
  p.out_bf16 = out_dtype == TV_BF16;
  p.lse = lse;
  p.sched = nullptr;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (ws.total > 0) {
    char* base = static_cast<char*>(workspace);
    p.sched = reinterpret_cast<int32_t*>(base + ws.sched);
    p.part_o = reinterpret_cast<float*>(base + ws.part_o);
    p.part_ml = reinterpret_cast<float4*>(base + ws.part_ml);
  }
  p.row_status = row_status;
  const bool combine = ws.total > 0;
  if (D == 128)
    row_start ? launch_all<128, true>(p, in_dtype, combine, stream)
              : launch_all<128, false>(p, in_dtype, combine, stream);
  else
    row_start ? launch_all<64, true>(p, in_dtype, combine, stream)
              : launch_all<64, false>(p, in_dtype, combine, stream);
  return tvh::launch_status();
}

}  // namespace

extern "C" int tv_tree_attention(const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                                 const void* k, const void* v, int64_t kv_sb, int64_t kv_sh,
                                 int64_t kv_ss, const int32_t* ctx_len, const int32_t* n_nodes,
                                 const uint32_t* mask, int B, int T, int Hq, int Hkv, int D,
                                 int max_ctx, int kv_capacity, float scale, int in_dtype,
                                 int out_dtype, int probability_parts, int chunk_keys, void* out,
                                 float* lse, void* workspace, size_t ws_bytes,
                                 int32_t* row_status, hipStream_t stream) {
  return attention_call(q, q_sb, q_st, q_sh, k, v, kv_sb, kv_sh, kv_ss, ctx_len, n_nodes, mask,
                        nullptr, 0, B, T, Hq, Hkv, D, max_ctx, kv_capacity, scale, in_dtype,
                        out_dtype, probability_parts, chunk_keys, out, lse, workspace, ws_bytes,
                        row_status, stream);
}

extern "C" int tv_tree_attention_packed(const void* q, int64_t q_st, int64_t q_sh, const void* k,
                                        const void* v, int64_t kv_sb, int64_t kv_sh,
                                        int64_t kv_ss, const int32_t* ctx_len,
                                        const int32_t* n_nodes, const uint32_t* mask,
                                        const int32_t* row_start, int rows_total, int B, int T,
                                        int Hq, int Hkv, int D, int max_ctx, int kv_capacity,
                                        float scale, int in_dtype, int out_dtype,
                                        int probability_parts, int chunk_keys, void* out,
                                        float* lse, void* workspace, size_t ws_bytes,
                                        int32_t* row_status, hipStream_t stream) {
  if (!row_start) return TV_ERR_NULL;
  if (rows_total < 0) return TV_ERR_SHAPE;
  return attention_call(q, 0, q_st, q_sh, k, v, kv_sb, kv_sh, kv_ss, ctx_len, n_nodes, mask,
                        row_start, rows_total, B, T, Hq, Hkv, D, max_ctx, kv_capacity, scale,
                        in_dtype, out_dtype, probability_parts, chunk_keys, out, lse, workspace,
                        ws_bytes, row_status, stream);
}
