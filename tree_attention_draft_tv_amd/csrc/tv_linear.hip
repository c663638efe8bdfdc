// Few-row projections of the verification rows, batch-invariant.
//
// Page: EmbodiInfer "perf(activevln): grammar-trie speculation and lossless
// throughput", commit "perf(activevln): batch-invariant Triton GEMMs for
// decode projections": tree verification runs every linear layer on a few
// dozen to a few hundred rows; the projections accumulate in FP32 in
// sequential K order with no split-K, so a row's result depends neither on
// the tiles nor on the row count and differs from the vendor GEMM only by
// output rounding. Q, K and V share one launch (one weight matrix holding
// the three, one output row per input row); gate and up share one launch
// with the rounded SwiGLU in the epilogue.
//
// MI355X: y^T = W x^T on v_mfma_f32_16x16x32_bf16, so that each lane ends
// with four consecutive output features of one row (one 8-byte store). A
// workgroup (4 waves) owns ROWS rows x 64 output features; wave w the
// features [16 w, 16 w + 16) of all ROWS rows (ROWS / 16 accumulator tiles,
// twice that with SwiGLU). Every output element is one accumulator chain over
// k = 0, 32, 64, ... in order, whatever the tile, the chunk depth and the row
// count (the variants give the same bits; tested). K is walked in chunks of
// KC: the input rows of a chunk are loaded into registers NST - 1 chunks
// ahead and written to a two-stage LDS ring shared by the four waves one
// chunk ahead; each wave's weight rows go straight to registers, also
// NST - 1 chunks ahead. Loads are plain (in-order) vector loads, so the
// compiler's partial waits keep those chunks in flight; the barrier that
// closes a chunk waits for LDS operations only (a full __syncthreads would
// also wait for every load in flight and serialise the chunks). Workgroups
// are numbered so that the row groups of one weight slice run on the same
// XCD and share its L2.
#include "tv_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLinFeat = 64;    // N granularity of the arguments (16 features per wave)
constexpr int kLinKC = 64;      // K granularity of the arguments (two MFMA k-steps)
// Rows per workgroup: 96 keeps a 264-row batch (three row groups) at 216
// workgroups for the QKV shape, one per compute unit; with 64 rows the 360
// workgroups put two on 104 units and take 1.6x as long (measured). Chunk
// depth and register stages were measured per kernel: 64-deep chunks for the
// plain projection, 128-deep for gate/up where K allows.
constexpr int kRows = 96;
constexpr int kDeepKC = 128;
constexpr int kWavesWide = 8;

struct LinParams {
  const uint16_t* x;
  const uint16_t* w0;  // weights, or the gate weights
  const uint16_t* w1;  // the up weights (SwiGLU only)
  int64_t x_stride, w_stride, y_stride;
  int M, K, N;
  int mgroups, work;
  uint16_t* y;
};

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(p));
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// Workgroup barrier for the LDS ring: this wave's LDS operations complete
// (lgkmcnt(0)), then s_barrier; global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS layout of an input chunk of KC k: 64 rows of P = KC / 8 16-byte
// pieces; piece c of row r sits at piece c ^ (r & (P - 1)), so the 16 rows an
// MFMA operand read touches at one k-offset spread over the banks.
template <int P>
__device__ __forceinline__ int x_slot(int row, int piece) {
  return row * P + (piece ^ (row & (P - 1)));
}

// NST register stages: chunk c + NST - 1 is requested while chunk c is
// computed. Input rows go registers -> LDS one chunk ahead (two LDS stages
// suffice: the barrier closing every chunk keeps all waves on the same chunk,
// which reads stage c % 2 while stage (c + 1) % 2 is written).
template <bool SWIGLU, int NST, int KC, int ROWS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void linear_rows_kernel(LinParams p) {
  constexpr int THREADS = 64 * WAVES;
  constexpr int FEAT = 16 * WAVES;              // output features per workgroup
  constexpr int P = KC / 8;                     // 16-byte pieces per row of a chunk
  constexpr int XL = ROWS * P / THREADS;        // input pieces per thread per chunk
  constexpr int KS = KC / 32;                   // MFMA k-steps per chunk
  constexpr int MT = ROWS / 16;                 // row tiles per wave
  static_assert(ROWS * P % THREADS == 0, "staging must divide evenly");
  __shared__ __attribute__((aligned(16))) u16x8_t sX[2][ROWS * P];
  // Work item -> (weight slice, row group): the workgroups sharing
  // blockIdx mod 8 (one XCD) take one contiguous run of work items, and the
  // row groups of a slice are consecutive work items.
  const int per_xcd = gridDim.x >> 3;
  const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (work >= p.work) return;
  const int slice = work / p.mgroups;
  const int mg = work - slice * p.mgroups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int n0 = slice * FEAT + wave * 16;
  const int m0 = mg * ROWS;
  const int nchunks = p.K / KC;

  // Staging: thread t loads pieces t, t + 256, ... of a chunk (row = s / P,
  // piece = s % P); rows past M re-read row M - 1.
  const uint16_t* xs[XL];
  int xslot[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int sidx = tid + THREADS * j;
    const int row = sidx / P;
    const int piece = sidx % P;
    xs[j] = p.x + static_cast<int64_t>(min(m0 + row, p.M - 1)) * p.x_stride + 8 * piece;
    xslot[j] = x_slot<P>(row, piece);
  }
  // This lane's weight row (feature n0 + i16), 16 bytes per k-step.
  const uint16_t* wg = p.w0 + static_cast<int64_t>(n0 + i16) * p.w_stride + 8 * kg;
  const uint16_t* wu =
      SWIGLU ? p.w1 + static_cast<int64_t>(n0 + i16) * p.w_stride + 8 * kg : nullptr;

  struct Stage {
    u16x8_t x[XL];
    bf16x8_t g[KS];  // [k-step]
    bf16x8_t u[SWIGLU ? KS : 1];
  };
  auto load_chunk = [&](Stage& st, int c) __attribute__((always_inline)) {
    const int k0 = c * KC;
#pragma unroll
    for (int j = 0; j < XL; ++j) st.x[j] = *reinterpret_cast<const u16x8_t*>(xs[j] + k0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      st.g[s] = load8(wg + k0 + 32 * s);
      if constexpr (SWIGLU) st.u[s] = load8(wu + k0 + 32 * s);
    }
  };
  auto store_x = [&](const Stage& st, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XL; ++j) sX[stage][xslot[j]] = st.x[j];
  };

  f32x4_t a0[MT], a1[SWIGLU ? MT : 1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    a0[mt] = f32x4_t(0.f);
    if constexpr (SWIGLU) a1[mt] = f32x4_t(0.f);
  }
  auto compute = [&](const Stage& st, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8_t xf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xf[mt] = __builtin_bit_cast(bf16x8_t, sX[stage][x_slot<P>(16 * mt + i16, 4 * s + kg)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a0[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.g[s], xf[mt], a0[mt], 0, 0, 0);
        if constexpr (SWIGLU)
          a1[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.u[s], xf[mt], a1[mt], 0, 0, 0);
      }
    }
  };

  // Chunk c lives in register stage c % NST and LDS stage c % 2.
  Stage r[NST];
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) load_chunk(r[j], min(j, nchunks - 1));
  store_x(r[0], 0);
  __syncthreads();
  int c = 0;
  // No branches around the loads, here or in the prologue: the compiler then
  // counts the loads in flight exactly (a path that skipped some would make
  // it wait for nearly all of them in every iteration). Near the end the
  // chunk index is clamped, so the last chunk is re-read into stages that
  // are never computed, and the LDS stage past the last chunk receives data
  // nobody reads.
  for (; c + NST <= nchunks; c += NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      load_chunk(r[(j + NST - 1) % NST], min(c + j + NST - 1, nchunks - 1));
      store_x(r[(j + 1) % NST], ((j + 1) & 1) ^ (c & 1));
      compute(r[j], (j & 1) ^ (c & 1));
      lds_barrier();
    }
  }
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) {
    if (c + j < nchunks) {
      if (c + j + NST - 1 < nchunks) load_chunk(r[(j + NST - 1) % NST], c + j + NST - 1);
      if (c + j + 1 < nchunks) store_x(r[(j + 1) % NST], ((j + 1) & 1) ^ (c & 1));
      compute(r[j], (j & 1) ^ (c & 1));
      lds_barrier();
    }
  }

  // Lane holds output features n0 + 4 kg + e (e = 0..3) of row m0 + 16 mt + i16.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + i16;
    if (m >= p.M) continue;
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v;
      if constexpr (SWIGLU) {
        // The two projections rounded as separate outputs, then SwiGLU.
        const float gr = tv::bf16_to_f32(tv::f32_to_bf16_rne(a0[mt][e]));
        const float ur = tv::bf16_to_f32(tv::f32_to_bf16_rne(a1[mt][e]));
        v = silu(gr) * ur;
      } else {
        v = a0[mt][e];
      }
      h[e] = tv::f32_to_bf16_rne(v);
    }
    *reinterpret_cast<uint2*>(p.y + static_cast<int64_t>(m) * p.y_stride + n0 + 4 * kg) =
        make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

// ---- All rows per workgroup (gate/up: large N, M up to 272) ----
// The batch's rows and the weight rows of the workgroup's feature tiles both
// go through LDS, in chunks of 32 k, and are shared by the eight waves: wave
// w owns row tiles w and w + 8 (rows 16 w .. and 16 (w + 8) ..) for every
// feature tile of the workgroup and, with a 17th row tile, the products of
// that tile with feature tile w. Each workgroup takes a contiguous run of
// ceil or floor N / (16 nwg) feature tiles (at most FTMAX), so a single pass
// of one workgroup per compute unit covers N, and each weight byte crosses
// from L2 to the compute units once (the 96-row groups above stream every
// weight slice through three of them, in two passes). The input rows,
// re-read by every workgroup, stay in L2. Same MFMA operands and k order as
// linear_rows_kernel, so every output has the same bits.
constexpr int kAllRowTiles = 17;              // rows per workgroup: up to 272
constexpr int kAllRows = 16 * kAllRowTiles;
constexpr int kAllThreads = 512;
constexpr int kAllStages = 4;                 // register stages (chunks of 32 k)

struct LinAllParams {
  const uint16_t* x;
  const uint16_t* w0;
  const uint16_t* w1;
  int64_t x_stride, w_stride, y_stride;
  int M, K, ntiles, nwg;
  uint16_t* y;
};

// 16-byte piece c (k-group of 8) of LDS row r of a 32-k chunk (4 pieces per
// 64-byte row, XOR-swizzled by (r / 2) mod 4): the eight consecutive rows
// that one phase of an MFMA operand read touches (eight lanes, 16 bytes
// each) land on eight different 16-byte slots modulo 128 bytes, so the read
// is free of bank conflicts (with r / 4 instead, rows r and r + 2 collided).
__device__ __forceinline__ int all_slot(int r, int c) { return r * 4 + (c ^ ((r >> 1) & 3)); }

template <bool SWIGLU, int FTMAX, int NST>
__global__ __launch_bounds__(kAllThreads) void linear_allrows_kernel(LinAllParams p) {
  constexpr int NMAT = SWIGLU ? 2 : 1;
  constexpr int WROWS = 16 * FTMAX * NMAT;                          // weight rows per chunk
  constexpr int XPIECES = kAllRows * 4;                             // 16-byte pieces per chunk
  constexpr int WPIECES = WROWS * 4;
  constexpr int XL = (XPIECES + kAllThreads - 1) / kAllThreads;     // per thread
  constexpr int WL = (WPIECES + kAllThreads - 1) / kAllThreads;
  __shared__ __attribute__((aligned(16))) u16x8_t sX[2][XPIECES + 1];
  __shared__ __attribute__((aligned(16))) u16x8_t sW[2][WPIECES + 1];
  const int g = blockIdx.x;
  if (g >= p.nwg) return;
  const int ft0 = static_cast<int>(static_cast<int64_t>(g) * p.ntiles / p.nwg);
  const int ft1 = static_cast<int>(static_cast<int64_t>(g + 1) * p.ntiles / p.nwg);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (a scalar register): the extra products below are skipped
  // by a scalar branch; an MFMA does not honour the EXEC mask, so a per-lane
  // condition around it would not skip it.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15;
  const int kg = lane >> 4;
  const int nchunks = p.K / 32;

  // Staging: thread t copies pieces t, t + 512, ... (row = s / 4, piece =
  // s % 4). Input rows past M re-read row M - 1; weight rows past the
  // workgroup's tiles re-read its last row (their products are not stored);
  // threads past the last piece re-read it into the spare slot.
  // Element offsets below 2^31 (the host checks), from uniform bases.
  int xoff[XL], xslot[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int sraw = tid + kAllThreads * j;
    const int sidx = min(sraw, XPIECES - 1);
    const int row = sidx >> 2, c = sidx & 3;
    xoff[j] = min(row, p.M - 1) * static_cast<int>(p.x_stride) + 8 * c;
    xslot[j] = sraw >= XPIECES ? XPIECES : all_slot(row, c);
  }
  int woff[WL], wslot[WL];
  bool wup[WL];
  const int nfeat = 16 * (ft1 - ft0);
  const uint16_t* wbase0 = p.w0 + static_cast<int64_t>(16 * ft0) * p.w_stride;
  const uint16_t* wbase1 = SWIGLU ? p.w1 + static_cast<int64_t>(16 * ft0) * p.w_stride : nullptr;
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int sraw = tid + kAllThreads * j;
    const int sidx = min(sraw, WPIECES - 1);
    const int row = sidx >> 2, c = sidx & 3;  // row = mat * 16 FTMAX + feature
    const int mat = row / (16 * FTMAX);
    const int f = min(row - mat * 16 * FTMAX, nfeat - 1);
    woff[j] = f * static_cast<int>(p.w_stride) + 8 * c;
    wup[j] = SWIGLU && mat;
    wslot[j] = sraw >= WPIECES ? WPIECES : all_slot(row, c);
  }

  struct Stage {
    u16x8_t x[XL];
    u16x8_t w[WL];
  };
  auto load_chunk = [&](Stage& st, int c) __attribute__((always_inline)) {
    const int k0 = 32 * c;
#pragma unroll
    for (int j = 0; j < XL; ++j) st.x[j] = *reinterpret_cast<const u16x8_t*>(p.x + xoff[j] + k0);
#pragma unroll
    for (int j = 0; j < WL; ++j)
      st.w[j] = *reinterpret_cast<const u16x8_t*>((wup[j] ? wbase1 : wbase0) + woff[j] + k0);
  };
  auto store_chunk = [&](const Stage& st, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XL; ++j) sX[stage][xslot[j]] = st.x[j];
#pragma unroll
    for (int j = 0; j < WL; ++j) sW[stage][wslot[j]] = st.w[j];
  };

  // Accumulators: [row tile w, w + 8][feature tile][matrix], and the extra
  // (row tile 16, feature tile = wave) pair.
  f32x4_t acc[2][FTMAX][NMAT], ext[NMAT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int f = 0; f < FTMAX; ++f)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[a][f][m] = f32x4_t(0.f);
#pragma unroll
  for (int m = 0; m < NMAT; ++m) ext[m] = f32x4_t(0.f);
  const bool has_ext = wave < FTMAX;
  auto compute = [&](int stage) __attribute__((always_inline)) {
    bf16x8_t xf[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const int rt = a < 2 ? wave + 8 * a : 16;
      xf[a] = __builtin_bit_cast(bf16x8_t, sX[stage][all_slot(16 * rt + i16, kg)]);
    }
#pragma unroll
    for (int f = 0; f < FTMAX; ++f) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const bf16x8_t wf = __builtin_bit_cast(
            bf16x8_t, sW[stage][all_slot(m * 16 * FTMAX + 16 * f + i16, kg)]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
          acc[a][f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[a], acc[a][f][m], 0, 0, 0);
        if (f == wave)
          ext[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[2], ext[m], 0, 0, 0);
      }
    }
  };

  // Chunk c lives in register stage c % NST and LDS stage c % 2 (see
  // linear_rows_kernel: loads run NST - 1 chunks ahead, no branch around
  // them, the last chunk re-read past the end).
  Stage r[NST];
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) load_chunk(r[j], min(j, nchunks - 1));
  store_chunk(r[0], 0);
  __syncthreads();
  int c = 0;
  for (; c + NST <= nchunks; c += NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      load_chunk(r[(j + NST - 1) % NST], min(c + j + NST - 1, nchunks - 1));
      store_chunk(r[(j + 1) % NST], ((j + 1) & 1) ^ (c & 1));
      compute((j & 1) ^ (c & 1));
      lds_barrier();
    }
  }
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) {
    if (c + j < nchunks) {
      if (c + j + NST - 1 < nchunks) load_chunk(r[(j + NST - 1) % NST], c + j + NST - 1);
      if (c + j + 1 < nchunks) store_chunk(r[(j + 1) % NST], ((j + 1) & 1) ^ (c & 1));
      compute((j & 1) ^ (c & 1));
      lds_barrier();
    }
  }

  // Lane holds output features 4 kg + e (e = 0..3) of a feature tile for row
  // i16 of a row tile.
  auto store_tile = [&](const f32x4_t* a, int rt, int f) __attribute__((always_inline)) {
    const int m = 16 * rt + i16;
    if (m >= p.M || ft0 + f >= ft1) return;
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v;
      if constexpr (SWIGLU) {
        const float gr = tv::bf16_to_f32(tv::f32_to_bf16_rne(a[0][e]));
        const float ur = tv::bf16_to_f32(tv::f32_to_bf16_rne(a[1][e]));
        v = silu(gr) * ur;
      } else {
        v = a[0][e];
      }
      h[e] = tv::f32_to_bf16_rne(v);
    }
    *reinterpret_cast<uint2*>(p.y + static_cast<int64_t>(m) * p.y_stride + 16 * (ft0 + f) + 4 * kg) =
        make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  };
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int f = 0; f < FTMAX; ++f) store_tile(acc[a][f], wave + 8 * a, f);
  if (has_ext) store_tile(ext, 16, wave);
}

int launch_linear(const void* x, int64_t x_stride, const void* w0, const void* w1,
                  int64_t w_stride, int M, int K, int N, void* y, int64_t y_stride,
                  bool swiglu, hipStream_t stream) {
  if (!x || !w0 || !y || (swiglu && !w1)) return TV_ERR_NULL;
  if (M < 0 || K < kLinKC || N < kLinFeat || K % kLinKC || N % kLinFeat) return TV_ERR_SHAPE;
  if (M > 65536) return TV_ERR_SHAPE;
  if (!tvh::aligned16(x) || !tvh::aligned16(w0) || (swiglu && !tvh::aligned16(w1)) ||
      !tvh::aligned16(y))
    return TV_ERR_ALIGN;
  if (x_stride < K || w_stride < K || y_stride < N) return TV_ERR_SHAPE;
  if (x_stride % 8 || w_stride % 8 || y_stride % 4) return TV_ERR_ALIGN;
  if (M == 0) return TV_OK;
  LinParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.w0 = static_cast<const uint16_t*>(w0);
  p.w1 = static_cast<const uint16_t*>(w1);
  p.x_stride = x_stride;
  p.w_stride = w_stride;
  p.y_stride = y_stride;
  p.M = M;
  p.K = K;
  p.N = N;
  p.y = static_cast<uint16_t*>(y);
  auto launch = [&](auto kernel, int rows, int waves) {
    p.mgroups = (M + rows - 1) / rows;
    const int64_t work = static_cast<int64_t>(p.mgroups) * (N / (16 * waves));
    if (work > (int64_t(1) << 30)) return TV_ERR_SHAPE;
    p.work = static_cast<int>(work);
    const int grid = (p.work + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * waves), 0, stream, p);
    return TV_OK;
  };
  int rc;
  // All rows per workgroup when they are many (193..272) and N gives every
  // workgroup of one pass 4 or 5 feature tiles.
  const int ntiles = N / 16;
  const int nw = tvh::grid_workgroups();
  const int ftmax = (ntiles + nw - 1) / nw;
  if (M > 192 && M <= kAllRows && (ftmax == 4 || ftmax == 5) &&
      static_cast<int64_t>(M) * x_stride < INT32_MAX &&
      static_cast<int64_t>(16 * ftmax) * w_stride < INT32_MAX) {
    LinAllParams a;
    a.x = p.x;
    a.w0 = p.w0;
    a.w1 = p.w1;
    a.x_stride = x_stride;
    a.w_stride = w_stride;
    a.y_stride = y_stride;
    a.M = M;
    a.K = K;
    a.ntiles = ntiles;
    a.nwg = (ntiles + ftmax - 1) / ftmax;
    a.y = p.y;
    const dim3 grid(a.nwg), block(kAllThreads);
    if (swiglu) {
      if (ftmax == 5)
        hipLaunchKernelGGL((linear_allrows_kernel<true, 5, kAllStages>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((linear_allrows_kernel<true, 4, kAllStages>), grid, block, 0, stream, a);
    } else {
      if (ftmax == 5)
        hipLaunchKernelGGL((linear_allrows_kernel<false, 5, kAllStages>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((linear_allrows_kernel<false, 4, kAllStages>), grid, block, 0, stream, a);
    }
    return tvh::launch_status();
  }
  if (!swiglu)
    rc = launch(linear_rows_kernel<false, 6, 64, kRows, 4>, kRows, 4);
  else if (K % kDeepKC == 0 && N % (16 * kWavesWide) == 0)
    rc = launch(linear_rows_kernel<true, 3, kDeepKC, kRows, kWavesWide>, kRows, kWavesWide);
  else
    rc = launch(linear_rows_kernel<true, 5, 64, kRows, 4>, kRows, 4);
  if (rc != TV_OK) return rc;
  return tvh::launch_status();
}

}  // namespace

extern "C" int tv_linear_rows(const void* x, int64_t x_stride, const void* w, int64_t w_stride,
                              int M, int K, int N, void* y, int64_t y_stride,
                              hipStream_t stream) {
  return launch_linear(x, x_stride, w, nullptr, w_stride, M, K, N, y, y_stride, false, stream);
}

extern "C" int tv_linear_swiglu_rows(const void* x, int64_t x_stride, const void* w_gate,
                                     const void* w_up, int64_t w_stride, int M, int K, int N,
                                     void* y, int64_t y_stride, hipStream_t stream) {
  return launch_linear(x, x_stride, w_gate, w_up, w_stride, M, K, N, y, y_stride, true, stream);
}
