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
