// Status strings and version of the tree-verification library.
#include "tv_common.h"

extern "C" const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_SHAPE: return "a size or stride is out of range";
    case TV_ERR_DTYPE: return "unknown element type";
    case TV_ERR_ALIGN: return "pointer or stride misaligned";
    case TV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TV_ERR_UNSUPPORTED: return "unsupported configuration";
    case TV_ERR_HIP: return "HIP runtime error";
    case TV_ROW_BAD_PARENT: return "row: a parent link is not a smaller node index";
    case TV_ROW_CTX_BOUND: return "row: context length outside its bounds";
    case TV_ROW_NNODES: return "row: n_nodes outside [0, T]";
    case TV_ROW_BAD_TOKEN: return "row: a draft token is outside the vocabulary";
    case TV_ROW_BAD_PATH: return "row: the accepted path is not an increasing walk from the root";
    case TV_ROW_BAD_START: return "row: packed rows outside [0, rows_total)";
    default: return "unknown status";
  }
}

extern "C" int tv_version(void) { return 100; }

// ----------------------------------------------------- read-rate probe ---
// Streams a buffer once (16 bytes per lane, non-temporal, every load of a
// thread's batch in flight together) and folds it into one 32-bit XOR,
// which keeps the loads from being removed. Used to measure the chip's
// streaming-read rate beside the library's own kernels.
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBatch = 8;  // 16-byte loads per thread per round

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t step = static_cast<size_t>(gridDim.x) * kProbeThreads * kProbeBatch;
  for (size_t i0 = static_cast<size_t>(blockIdx.x) * kProbeThreads * kProbeBatch + threadIdx.x;
       i0 < n16; i0 += step) {
    u32x4_t v[kProbeBatch];
#pragma unroll
    for (int u = 0; u < kProbeBatch; ++u) {
      const size_t i = i0 + static_cast<size_t>(u) * kProbeThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kProbeBatch; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

extern "C" int tv_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return TV_ERR_NULL;
  if (bytes == 0 || (bytes & 15u) != 0) return TV_ERR_SHAPE;
  if (!tvh::aligned16(buf)) return TV_ERR_ALIGN;
  const size_t n16 = bytes / 16;
  // Four workgroups per CU over 256 CUs; each thread keeps eight loads in
  // flight.
  const size_t per_wg = static_cast<size_t>(kProbeThreads) * kProbeBatch;
  const int grid = static_cast<int>(std::min<size_t>(1024, (n16 + per_wg - 1) / per_wg));
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4_t*>(buf), n16, sink);
  return tvh::launch_status();
}
