// Shared device/host helpers of the tree-verification kernels (gfx950).
#ifndef TV_COMMON_H_
#define TV_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

constexpr int kWave = 64;

// Per-sequence validity shared by the kernels that read ctx_len/n_nodes.
enum RowCheck { kRowLive = 0, kRowPadded = 1, kRowBad = 2 };

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}

}  // namespace tv

// Host-side helpers shared by the entry points.
namespace tvh {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tvh

#endif  // TV_COMMON_H_
