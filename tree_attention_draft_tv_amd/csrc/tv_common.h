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

// Cross-lane moves on the vector ALU (DPP and the gfx950 lane-swap
// instructions), so that reductions and scans wait on the vector pipeline
// instead of on LDS round trips (__shfl compiles to ds_bpermute). kDppXor1
// and kDppXor2 exchange within quads (lane ^ 1, lane ^ 2); kDppHalfMirror
// pairs lane i with 7 - i in each group of 8; kDppRowRor8 is lane ^ 8 within
// a row of 16; kDppRowShr(n) reads lane - n within the row (lanes below n
// keep the `old` operand, 0 here).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppRowRor8 = 0x128;     // row_ror:8
constexpr int kDppRowShr(int n) { return 0x110 + n; }

template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, 0xF, 0xF, false);
}

// Sum / max over the wave, in every lane: within rows of 16 by DPP, then
// across rows with permlane16_swap (rows 0 <-> 1, 2 <-> 3) and
// permlane32_swap (the two halves).
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += dpp_i32<kDppXor1>(x);
  x += dpp_i32<kDppXor2>(x);
  x += dpp_i32<kDppHalfMirror>(x);
  x += dpp_i32<kDppRowRor8>(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = static_cast<int>(p16[0]) + static_cast<int>(p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return static_cast<int>(p32[0]) + static_cast<int>(p32[1]);
}

__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, dpp_i32<kDppXor1>(x));
  x = max(x, dpp_i32<kDppXor2>(x));
  x = max(x, dpp_i32<kDppHalfMirror>(x));
  x = max(x, dpp_i32<kDppRowRor8>(x));
  const auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(static_cast<int>(p16[0]), static_cast<int>(p16[1]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(static_cast<int>(p32[0]), static_cast<int>(p32[1]));
}

// Inclusive prefix sum over the lanes of a wave: shifted adds within each
// row of 16, then the totals of the earlier rows (scalar reads).
__device__ __forceinline__ int wave_scan_i32(int x, int lane) {
  x += dpp_i32<kDppRowShr(1)>(x);
  x += dpp_i32<kDppRowShr(2)>(x);
  x += dpp_i32<kDppRowShr(4)>(x);
  x += dpp_i32<kDppRowShr(8)>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  if (lane >= 16) x += r0;
  if (lane >= 32) x += r1;
  if (lane >= 48) x += r2;
  return x;
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

// Compute units of the current device rounded down to a multiple of 8 (the
// XCDs of a gfx950), cached per device; 256 (MI355X) if it cannot be queried.
inline int grid_workgroups() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu < 8)
      cu = 256;
    cache[dev] = cu / 8 * 8;
  }
  return cache[dev];
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tvh

#endif  // TV_COMMON_H_
