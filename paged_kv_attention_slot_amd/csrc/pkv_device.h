// Device helpers shared by the gfx950 kernels of the paged-KV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

constexpr int kWave = 64;        // CDNA wavefront width

// bf16 <-> fp32.  A bf16 value is the high half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load of data read once (K/V tiles): marked nontemporal so it
// streams past the caches instead of displacing reused lines.
typedef unsigned int pkv_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
#if PKV_STREAM_LOADS
  const pkv_u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const pkv_u32x4 *>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
#else
  return *p;
#endif
}

// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;      // lane i <- 15-i inside each 16-lane row

// Sum over aligned groups of W consecutive lanes (W = 1, 2, 4, 8, 16, 32, 64);
// every lane of a group receives the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_mov<kDppMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16);
  if constexpr (W >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

}  // namespace pkv
