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

// acc + the sum of four bf16 values (v_dot2_f32_bf16 against (1, 1); the
// products are exact).  A softmax row sum built this way adds exactly the
// bf16-rounded weights that a bf16 matrix product consumes.
typedef __bf16 pkv_bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pkv_bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float add_bf16x4(pkv_bf16x4 v, float acc) {
  const pkv_bf16x2 one2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, acc, false);
}

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

// Max over aligned groups of 16 consecutive lanes; every lane gets its group's.
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppMirror>(v));
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);  // works for any wave of a multi-wave block
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

struct SegInfo {
  int slot, L, n, row0;
  bool ok;
};

// Segment b's metadata, with every value that could send a kernel out of
// bounds rejected or clamped.
__device__ __forceinline__ SegInfo seg_info(const AttendArgs &a, int b) {
  SegInfo s{0, 0, 0, 0, false};
  if (b < 0 || b >= a.num_segments) return s;
  const int n = a.query_len[b];
  const int slot = a.row_to_slot[b];
  const int r0 = a.query_start[b];
  if (n < 1 || n > a.max_query || slot < 0 || slot >= a.num_slots || r0 < 0 || r0 > a.total_q - n) return s;
  int L = a.context_lens[slot];
  L = min(min(L, a.max_blocks * kBlockTokens), a.max_context);
  if (L < n) return s;
  s.slot = slot;
  s.L = L;
  s.n = n;
  s.row0 = r0;
  s.ok = true;
  return s;
}

// The same for a wave-uniform b, with the fields moved to scalar registers so
// that loop bounds and block lookups derived from them stay scalar.
__device__ __forceinline__ SegInfo seg_info_uniform(const AttendArgs &a, int b) {
  const SegInfo v = seg_info(a, __builtin_amdgcn_readfirstlane(b));
  SegInfo s;
  s.slot = __builtin_amdgcn_readfirstlane(v.slot);
  s.L = __builtin_amdgcn_readfirstlane(v.L);
  s.n = __builtin_amdgcn_readfirstlane(v.n);
  s.row0 = __builtin_amdgcn_readfirstlane(v.row0);
  s.ok = __builtin_amdgcn_readfirstlane(static_cast<int>(v.ok)) != 0;
  return s;
}

// Work units are numbered segment by segment; units_fn(b) gives segment b's
// count (0 past the end).  Each wavefront runs these on its own.
template <typename F>
__device__ __forceinline__ int count_units(int num_segments, F units_fn) {
  const int lane = threadIdx.x & (kWave - 1);
  int total = 0;
  for (int c0 = 0; c0 < num_segments; c0 += kWave) {
    int u = units_fn(c0 + lane);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) u += __shfl_xor(u, d);
    total += u;
  }
  return total;
}

// Sum of units_fn(b') over the segments b' < b (the same on every lane).
template <typename F>
__device__ __forceinline__ int64_t units_before(int b, F units_fn) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t total = 0;
  for (int c0 = 0; c0 < b; c0 += kWave) {
    int u = c0 + lane < b ? units_fn(c0 + lane) : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) u += __shfl_xor(u, d);
    total += u;
  }
  return total;
}

template <typename F>
__device__ __forceinline__ int find_unit(int num_segments, int unit, F units_fn, int *rest) {
  const int lane = threadIdx.x & (kWave - 1);
  int base = 0;
  for (int c0 = 0; c0 < num_segments; c0 += kWave) {
    const int u = units_fn(c0 + lane);
    const int incl = wave_inclusive_scan(u);
    const int ct = __shfl(incl, kWave - 1);
    if (unit < base + ct) {
      const unsigned long long mask = __ballot(base + incl > unit);
      const int bl = __ffsll(static_cast<long long>(mask)) - 1;
      *rest = unit - (base + __shfl(incl, bl) - __shfl(u, bl));
      return c0 + bl;
    }
    base += ct;
  }
  *rest = 0;
  return -1;
}

// Where a work unit falls: its segment b (-1 past the last unit), its index
// within the segment, the segment's metadata, and the sum of the partial
// slots of the segments before b.  All uniform over the wavefront.
struct UnitPlace {
  int b, rest;
  int64_t slots_before;
  SegInfo si;
};

// Work units and partial slots per segment, from units_of(SegInfo) and
// slots_of(SegInfo) (both 0 for a segment that fails its checks).  When every
// segment fits one wavefront the metadata is read once, lane b holding
// segment b, so locating a unit costs one round of dependent loads and no
// more; past that, each question walks the segments again.
template <typename FU, typename FS>
struct UnitMap {
  const AttendArgs &a;
  FU units_of;
  FS slots_of;
  bool in_lanes;
  SegInfo mine;        // segment `lane` (in_lanes only)
  int units, incl;     // its units and the inclusive scan over lanes
  int total;           // units over all segments (uniform)

  __device__ __forceinline__ UnitMap(const AttendArgs &args, FU fu, FS fs)
      : a(args), units_of(fu), slots_of(fs), in_lanes(args.num_segments <= kWave) {
    if (in_lanes) {
      mine = seg_info(a, static_cast<int>(threadIdx.x & (kWave - 1)));
      units = units_of(mine);
      incl = wave_inclusive_scan(units);
      total = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
    } else {
      mine = SegInfo{0, 0, 0, 0, false};
      units = incl = 0;
      total = __builtin_amdgcn_readfirstlane(
          count_units(a.num_segments, [&](int b) { return units_of(seg_info(a, b)); }));
    }
  }

  __device__ __forceinline__ UnitPlace place(int unit) const {
    UnitPlace p;
    p.b = -1;
    p.rest = 0;
    p.slots_before = 0;
    p.si = SegInfo{0, 0, 0, 0, false};
    if (unit < 0 || unit >= total) return p;
    const int lane = threadIdx.x & (kWave - 1);
    if (in_lanes) {
      const int bl = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(__ballot(incl > unit))) - 1);
      p.b = bl;
      p.rest = unit - (__builtin_amdgcn_readlane(incl, bl) - __builtin_amdgcn_readlane(units, bl));
      p.si.slot = __builtin_amdgcn_readlane(mine.slot, bl);
      p.si.L = __builtin_amdgcn_readlane(mine.L, bl);
      p.si.n = __builtin_amdgcn_readlane(mine.n, bl);
      p.si.row0 = __builtin_amdgcn_readlane(mine.row0, bl);
      p.si.ok = true;                                   // a segment with units passed its checks
      long long sb = lane < bl ? static_cast<long long>(slots_of(mine)) : 0;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) sb += __shfl_xor(sb, d);
      p.slots_before = sb;
      return p;
    }
    int r;
    p.b = __builtin_amdgcn_readfirstlane(
        find_unit(a.num_segments, unit, [&](int b) { return units_of(seg_info(a, b)); }, &r));
    p.rest = __builtin_amdgcn_readfirstlane(r);
    p.si = seg_info_uniform(a, p.b);
    p.slots_before = units_before(p.b, [&](int b) { return slots_of(seg_info(a, b)); });
    return p;
  }
};

template <typename FU, typename FS>
__device__ __forceinline__ UnitMap<FU, FS> make_unit_map(const AttendArgs &a, FU units_of, FS slots_of) {
  return UnitMap<FU, FS>(a, units_of, slots_of);
}

}  // namespace pkv
