// Decode-row paged attention with split-context partitions, and the reduce
// that merges partitions.
//
// "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog),
// §Paged KV and paged attention: a row reads its sequence's cached history by
// following the slot's block table and visiting blocks in logical order, with
// no gather or relocation.  §Keeping track of each request: the row reaches
// its slot through the explicit row-to-slot map.
//
// Work item = (segment, KV head g, partition of kDecodePartitionTokens tokens);
// one wavefront per item, all G = Hq/Hkv query heads of the group at once, so
// every K/V tile is read from HBM once for the whole group.  Items are
// enumerated on the device from the step metadata (no host copy of the
// lengths is needed) and handed to a persistent grid in a fixed order.
//
// Lane layout inside a wave: one (block, head) tile of K is 16 token rows of
// D elements; the wave reads it with 1 KiB loads of 16 B per lane, so lane
// (r, c) holds 16 B (column c) of token rows r, r + TPL, r + 2 TPL, ...  The
// q . k dot products are reduced across the LPR lanes of a row with DPP.
// Each lane row r keeps its own online-softmax state (m, l, acc) over its
// tokens; rows merge once per item (log-sum-exp), partitions merge in the
// reduce kernel, in partition order.  The reduction order of a row depends
// only on its own context length.
#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T, int D>
struct Geo {
  static constexpr int kElem = sizeof(T);
  static constexpr int kRowBytes = D * kElem;
  static constexpr int kLPR = kRowBytes / 16;          // lanes per token row
  static constexpr int kTPL = kWave / kLPR;            // token rows per 1 KiB load
  static constexpr int kLoads = kBlockTokens / kTPL;   // loads per (block, head) tile
  static constexpr int kEPL = 16 / kElem;              // elements per lane per load
  static constexpr int kTileBytes = kBlockTokens * kRowBytes;
};

__device__ __forceinline__ int num_parts(int L) {
  return (L + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
}

__device__ __forceinline__ int units_of(const AttendArgs &a, int b) {
  const SegInfo s = seg_info(a, b);
  if (!s.ok) return 0;
  if (!a.multirow && s.n != 1) return 0;
  return a.multirow ? s.n * num_parts(s.L) : num_parts(s.L);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

// Find the segment holding `unit` and the unit's index inside it.
__device__ __forceinline__ void locate(const AttendArgs &a, int unit, int u0, int incl0, int *seg, int *rest) {
  const int total0 = __shfl(incl0, kWave - 1);
  if (unit < total0) {
    const unsigned long long mask = __ballot(incl0 > unit);
    const int bl = __ffsll(static_cast<long long>(mask)) - 1;
    *seg = bl;
    *rest = unit - (__shfl(incl0, bl) - __shfl(u0, bl));
    return;
  }
  int base = total0;
  const int lane = threadIdx.x;
  for (int c0 = kWave; c0 < a.num_segments; c0 += kWave) {
    const int u = units_of(a, c0 + lane);
    const int incl = wave_inclusive_scan(u);
    const int ct = __shfl(incl, kWave - 1);
    if (unit < base + ct) {
      const unsigned long long mask = __ballot(base + incl > unit);
      const int bl = __ffsll(static_cast<long long>(mask)) - 1;
      *seg = c0 + bl;
      *rest = unit - (base + __shfl(incl, bl) - __shfl(u, bl));
      return;
    }
    base += ct;
  }
  *seg = -1;
  *rest = 0;
}

template <typename T>
__device__ __forceinline__ float dot16(const uint4 &k, const uint4 &q);

template <>
__device__ __forceinline__ float dot16<uint16_t>(const uint4 &k, const uint4 &q) {
  float acc = 0.f;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x), __builtin_bit_cast(bf16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y), __builtin_bit_cast(bf16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z), __builtin_bit_cast(bf16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w), __builtin_bit_cast(bf16x2_t, q.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<float>(const uint4 &k, const uint4 &q) {
  float acc = __uint_as_float(k.x) * __uint_as_float(q.x);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

template <typename T, int EPL>
__device__ __forceinline__ void unpack16(const uint4 &v, float (&f)[EPL]) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

template <int NL>
struct Tile {
  uint4 k[NL];
  uint4 v[NL];
};

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void decode_kernel(AttendArgs a) {
  using Gm = Geo<T, D>;
  constexpr int LPR = Gm::kLPR, TPL = Gm::kTPL, NL = Gm::kLoads, EPL = Gm::kEPL;
  constexpr int PT = kDecodePartitionTokens;
  static_assert(PT % kBlockTokens == 0 && PT / kBlockTokens <= kWave, "partition must fit one table load");
  const int lane = threadIdx.x;
  const int r = lane / LPR;
  const int c = lane % LPR;

  // Lane b keeps segment b's metadata (first 64 segments) so work items do
  // not re-read it from memory.
  const SegInfo mine = seg_info(a, lane);
  const int u0 = mine.ok && (a.multirow || mine.n == 1) ? (a.multirow ? mine.n : 1) * num_parts(mine.L) : 0;
  const int incl0 = wave_inclusive_scan(u0);
  int total = __shfl(incl0, kWave - 1);
  for (int c0 = kWave; c0 < a.num_segments; c0 += kWave) total += wave_sum_int(units_of(a, c0 + lane));
  const int64_t items = static_cast<int64_t>(total) * a.num_kv_heads;
  const float c_log2 = a.scale_log2;

  for (int64_t f = blockIdx.x; f < items; f += gridDim.x) {
    const int unit = static_cast<int>(f / a.num_kv_heads);
    const int g = static_cast<int>(f - static_cast<int64_t>(unit) * a.num_kv_heads);
    int b, rest;
    locate(a, unit, u0, incl0, &b, &rest);
    SegInfo si;
    if (b >= 0 && b < kWave) {
      si.slot = __builtin_amdgcn_readlane(mine.slot, b);
      si.L = __builtin_amdgcn_readlane(mine.L, b);
      si.n = __builtin_amdgcn_readlane(mine.n, b);
      si.row0 = __builtin_amdgcn_readlane(mine.row0, b);
      si.ok = true;
    } else {
      si = seg_info(a, b);
      if (!si.ok) continue;
    }
    const int np = num_parts(si.L);
    const int i = a.multirow ? rest / np : 0;
    const int part = a.multirow ? rest - i * np : rest;
    const int row = si.row0 + i;
    const int limit = si.L - si.n + i + 1;             // tokens visible to this row
    // Partitions past the row's own position hold none of its keys: no item
    // (a decode row sees all of its segment's partitions).
    const int np_row = num_parts(limit);
    if (part >= np_row) continue;
    const int tok0 = part * PT;
    const int tok1 = min(limit, tok0 + PT);
    const int hq0 = g * G;

    // Online-softmax state of this lane row: running max m (already scaled by
    // scale * log2 e), running sum l, unnormalised output acc.
    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -FLT_MAX;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }

    if (tok0 < tok1) {
      const int j0 = tok0 / kBlockTokens;
      const int nb = (tok1 + kBlockTokens - 1) / kBlockTokens - j0;
      int phys_lane = 0;
      if (lane < nb) {
        phys_lane = a.block_tables[static_cast<int64_t>(si.slot) * a.max_blocks + j0 + lane];
        phys_lane = min(max(phys_lane, 0), a.num_blocks - 1);
      }
      uint4 q[G];
      const uint4 *qrow = reinterpret_cast<const uint4 *>(static_cast<const T *>(a.q) +
                                                          (static_cast<int64_t>(row) * a.num_q_heads + hq0) * D);
#pragma unroll
      for (int h = 0; h < G; ++h) q[h] = qrow[h * LPR + c];

      const char *kbase = static_cast<const char *>(a.k);
      const char *vbase = static_cast<const char *>(a.v);
      auto load_tile = [&](Tile<NL> &t, int jj) {
        const int phys = __builtin_amdgcn_readlane(phys_lane, jj);
        const int64_t off = (static_cast<int64_t>(phys) * a.num_kv_heads + g) * Gm::kTileBytes;
        const uint4 *kp = reinterpret_cast<const uint4 *>(kbase + off);
        const uint4 *vp = reinterpret_cast<const uint4 *>(vbase + off);
#pragma unroll
        for (int x = 0; x < NL; ++x) t.k[x] = stream_load(kp + x * kWave + lane);
#pragma unroll
        for (int x = 0; x < NL; ++x) t.v[x] = stream_load(vp + x * kWave + lane);
      };
      auto compute_tile = [&](const Tile<NL> &t, int jj, auto partial_tag) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        const int tokbase = (j0 + jj) * kBlockTokens;
        float s[NL][G];
#pragma unroll
        for (int x = 0; x < NL; ++x)
#pragma unroll
          for (int h = 0; h < G; ++h) s[x][h] = group_sum<LPR>(dot16<T>(t.k[x], q[h]));
        bool valid[NL];
#pragma unroll
        for (int x = 0; x < NL; ++x) valid[x] = !PARTIAL || (tokbase + x * TPL + r < tok1);
        if constexpr (PARTIAL) {
#pragma unroll
          for (int x = 0; x < NL; ++x)
#pragma unroll
            for (int h = 0; h < G; ++h) s[x][h] = valid[x] ? s[x][h] : -INFINITY;
        }
        // Raise the running max only when this tile exceeds it (rare after
        // the first tiles); the rescale is skipped for the whole wave otherwise.
        float mnew[G];
        bool raise = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float bm = s[0][h];
#pragma unroll
          for (int x = 1; x < NL; ++x) bm = fmaxf(bm, s[x][h]);
          mnew[h] = fmaxf(m[h], bm * c_log2);
          raise |= mnew[h] > m[h];
        }
        if (__ballot(raise) != 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float alpha = fast_exp2(m[h] - mnew[h]);
            m[h] = mnew[h];
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
          }
        }
#pragma unroll
        for (int x = 0; x < NL; ++x) {
          float vf[EPL];
          unpack16<T, EPL>(t.v[x], vf);
          if constexpr (PARTIAL) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vf[e] = valid[x] ? vf[e] : 0.f;   // select, never multiply poison
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = fast_exp2(fmaf(s[x][h], c_log2, -m[h]));
            l[h] += p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
          }
        }
      };
      auto compute_any = [&](const Tile<NL> &t, int jj) {
        if ((j0 + jj + 1) * kBlockTokens > tok1)
          compute_tile(t, jj, std::true_type{});
        else
          compute_tile(t, jj, std::false_type{});
      };

      // kDecodeStages tiles in flight; the scheduling barriers keep each
      // prefetch ahead of the compute it overlaps.  Out-of-range prefetches
      // re-read the last tile (a cache hit) so the count of outstanding loads
      // is static.
      constexpr int S = kDecodeStages;
      Tile<NL> t[S];
#pragma unroll
      for (int st = 0; st < S - 1; ++st) load_tile(t[st], min(st, nb - 1));
      __builtin_amdgcn_sched_barrier(0);
      for (int jj = 0; jj < nb; jj += S) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
          if (jj + st >= nb) break;
          load_tile(t[(st + S - 1) % S], min(jj + st + S - 1, nb - 1));
          __builtin_amdgcn_sched_barrier(0);
          compute_any(t[st], jj + st);
        }
      }
    }

    // Merge the lane rows' (m, l, acc) states.  Both lanes of a pair combine
    // (lower, upper) in the same order, so every lane row ends with the same
    // bits and the result does not depend on which lane row stores a head.
#pragma unroll
    for (int step = LPR; step < kWave; step <<= 1) {
      const bool upper = (lane & step) != 0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = __shfl_xor(m[h], step);
        const float lo = __shfl_xor(l[h], step);
        const float ma = upper ? mo : m[h], mb = upper ? m[h] : mo;
        const float la = upper ? lo : l[h], lb = upper ? l[h] : lo;
        const float mx = fmaxf(ma, mb);
        const float fa = fast_exp2(ma - mx);
        const float fb = fast_exp2(mb - mx);
        l[h] = la * fa + lb * fb;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float ao = __shfl_xor(acc[h][e], step);
          const float aa = upper ? ao : acc[h][e], ab = upper ? acc[h][e] : ao;
          acc[h][e] = aa * fa + ab * fb;
        }
        m[h] = mx;
      }
    }

    const bool direct = (np_row == 1);
    const int prow = a.multirow ? row : b;
    // A host bound smaller than the truth leaves no room for this partial.
    if (!direct && (a.part_acc == nullptr || part >= a.part_max)) continue;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (r != h % TPL) continue;
      const int hq = hq0 + h;
      if (direct) {
        const float inv = 1.f / l[h];
        const int64_t o = (static_cast<int64_t>(row) * a.num_q_heads + hq) * D + c * EPL;
        if (a.out_bf16) {
          uint32_t w[EPL / 2];
#pragma unroll
          for (int e = 0; e < EPL / 2; ++e)
            w[e] = f32_to_bf16_rne(acc[h][2 * e] * inv) | (f32_to_bf16_rne(acc[h][2 * e + 1] * inv) << 16);
          uint16_t *op = static_cast<uint16_t *>(a.out) + o;
          if constexpr (EPL == 8) {
            *reinterpret_cast<uint4 *>(op) = make_uint4(w[0], w[1], w[2], w[3]);
          } else {
            *reinterpret_cast<uint2 *>(op) = make_uint2(w[0], w[1]);
          }
        } else {
          float *op = static_cast<float *>(a.out) + o;
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4 *>(op + e) =
                make_float4(acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv);
        }
      } else {
        const int64_t pidx = (static_cast<int64_t>(prow) * a.num_q_heads + hq) * a.part_max + part;
        float *pa = a.part_acc + pidx * D + c * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<float4 *>(pa + e) = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
        if (c == 0) *reinterpret_cast<float2 *>(a.part_ml + pidx * 2) = make_float2(m[h], l[h]);
      }
    }
  }
}

// Merge the partitions of each decode row: O = sum_p 2^(m_p - M) acc_p /
// sum_p 2^(m_p - M) l_p, summed in partition order.
template <int D>
__global__ __launch_bounds__(64) void reduce_kernel(AttendArgs a) {
  extern __shared__ float wsh[];
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.num_q_heads;
  const int hq = blockIdx.x - b * a.num_q_heads;
  const SegInfo si = seg_info(a, b);
  if (!si.ok || (!a.multirow && si.n != 1)) return;
  if (a.part_acc == nullptr || num_parts(si.L) <= 1) return;
  const int rows = a.multirow ? si.n : 1;
  constexpr int DPL = D / kWave;
  // grid y spreads a multi-row segment's rows over workgroups
  for (int i = blockIdx.y; i < rows; i += gridDim.y) {
    const int row = si.row0 + i;
    // Row i of the segment has partials for the partitions up to its own
    // position (all of them for a decode row); one partition: written
    // directly by the decode kernel.
    const int np = min(num_parts(si.L - si.n + i + 1), a.part_max);
    if (np <= 1) continue;
    const int prow = a.multirow ? row : b;
    const int64_t base = (static_cast<int64_t>(prow) * a.num_q_heads + hq) * a.part_max;
    const float *ml = a.part_ml + base * 2;
    float mx = -FLT_MAX;
    for (int p = lane; p < np; p += kWave) mx = fmaxf(mx, ml[2 * p]);
    mx = wave_max(mx);
    float lsum = 0.f;
    for (int p = lane; p < np; p += kWave) {
      const float w = fast_exp2(ml[2 * p] - mx);
      wsh[p] = w;
      lsum += w * ml[2 * p + 1];
    }
    lsum = wave_sum(lsum);
    __syncthreads();
    const float *pa = a.part_acc + base * D;
    float o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int p = 0; p < np; ++p) {
      const float w = wsh[p];
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = fmaf(w, pa[static_cast<int64_t>(p) * D + lane + k * kWave], o[k]);
    }
    const float inv = 1.f / lsum;
    const int64_t ob = (static_cast<int64_t>(row) * a.num_q_heads + hq) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const float val = o[k] * inv;
      if (a.out_bf16)
        static_cast<uint16_t *>(a.out)[ob + lane + k * kWave] = static_cast<uint16_t>(f32_to_bf16_rne(val));
      else
        static_cast<float *>(a.out)[ob + lane + k * kWave] = val;
    }
    __syncthreads();
  }
}

template <typename T, int D, int G>
int launch_decode_t(const AttendArgs &a, int64_t items_bound, hipStream_t stream) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * kDecodeWavesPerCU;
  const int64_t grid = items_bound < cap ? items_bound : cap;
  if (grid <= 0) return PKV_OK;
  decode_kernel<T, D, G><<<dim3(static_cast<unsigned>(grid)), dim3(kWave), 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <typename T, int D>
int dispatch_g(const AttendArgs &a, int G, int64_t items_bound, hipStream_t stream) {
  switch (G) {
    case 1: return launch_decode_t<T, D, 1>(a, items_bound, stream);
    case 2: return launch_decode_t<T, D, 2>(a, items_bound, stream);
    case 3: return launch_decode_t<T, D, 3>(a, items_bound, stream);
    case 4: return launch_decode_t<T, D, 4>(a, items_bound, stream);
    case 5: return launch_decode_t<T, D, 5>(a, items_bound, stream);
    case 6: return launch_decode_t<T, D, 6>(a, items_bound, stream);
    case 7: return launch_decode_t<T, D, 7>(a, items_bound, stream);
    case 8: return launch_decode_t<T, D, 8>(a, items_bound, stream);
    default: return PKV_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_decode(const AttendArgs &a, int32_t dtype, int32_t head_dim, int32_t max_context_len, bool need_reduce,
                  int64_t work_waves, int32_t decode_rows, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t parts = (static_cast<int64_t>(max_context_len) + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
  const int64_t rows = a.multirow ? static_cast<int64_t>(a.total_q) : a.num_segments;
  const int64_t items_bound = rows * (parts > 0 ? parts : 1) * a.num_kv_heads;
  int st;
  if (dtype == PKV_I8) {
    const int stages =
        work_waves >= 0 && work_waves < PKV_DECODE_FEW_WAVES ? PKV_DECODE_Q8_STAGES_FEW : PKV_DECODE_Q8_STAGES;
    st = launch_decode_q8(a, head_dim, max_context_len, stages, decode_rows, stream);
  } else if (dtype == PKV_BF16 && !a.multirow && PKV_DECODE_MFMA) {
    const int stages =
        work_waves >= 0 && work_waves < PKV_DECODE_FEW_WAVES ? PKV_DECODE_MFMA_STAGES_FEW : kDecodeMfmaStages;
    st = launch_decode_mfma(a, head_dim, max_context_len, stages, stream);
  } else if (dtype == PKV_BF16) {
    st = head_dim == 128 ? dispatch_g<uint16_t, 128>(a, G, items_bound, stream)
                         : dispatch_g<uint16_t, 64>(a, G, items_bound, stream);
  } else {
    st = head_dim == 128 ? dispatch_g<float, 128>(a, G, items_bound, stream)
                         : dispatch_g<float, 64>(a, G, items_bound, stream);
  }
  // (a whole-context ablation build writes every bf16 decode row directly)
  if (st != PKV_OK || a.part_max <= 1 || !need_reduce ||
      (PKV_DECODE_WHOLE_CONTEXT && dtype == PKV_BF16 && !a.multirow && PKV_DECODE_MFMA))
    return st;
  // x: (segment, query head); y: rows of multi-row segments (one each up to
  // 65535, then strided)
  const unsigned grid = static_cast<unsigned>(a.num_segments) * static_cast<unsigned>(a.num_q_heads);
  const unsigned grid_rows = a.multirow ? static_cast<unsigned>(std::min(std::max(a.max_query, 1), 65535)) : 1u;
  const size_t lds = static_cast<size_t>(a.part_max) * sizeof(float);
  if (head_dim == 128)
    reduce_kernel<128><<<dim3(grid, grid_rows), dim3(kWave), lds, stream>>>(a);
  else
    reduce_kernel<64><<<dim3(grid, grid_rows), dim3(kWave), lds, stream>>>(a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
