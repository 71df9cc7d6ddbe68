// Decode rows (bf16 pool) with the per-tile products on MFMA.
//
// Same work as the decode kernel in decode.hip - one wavefront per (decode
// row, KV head g, split-context partition), all G query heads of the group
// sharing every K/V tile read, online softmax, partition partials merged by
// the reduce kernel - but each 16-token tile is handled as two small dense
// contractions so the vector ALU is left nearly idle and the wave only waits
// on memory ("Continuous batching: Qwen3.8-27B at 301 tok/s ...", lucebox
// blog, §Paged KV and paged attention: walk the block table in logical order
// over the shared pool, no gather):
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, 1
//     KiB per instruction, nontemporal), kDecodeMfmaStages tiles in flight; the
//     16-byte chunks of each token row are XOR-swizzled so that the reads
//     below are free of bank conflicts;
//   * S^T[token][head] = K Q^T on v_mfma_f32_16x16x32_bf16 (heads are the 16
//     columns, G of them used): lane owns head lane % 16, tokens
//     4 (lane / 16) .. + 3;
//   * online softmax on those values: the tile max needs two cross-row
//     shuffles, the running sum (of the bf16-rounded weights the PV product
//     consumes) stays per lane until the end;
//   * O^T[dim][head] += V^T P^T on v_mfma_f32_16x16x16_bf16, V^T read with
//     ds_read_b64_tr_b16 straight from the [token][dim] tile, P^T straight
//     from the S^T accumulator (P rounded to bf16, as for any bf16 MFMA).
#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned lds_addr(const unsigned char *p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p)));
}

__device__ __forceinline__ shortx4_t lds_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t *)(p));
}

template <int D>
struct MGeo {
  static constexpr int kRowBytes = D * 2;                    // one token row of one head
  static constexpr int kCPR = kRowBytes / 16;                // 16-byte chunks per row
  static constexpr int kTile = kBlockTokens * kRowBytes;     // bytes of a K (or V) tile
  static constexpr int kLoads = kTile / 1024;                // 1 KiB direct-to-LDS loads per tile
  static constexpr int kKSteps = D / 32;
  static constexpr int kDTiles = D / 16;
  // Position of chunk c of token row t inside the row (bank-conflict-free
  // for the K operand reads and the transposed V reads).
  static __device__ __forceinline__ int swz(int t, int c) {
    if constexpr (D == 128) return c ^ (((t & 7) << 1) | ((t >> 3) & 1));
    else return c ^ ((((t >> 1) & 3) << 1) | ((t >> 3) & 1));
  }
};

// Ablation builds only (both 0 in the library): kNoShare gives every query
// head its own wavefront, which reads the group's K/V tiles again (GQA
// sharing off); kWholeContext walks each row's whole context in one
// wavefront (split-context partitions off; the block table is then read in
// slices of 64 entries).
constexpr bool kNoShare = PKV_DECODE_NO_GQA_SHARE;
constexpr bool kWholeContext = PKV_DECODE_WHOLE_CONTEXT;

__device__ __forceinline__ int num_parts_m(int L) {
  return kWholeContext ? 1 : (L + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
}

__device__ __forceinline__ int decode_units(const AttendArgs &a, int b, int G) {
  const SegInfo s = seg_info(a, b);
  return s.ok && s.n == 1 ? num_parts_m(s.L) * (kNoShare ? G : 1) : 0;
}

template <int D, int S>
__global__ __launch_bounds__(64, kDecodeMfmaMinWaves) void decode_mfma_kernel(AttendArgs a, int G) {
  using M = MGeo<D>;
  static_assert(S >= 1 && S <= 3, "1 to 3 tiles in flight");
  constexpr int PT = kDecodePartitionTokens;
  // One LDS array per stage and per K/V so the compiler can tell the
  // in-flight tile loads apart from the tile being read.
  __shared__ __align__(16) unsigned char k0[M::kTile], v0[M::kTile];
  __shared__ __align__(16) unsigned char k1[S > 1 ? M::kTile : 16], v1[S > 1 ? M::kTile : 16];
  __shared__ __align__(16) unsigned char k2[S > 2 ? M::kTile : 16], v2[S > 2 ? M::kTile : 16];
  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const SegInfo mine = seg_info(a, lane);
  const int u0 = mine.ok && mine.n == 1 ? num_parts_m(mine.L) * (kNoShare ? G : 1) : 0;
  const int incl0 = wave_inclusive_scan(u0);
  int total = __shfl(incl0, kWave - 1);
  if (a.num_segments > kWave) total = count_units(a.num_segments, [&](int b) { return decode_units(a, b, G); });
  const int64_t items = static_cast<int64_t>(total) * a.num_kv_heads;
  const float c_log2 = a.scale_log2;

  for (int64_t f = blockIdx.x; f < items; f += gridDim.x) {
    const int unit = static_cast<int>(f / a.num_kv_heads);
    const int g = static_cast<int>(f - static_cast<int64_t>(unit) * a.num_kv_heads);
    int b, part;
    SegInfo si;
    if (unit < __shfl(incl0, kWave - 1)) {
      const unsigned long long mask = __ballot(incl0 > unit);
      b = __ffsll(static_cast<long long>(mask)) - 1;
      part = unit - (__shfl(incl0, b) - __shfl(u0, b));
      si.slot = __builtin_amdgcn_readlane(mine.slot, b);
      si.L = __builtin_amdgcn_readlane(mine.L, b);
      si.n = 1;
      si.row0 = __builtin_amdgcn_readlane(mine.row0, b);
      si.ok = true;
    } else {
      b = find_unit(a.num_segments, unit, [&](int bb) { return decode_units(a, bb, G); }, &part);
      si = seg_info(a, b);
      if (!si.ok) continue;
    }
    int hsel = 0;                            // kNoShare: this wavefront's query head of the group
    if constexpr (kNoShare) {
      hsel = part % G;
      part /= G;
    }
    const int np = num_parts_m(si.L);
    const int row = si.row0;
    const int tok0 = kWholeContext ? 0 : part * PT;
    const int tok1 = kWholeContext ? si.L : min(si.L, tok0 + PT);
    const int j0 = tok0 / kBlockTokens;
    const int nb = (tok1 + kBlockTokens - 1) / kBlockTokens - j0;
    const int head = kNoShare ? hsel : l16;  // MFMA column = query head of the group
    const bool hv = kNoShare ? l16 == 0 : head < G;
    const int hq = g * G + (hv ? head : 0);

    int phys_lane = 0;
    int slice = 0;                           // kWholeContext: the 64-entry table slice held
    auto load_slice = [&](int sl) {
      phys_lane = 0;
      if (lane + sl * kWave < nb) {
        phys_lane = a.block_tables[static_cast<int64_t>(si.slot) * a.max_blocks + j0 + sl * kWave + lane];
        phys_lane = min(max(phys_lane, 0), a.num_blocks - 1);
      }
    };
    load_slice(0);
    // Q^T operand: lane holds dims 32 kk + 8 lg .. + 7 of its head.
    bf16x8_t qb[M::kKSteps];
    {
      const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                        (static_cast<int64_t>(row) * a.num_q_heads + hq) * D);
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) {
        const uint4 w = hv ? qp[kk * 4 + lg] : make_uint4(0, 0, 0, 0);
        qb[kk] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // Per-lane source offsets of the direct-to-LDS loads: load x of a tile
    // fills LDS chunk x * 64 + lane = (row t, position p) with chunk
    // swz^-1 = p ^ f(t) of that row.
    int src_off[M::kLoads];
#pragma unroll
    for (int x = 0; x < M::kLoads; ++x) {
      const int P = x * kWave + lane;
      const int t = P / M::kCPR;
      const int p = P - t * M::kCPR;
      src_off[x] = t * M::kRowBytes + M::swz(t, p) * 16;
    }
    const char *kbase = static_cast<const char *>(a.k);
    const char *vbase = static_cast<const char *>(a.v);
    // The loads are issued as inline assembly: M0 takes the LDS destination
    // (nothing else in this kernel uses M0), and the compiler, which cannot
    // tell the tile in flight from the tile being read, does not wait on them
    // - the explicit s_waitcnt counts below do.
    auto issue = [&](int stage, int jj) {
      if constexpr (kWholeContext) {
        if ((jj >> 6) != slice) {
          slice = jj >> 6;
          load_slice(slice);
          // drains the tile loads too, so every count below stays exact
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        jj &= kWave - 1;
      }
      const int phys = __builtin_amdgcn_readlane(phys_lane, jj);
      const int64_t off = (static_cast<int64_t>(phys) * a.num_kv_heads + g) * M::kTile;
      unsigned char *kd = stage == 0 ? k0 : (stage == 1 ? k1 : k2);
      unsigned char *vd = stage == 0 ? v0 : (stage == 1 ? v1 : v2);
#pragma unroll
      for (int x = 0; x < M::kLoads; ++x) {
        const unsigned ldsk = lds_addr(kd + x * 1024);
        const unsigned ldsv = lds_addr(vd + x * 1024);
        const void *gk = kbase + off + src_off[x];
        const void *gv = vbase + off + src_off[x];
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT
                     ::"s"(ldsk), "v"(gk) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT
                     ::"s"(ldsv), "v"(gv) : "memory");
      }
    };

    // Q and the table slice must have landed before the tile loads start:
    // the compiler does not see those, so it could not place this wait later
    // without waiting on every tile in flight.  (vmcnt(0); expcnt and lgkmcnt
    // left at their maxima.)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    float m_run = -FLT_MAX, l_run = 0.f;
    floatx4_t o[M::kDTiles];
#pragma unroll
    for (int dt = 0; dt < M::kDTiles; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // A landed tile's operands go to registers first, so that its stage can
    // be refilled before the tile's arithmetic: K (lane holds key l16, dims
    // 32 kk + 8 lg .. + 7) and V^T (lane i of each 16-lane group points at
    // row 4 lg + i / 4, dims 16 dt + 4 (i % 4); it receives rows
    // 4 lg .. + 3 of dim 16 dt + i).
    const int vt_row = lg * 4 + (l16 >> 2);
    auto read_tile = [&](const unsigned char *kt, const unsigned char *vt, bf16x8_t(&ka)[M::kKSteps],
                         shortx4_t(&va)[M::kDTiles]) {
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk)
        ka[kk] = *reinterpret_cast<const bf16x8_t *>(kt + l16 * M::kRowBytes + M::swz(l16, kk * 4 + lg) * 16);
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        const int dd = dt * 16 + 4 * (l16 & 3);
        va[dt] = lds_tr16(vt + vt_row * M::kRowBytes + M::swz(vt_row, dd >> 3) * 16 + (dd & 7) * 2);
      }
    };
    auto compute = [&](const bf16x8_t(&ka)[M::kKSteps], shortx4_t(&va)[M::kDTiles], int jj, auto partial_tag) {
      constexpr bool PARTIAL = decltype(partial_tag)::value;
      const int tokbase = (j0 + jj) * kBlockTokens;
      const int valid = tok1 - tokbase;       // tokens of this tile in range (< 16 only if PARTIAL)
      floatx4_t s = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qb[kk], s, 0, 0, 0);
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ok[e] = !PARTIAL || lg * 4 + e < valid;
      if constexpr (PARTIAL) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = ok[e] ? s[e] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run, mx * c_log2);
      if (__ballot(mnew > m_run) != 0) {
        const float alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < M::kDTiles; ++dt) o[dt] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[e], c_log2, -m_run));
      const bf16x4_t pb = bf16x4_t{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]), static_cast<__bf16>(p[2]),
                                   static_cast<__bf16>(p[3])};
      // the row sum adds the bf16 weights the PV product consumes, so that
      // the normalisation matches the numerator
      l_run = add_bf16x4(pb, l_run);
      const shortx4_t pbs = __builtin_bit_cast(shortx4_t, pb);
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        shortx4_t v = va[dt];
        if constexpr (PARTIAL) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = ok[e] ? v[e] : static_cast<short>(0);   // select, never multiply poison
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pbs, o[dt], 0, 0, 0);
      }
    };

    // kDecodeMfmaStages tiles in flight.  Past the last tile the prefetch re-reads
    // the last tile (a cache hit) so every wait below has a static count.
    issue(0, 0);
    if constexpr (S > 1) issue(1, min(1, nb - 1));
    if constexpr (S > 2) issue(2, min(2, nb - 1));
    for (int jj = 0; jj < nb; jj += S) {
#pragma unroll
      for (int st = 0; st < S; ++st) {
        if (jj + st >= nb) break;
        // tile jj + st sits in stage st; wait until its loads have landed
        if constexpr (S == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if constexpr (S == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * M::kLoads) : "memory");
        if constexpr (S == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * M::kLoads) : "memory");
        const unsigned char *kt = st == 0 ? k0 : (st == 1 ? k1 : k2);
        const unsigned char *vt = st == 0 ? v0 : (st == 1 ? v1 : v2);
        bf16x8_t ka[M::kKSteps];
        shortx4_t va[M::kDTiles];
        read_tile(kt, vt, ka, va);
        // every LDS read of the tile has returned: refill its stage with the
        // tile S ahead, then do the tile's arithmetic from registers
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (S > 1) issue(st, min(jj + st + S, nb - 1));
        else if (jj + 1 < nb) issue(0, jj + 1);
        if ((j0 + jj + st + 1) * kBlockTokens > tok1)
          compute(ka, va, jj + st, std::true_type{});
        else
          compute(ka, va, jj + st, std::false_type{});
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Lane groups hold disjoint tokens: combine their sums.
    float lt = l_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (!hv) continue;
    const bool direct = (np == 1);
    if (!direct && (a.part_acc == nullptr || part >= a.part_max)) continue;
    if (direct) {
      const float inv = 1.f / lt;
      const int64_t ob = (static_cast<int64_t>(row) * a.num_q_heads + hq) * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        const floatx4_t v = o[dt] * inv;
        if (a.out_bf16) {
          uint16_t *op = static_cast<uint16_t *>(a.out) + ob + dt * 16;
          *reinterpret_cast<uint2 *>(op) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                      f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
        } else {
          *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + ob + dt * 16) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    } else {
      const int64_t pidx = (static_cast<int64_t>(b) * a.num_q_heads + hq) * a.part_max + part;
      float *pa = a.part_acc + pidx * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt)
        *reinterpret_cast<float4 *>(pa + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (lg == 0) *reinterpret_cast<float2 *>(a.part_ml + pidx * 2) = make_float2(m_run, lt);
    }
  }
}

}  // namespace

template <int D>
int launch_decode_mfma_d(const AttendArgs &a, int G, int64_t grid, int stages, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(kWave);
  if (stages >= 3) decode_mfma_kernel<D, 3><<<g, b, 0, stream>>>(a, G);
  else if (stages == 2) decode_mfma_kernel<D, 2><<<g, b, 0, stream>>>(a, G);
  else decode_mfma_kernel<D, 1><<<g, b, 0, stream>>>(a, G);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int launch_decode_mfma(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, int stages,
                       hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t parts = (static_cast<int64_t>(max_context_len) + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
  const int64_t items_bound = static_cast<int64_t>(a.num_segments) * (parts > 0 ? parts : 1) * a.num_kv_heads;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * kDecodeWavesPerCU;
  const int64_t grid = items_bound < cap ? items_bound : cap;
  if (grid <= 0) return PKV_OK;
  return head_dim == 128 ? launch_decode_mfma_d<128>(a, G, grid, stages, stream)
                         : launch_decode_mfma_d<64>(a, G, grid, stages, stream);
}

}  // namespace pkv
