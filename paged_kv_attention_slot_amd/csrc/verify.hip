// Short multi-row segments (speculative-verify drafts) on a streaming,
// decode-style kernel.
//
// "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog),
// §Packing unequal prompt chunks together: verifying a speculative draft
// needs a score for every proposed row, each row causal at its own position
// over the slot's paged KV.  A draft of n rows with G query heads per KV head
// is n * G (row, head) pairs sharing every K/V token: few enough pairs that
// the work is bound by reading the cache, not by the matrix cores.
//
// The segment's pairs m = i * G + h number at most verify_max_pairs(D): one
// column group of verify_col_tiles(D) 16-wide MFMA tiles (faster, measured,
// than spreading more pairs over several wavefronts that stream the same
// tiles).  One wavefront per (segment, KV head, 512-token partition, column
// group) streams the partition's 16-token K/V tiles through its own
// direct-to-LDS ring (no workgroup barrier) and, per tile:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16, the K operand read once and
//     used for every column tile of the group;
//   * the causal mask (row i sits at L - n + i) only on tiles reaching past
//     the first row's position or the partition's end;
//   * online softmax per pair, the running max allowed to lag by
//     PKV_VERIFY_RESCALE_SLACK before O and l are rescaled; l adds the
//     bf16-rounded weights that the PV product consumes;
//   * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16, V^T read transposed once
//     per output tile and used for every column tile.
// A row with one partition writes its output; otherwise partials (O, m, l)
// go to the workspace and verify_merge_kernel combines the partitions each
// row sees, in partition order.
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

__device__ __forceinline__ unsigned vlds_addr(const unsigned char *p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p)));
}

__device__ __forceinline__ shortx4_t vlds_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t *)(p));
}

template <int D>
struct VGeo {
  static constexpr int kRowBytes = D * 2;                    // one token row of one head
  static constexpr int kCPR = kRowBytes / 16;                // 16-byte chunks per row
  static constexpr int kTile = kBlockTokens * kRowBytes;     // bytes of a K (or V) tile
  static constexpr int kLoads = kTile / 1024;                // 1 KiB direct-to-LDS loads per tile
  static constexpr int kKSteps = D / 32;
  static constexpr int kDTiles = D / 16;
  // Position of chunk c of token row t inside the row: the K operand reads
  // (16 rows, one chunk) and the transposed V reads (4 rows, two chunks) hit
  // distinct banks.
  static __device__ __forceinline__ int swz(int t, int c) {
    if constexpr (D == 128) return c ^ (((t & 7) << 1) | ((t >> 3) & 1));
    else return c ^ ((((t >> 1) & 3) << 1) | ((t >> 3) & 1));
  }
};

constexpr int kVPT = kVerifyPartitionTokens;

__device__ __forceinline__ int vnum_parts(int L) { return (L + kVPT - 1) / kVPT; }

template <int NC>
__device__ __forceinline__ int vgroups(int n, int G) {
  return (n * G + NC * 16 - 1) / (NC * 16);
}

template <int D, int NC>
__device__ __forceinline__ int verify_units_of(const SegInfo &s, int G) {
  return s.ok && verify_segment(s.n, G, D) ? vnum_parts(s.L) * vgroups<NC>(s.n, G) : 0;
}

// Rows of segment b in the verify partials (all of a verify segment's rows).
template <int D>
__device__ __forceinline__ int verify_partial_rows_of(const SegInfo &s, int G) {
  return s.ok && verify_segment(s.n, G, D) ? s.n : 0;
}

// NC: 16-wide pair tiles per wavefront (the launch takes the fewest that hold
// its largest segment); S: K/V tiles in flight per wavefront.  Neither
// changes the arithmetic of any pair.
template <int D, int NC, int S>
__global__ __launch_bounds__(64, NC == 1 ? 3 : 2) void verify_kernel(AttendArgs a, int G) {
  using M = VGeo<D>;
  static_assert(NC >= 1 && NC <= verify_col_tiles(D) && S >= 1 && S <= 3, "verify geometry");
  __shared__ __align__(16) unsigned char kst[S][M::kTile];
  __shared__ __align__(16) unsigned char vst[S][M::kTile];
  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const float c_log2 = a.scale_log2;

  const auto map = make_unit_map(a, [&](const SegInfo &s) { return verify_units_of<D, NC>(s, G); },
                                 [&](const SegInfo &s) { return verify_partial_rows_of<D>(s, G); });
  const int64_t items = static_cast<int64_t>(map.total) * a.num_kv_heads;

  for (int64_t f = blockIdx.x; f < items; f += gridDim.x) {
    const int unit = static_cast<int>(f / a.num_kv_heads);
    const int g = static_cast<int>(f - static_cast<int64_t>(unit) * a.num_kv_heads);
    const UnitPlace place = map.place(unit);
    const int u = place.rest;
    const SegInfo si = place.si;
    if (!si.ok) continue;
    const int ngr = vgroups<NC>(si.n, G);
    const int part = u / ngr;
    const int cg = u - part * ngr;
    const int np = vnum_parts(si.L);
    const int pairs = si.n * G;
    const int tok0 = part * kVPT;
    const int tok1 = min(si.L, tok0 + kVPT);
    const int j0 = tok0 / kBlockTokens;
    const int nb = (tok1 + kBlockTokens - 1) / kBlockTokens - j0;
    const int first_pos = si.L - si.n;          // position of row 0
    // first row of this segment in the verify partials (uniform)
    const int64_t vrow0 = np > 1 ? place.slots_before : 0;

    // Column tile c of this group: pair m = (cg * NC + c) * 16 + l16.
    int pos[NC];
    bool pv[NC];
    bf16x8_t qb[NC][M::kKSteps];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int m = (cg * NC + c) * 16 + l16;
      pv[c] = m < pairs;
      const int i = pv[c] ? m / G : 0;
      const int h = pv[c] ? m - i * G : 0;
      pos[c] = pv[c] ? first_pos + i : -1;
      const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                        (static_cast<int64_t>(si.row0 + i) * a.num_q_heads + g * G + h) * D);
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) {
        const uint4 w = pv[c] ? qp[kk * 4 + lg] : make_uint4(0, 0, 0, 0);
        qb[c][kk] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // (a column tile of the group past the segment's pairs has zero Q and
    // is computed anyway: no branches inside the tile loop)

    int phys_lane = 0;
    if (lane < nb) {
      phys_lane = a.block_tables[static_cast<int64_t>(si.slot) * a.max_blocks + j0 + lane];
      phys_lane = min(max(phys_lane, 0), a.num_blocks - 1);
    }
    // Load x of a tile fills LDS chunk x * 64 + lane = (row t, position p)
    // with chunk swz^-1 = p ^ f(t) of that row.
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
    // Inline-assembly loads (M0 takes the LDS destination; nothing else here
    // uses M0): the compiler does not wait on them, the explicit vmcnt waits
    // below do.
    auto issue = [&](int stage, int jj) {
      const int phys = __builtin_amdgcn_readlane(phys_lane, jj);
      const int64_t off = (static_cast<int64_t>(phys) * a.num_kv_heads + g) * M::kTile;   // scalar
      const char *gk = kbase + off;
      const char *gv = vbase + off;
#pragma unroll
      for (int x = 0; x < M::kLoads; ++x) {
        const unsigned ldsk = vlds_addr(&kst[stage][x * 1024]);
        const unsigned ldsv = vlds_addr(&vst[stage][x * 1024]);
        const unsigned lo = static_cast<unsigned>(src_off[x]);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 " PKV_VERIFY_DMA_HINT
                     ::"s"(ldsk), "v"(lo), "s"(gk) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 " PKV_VERIFY_DMA_HINT
                     ::"s"(ldsv), "v"(lo), "s"(gv) : "memory");
      }
    };
    // Q and the table slice have landed before any tile load (vmcnt(0);
    // expcnt and lgkmcnt left at their maxima).
    __builtin_amdgcn_s_waitcnt(0x0F70);

    float m_run[NC], l_run[NC];
    floatx4_t o[NC][M::kDTiles];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      m_run[c] = -FLT_MAX;
      l_run[c] = 0.f;
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) o[c][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }

    // A landed tile's operands go to registers first, so that its stage can
    // be refilled before the tile's arithmetic: K (lane holds key l16, dims
    // 32 kk + 8 lg .. + 7) and V^T (lane i of each 16-lane group points at
    // row 4 lg + i / 4, dims 16 dt + 4 (i % 4); it receives rows
    // 4 lg .. + 3 of dim 16 dt + i).
    const int vt_row = lg * 4 + (l16 >> 2);
    auto read_tile = [&](int stage, bf16x8_t(&ka)[M::kKSteps], shortx4_t(&va)[M::kDTiles]) {
      const unsigned char *kt = kst[stage];
      const unsigned char *vt = vst[stage];
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk)
        ka[kk] = *reinterpret_cast<const bf16x8_t *>(kt + l16 * M::kRowBytes + M::swz(l16, kk * 4 + lg) * 16);
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        const int dd = dt * 16 + 4 * (l16 & 3);
        va[dt] = vlds_tr16(vt + vt_row * M::kRowBytes + M::swz(vt_row, dd >> 3) * 16 + (dd & 7) * 2);
      }
    };
    auto compute = [&](const bf16x8_t(&ka)[M::kKSteps], const shortx4_t(&va)[M::kDTiles], int jj, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int tokbase = (j0 + jj) * kBlockTokens;
      floatx4_t s[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) s[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) {
#pragma unroll
        for (int c = 0; c < NC; ++c) s[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qb[c][kk], s[c], 0, 0, 0);
      }
      // lane holds tokens tokbase + 4 lg + e of pair column l16
      bool tv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) tv[e] = !MASKED || tokbase + lg * 4 + e < tok1;
      shortx4_t pbs[NC];
      bool raise = false;
      float mnew[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (MASKED) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!tv[e] || tokbase + lg * 4 + e > pos[c]) s[c][e] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(s[c][0], s[c][1]), fmaxf(s[c][2], s[c][3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= c_log2;
        mnew[c] = fmaxf(m_run[c], mx);
        raise |= mx > m_run[c] + PKV_VERIFY_RESCALE_SLACK;
      }
      if (__ballot(raise) != 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float alpha = fast_exp2(m_run[c] - mnew[c]);
          m_run[c] = mnew[c];
          l_run[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < M::kDTiles; ++dt) o[c][dt] *= alpha;
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[c][e], c_log2, -m_run[c]));
        const bf16x4_t pb = bf16x4_t{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                                     static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
        l_run[c] = add_bf16x4(pb, l_run[c]);     // the weights the PV product consumes
        pbs[c] = __builtin_bit_cast(shortx4_t, pb);
      }
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        shortx4_t v = va[dt];
        if constexpr (MASKED) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = tv[e] ? v[e] : static_cast<short>(0);   // select, never multiply poison
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pbs[c], o[c][dt], 0, 0, 0);
      }
    };

    // S tiles in flight; past the last tile the prefetch re-reads the last
    // tile (a cache hit) so every wait has a static count.  One tile per
    // iteration, its stage chosen at run time (the loop is kept rolled to
    // hold the register budget).
#pragma unroll
    for (int st = 0; st < S; ++st) issue(st, min(st, nb - 1));
    auto step = [&](int jj, auto masked_tag) {
      const int st = jj % S;
      // tile jj sits in stage st: landed once at most S - 1 newer tiles'
      // loads are outstanding
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * M::kLoads * (S - 1)) : "memory");
      bf16x8_t ka[M::kKSteps];
      shortx4_t va[M::kDTiles];
      read_tile(st, ka, va);
      // every LDS read of the tile has returned: refill its stage, then do
      // the tile's arithmetic from registers
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(st, min(jj + S, nb - 1));
      compute(ka, va, jj, masked_tag);
    };
    // Tiles needing no mask (wholly before tok1 and before the first row's
    // position) come first: a loop of those, then the masked rest, so that
    // neither loop branches per tile.
    const int unmasked = max(0, min(nb, min(tok1, first_pos + 1) / kBlockTokens - j0));
    int jj = 0;
#pragma unroll 1
    for (; jj < unmasked; ++jj) step(jj, std::false_type{});
#pragma unroll 1
    for (; jj < nb; ++jj) step(jj, std::true_type{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Lane groups hold disjoint tokens: combine their sums, then store.
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float lt = l_run[c];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      if (!pv[c]) continue;
      const int m = (cg * NC + c) * 16 + l16;
      const int i = m / G;
      const int qrow = si.row0 + i;
      const int qhead = g * G + (m - i * G);
      if (np == 1) {
        const float inv = 1.f / lt;
        const int64_t ob = (static_cast<int64_t>(qrow) * a.num_q_heads + qhead) * D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < M::kDTiles; ++dt) {
          const floatx4_t v = o[c][dt] * inv;
          if (a.out_bf16) {
            uint16_t *op = static_cast<uint16_t *>(a.out) + ob + dt * 16;
            *reinterpret_cast<uint2 *>(op) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                        f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
          } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + ob + dt * 16) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      } else {
        if (a.verify_acc == nullptr || part >= a.part_max || vrow0 + si.n > a.verify_rows) continue;
        const int64_t prow = vrow0 + i;
        const int64_t pidx = (prow * a.num_q_heads + qhead) * a.part_max + part;
        float *pa = a.verify_acc + pidx * D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < M::kDTiles; ++dt)
          *reinterpret_cast<float4 *>(pa + dt * 16) = make_float4(o[c][dt][0], o[c][dt][1], o[c][dt][2], o[c][dt][3]);
        if (lg == 0) *reinterpret_cast<float2 *>(a.verify_ml + pidx * 2) = make_float2(m_run[c], lt);
      }
    }
  }
}

// Merge the partitions of every row of a split verify segment: row i sees
// partitions 0 .. (L - n + i) / 512; combined in partition order.  One
// wavefront per (segment, query head, row of the segment).
template <int D>
__global__ __launch_bounds__(64) void verify_merge_kernel(AttendArgs a, int G, int grid_rows) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / grid_rows;              // grid_rows: rows the longest verify segment has
  const int i = blockIdx.x - bh * grid_rows;
  const int b = bh / a.num_q_heads;
  const int hq = bh - b * a.num_q_heads;
  const SegInfo si = seg_info(a, b);
  if (!si.ok || !verify_segment(si.n, G, D) || a.verify_acc == nullptr || i >= si.n) return;
  if (vnum_parts(si.L) <= 1) return;
  const int64_t vrow0 = units_before(b, [&](int bb) { return verify_partial_rows_of<D>(seg_info(a, bb), G); });
  if (vrow0 + si.n > a.verify_rows) return;
  constexpr int DPL = D / kWave;
  const int pos = si.L - si.n + i;
  const int np = min(pos / kVPT + 1, a.part_max);
  const int64_t base = ((vrow0 + i) * a.num_q_heads + hq) * a.part_max;
  const float *ml = a.verify_ml + base * 2;
  float mx = -FLT_MAX;
  for (int p = lane; p < np; p += kWave) mx = fmaxf(mx, ml[2 * p]);
  mx = wave_max(mx);
  float lsum = 0.f;
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float2 mp = *reinterpret_cast<const float2 *>(ml + 2 * p);
    const float w = fast_exp2(mp.x - mx);
    lsum = fmaf(w, mp.y, lsum);
    const float *pa = a.verify_acc + (base + p) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, pa[lane + k * kWave], acc[k]);
  }
  const float inv = 1.f / lsum;
  const int64_t ob = (static_cast<int64_t>(si.row0 + i) * a.num_q_heads + hq) * D;
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float v = acc[k] * inv;
    if (a.out_bf16)
      static_cast<uint16_t *>(a.out)[ob + lane + k * kWave] = static_cast<uint16_t>(f32_to_bf16_rne(v));
    else
      static_cast<float *>(a.out)[ob + lane + k * kWave] = v;
  }
}

}  // namespace

template <int D, int NC>
void launch_verify_nc(const AttendArgs &a, int G, unsigned grid, bool deep, hipStream_t stream) {
  if (deep) verify_kernel<D, NC, 3><<<dim3(grid), dim3(kWave), 0, stream>>>(a, G);
  else verify_kernel<D, NC, PKV_VERIFY_SHALLOW_STAGES><<<dim3(grid), dim3(kWave), 0, stream>>>(a, G);
}

int launch_verify(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, bool need_merge,
                  int32_t max_pairs, int64_t work_waves, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nc_max = verify_col_tiles(head_dim);
  int nc = max_pairs > 0 ? (max_pairs + 15) / 16 : nc_max;
  nc = nc < 1 ? 1 : (nc > nc_max ? nc_max : nc);
  const int64_t parts = (static_cast<int64_t>(max_context_len) + kVPT - 1) / kVPT;
  const int64_t groups = (verify_max_pairs(head_dim) + nc * 16 - 1) / (nc * 16);
  const int64_t items_bound = static_cast<int64_t>(a.num_segments) * (parts > 0 ? parts : 1) * groups * a.num_kv_heads;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * kDecodeWavesPerCU;
  const int64_t grid = items_bound < cap ? items_bound : cap;
  if (grid <= 0) return PKV_OK;
  const bool deep = work_waves >= 0 && work_waves < PKV_DECODE_FEW_WAVES;
  const unsigned g = static_cast<unsigned>(grid);
  if (head_dim == 128) {
    if (nc == 1) launch_verify_nc<128, 1>(a, G, g, deep, stream);
    else launch_verify_nc<128, 2>(a, G, g, deep, stream);
  } else {
    if (nc == 1) launch_verify_nc<64, 1>(a, G, g, deep, stream);
    else if (nc == 2) launch_verify_nc<64, 2>(a, G, g, deep, stream);
    else launch_verify_nc<64, 3>(a, G, g, deep, stream);
  }
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (!need_merge || a.verify_acc == nullptr || a.part_max <= 1) return PKV_OK;
  // One workgroup per (segment, head, row) up to the most rows a verify
  // segment of this launch has (from the host's pair count when known).
  int grid_rows = verify_rows_cap(G, head_dim);
  if (max_pairs > 0 && (max_pairs + G - 1) / G < grid_rows) grid_rows = (max_pairs + G - 1) / G;
  const int64_t mgrid = static_cast<int64_t>(a.num_segments) * a.num_q_heads * grid_rows;
  if (mgrid <= 0) return PKV_OK;
  if (mgrid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  if (head_dim == 128)
    verify_merge_kernel<128><<<dim3(static_cast<unsigned>(mgrid)), dim3(kWave), 0, stream>>>(a, G, grid_rows);
  else
    verify_merge_kernel<64><<<dim3(static_cast<unsigned>(mgrid)), dim3(kWave), 0, stream>>>(a, G, grid_rows);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
