// Multi-row segments (prompt chunks, speculative drafts) on MFMA tiles: bf16
// pools directly, 8-bit pools through fp16 tiles converted in LDS (the
// "8-bit pools" section below).
//
// "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog):
// §Chunked prefill is a slot phase - a prompt advances by a bounded chunk
// per step, appended straight into the slot's paged KV; §Packing unequal
// prompt chunks together - per-query causal positions and block-table
// metadata let chunk rows and decode rows attend over the shared pool in one
// pass (speculative drafts need scores for every proposed row too).
//
// Row i of a segment with n rows and L cached tokens sits at position
// L - n + i and sees keys 0 .. L - n + i.  The contraction is dense, so it
// runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation of the exact bf16
// Q and K (the softmax scale multiplies each fp32 score):
//   * "M-rows" are (query row, head of the GQA group) pairs, m = i * G + h;
//     a workgroup of 4 wavefronts takes 128 consecutive M-rows of one
//     segment and one KV head, so all G query heads share every K/V tile;
//     a wavefront's 32 M-rows are one 32-wide MFMA column tile;
//   * K/V tiles (4 or 2 pool blocks, fetched through the block table) are
//     staged in LDS once per workgroup;
//   * scores are formed transposed, S^T = K Q^T: lane l owns M-row l % 32,
//     and its half h = l / 32 holds 16 of every 32 keys (accumulator element
//     e is key 8 (e / 4) + 4 h + e % 4), so a row max is one reduction over
//     the lane's scores and one swap with lane l ^ 32;
//   * the output is formed as O^T += V^T P^T.  P^T comes straight from the
//     accumulators: the 16 keys of PV step s are elements 8 (s % 2) .. + 7
//     of 32-key tile s / 2, i.e. keys 16 s + 4 h + {0..3} and
//     16 s + 8 + 4 h + {0..3} for half h.  V^T is two ds_read_b64_tr_b16
//     reads of exactly those keys from the natural [token][dim] tile (lane j
//     of each 16-lane group receives 4 consecutive keys of dimension j);
//   * row sums add the bf16 weights the products consume (v_dot2_f32_bf16
//     against (1, 1)); the two halves' sums are added at the end;
//   * the causal mask is applied per element only on tiles that reach past a
//     wavefront's first row; rows of a segment never see past their position.
#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

// Multi-row segments of 8-bit pools on the chunk kernel's 8-bit form (0: on
// the 8-bit decode kernel, column group by column group).
#ifndef PKV_CHUNK_Q8
#define PKV_CHUNK_Q8 1
#endif
// The 8-bit form's fp16 tiles hold the codes themselves (1: the constant
// 1152 comes off each converted pair in fp16, exactly) or 1152 + code (0:
// the constant comes off every score and off O at the end).
#ifndef PKV_CHUNK_Q8_EXACT_CODES
#define PKV_CHUNK_Q8_EXACT_CODES 1
#endif

// Unmasked tiles four at a time (one turn of the 4-stage ring), so that each
// tile's stage, and with it every LDS address of the tile, is a constant.
#ifndef PKV_CHUNK_STATIC_STAGES
#define PKV_CHUNK_STATIC_STAGES 1
#endif

// K and V of a tile refilled at different iterations: a tile's K is read one
// iteration before its V (the next tile's scores are formed while the current
// tile's weights are), so its K slot frees an iteration earlier.  Refilling
// each slot as soon as it frees loads K one tile further ahead with the same
// LDS (0: both slots of a stage refilled together).
#ifndef PKV_CHUNK_SPLIT_RING
#define PKV_CHUNK_SPLIT_RING 0
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Transposed LDS read: with lane i of a 16-lane group pointing at
// tile[t0 + i / 4][d0 + 4 (i % 4)], lane j receives tile[t0 .. t0 + 3][d0 + j].
__device__ __forceinline__ shortx4_t lds_read_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t *)(p));
}


// IEEE-754 maximum (NaN-propagating): lowers to v_maximum3_f32 / v_maximum_f32
// with no canonicalisation of matrix-core results, unlike fmaxf.
__device__ __forceinline__ float vmaxf(float a, float b) { return __builtin_elementwise_maximum(a, b); }

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;                 // one 32-wide MFMA column tile
constexpr int kMTile = kWaves * kRowsPerWave;    // M-rows per workgroup
constexpr int kKV = 64;                          // tokens per K/V tile
constexpr int kTableWindow = PKV_CHUNK_TABLE_WINDOW;   // block-table entries staged per pass

// Key-range splits of a segment: segments with few row tiles (speculative
// drafts, short chunks) would leave most compute units idle, so their keys
// are cut into `splits` ranges of whole 64-token tiles, each its own
// workgroup, merged afterwards in split order.  The count depends only on
// the segment's own (n, L, G), never on the rest of the batch.
struct ChunkShape {
  int mtiles;      // 128-row tiles of (query row, head) pairs
  int splits;      // key ranges
  int tps;         // 64-token K/V tiles per range
};

template <int D>
__host__ __device__ __forceinline__ ChunkShape chunk_shape(int n, int L, int G) {
  ChunkShape c;
  c.mtiles = (n * G + kMTile - 1) / kMTile;
  const int kv_tiles = (L + kKV - 1) / kKV;
  constexpr int kRT = chunk_split_row_tiles(D);
  int splits = c.mtiles >= kRT ? 1 : kRT / c.mtiles;
  constexpr int kMin = PKV_CHUNK_MIN_TILES_PER_SPLIT;
  const int by_len = (kv_tiles + kMin - 1) / kMin;              // at least kMin K/V tiles per range
  splits = splits < by_len ? splits : by_len;
  splits = splits > 1 ? splits : 1;
  c.tps = (kv_tiles + splits - 1) / splits;
  c.splits = (kv_tiles + c.tps - 1) / c.tps;
  return c;
}

template <int D>
__device__ __forceinline__ int chunk_units_of(const SegInfo &s, int G) {
  if (!s.ok || s.n < 2 || verify_segment(s.n, G, D)) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.mtiles * c.splits;
}

// Partial slots (per KV head) of a segment: one per (M-row, key range) when
// the segment is cut into key ranges, else none.
template <int D>
__device__ __forceinline__ int chunk_partial_slots_of(const SegInfo &s, int G) {
  if (!s.ok || s.n < 2 || verify_segment(s.n, G, D)) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.splits > 1 ? s.n * G * c.splits : 0;
}

// LDS ring of K/V tiles fed by direct-to-LDS loads: kRingTok tokens per
// stage, kRingStages stages (64 KiB or less per workgroup so two fit a CU).
template <int D>
struct Ring;
template <>
struct Ring<64> {
  static constexpr int kTok = PKV_CHUNK_RING_TOK_D64, kStages = PKV_CHUNK_RING_STAGES_D64;
  static constexpr int kMinWaves = PKV_CHUNK_MIN_WAVES_D64;
  static constexpr bool kEarlyV = PKV_CHUNK_EARLY_V_D64;
};
template <>
struct Ring<128> {
  static constexpr int kTok = PKV_CHUNK_RING_TOK_D128, kStages = PKV_CHUNK_RING_STAGES_D128;
  static constexpr int kMinWaves = PKV_CHUNK_MIN_WAVES_D128;
  static constexpr bool kEarlyV = PKV_CHUNK_EARLY_V_D128;
};

// Position of 16-byte chunk c of token row t within the row, so that both the
// K operand reads (consecutive rows, one chunk) and the transposed V reads
// (4 rows, two chunks) hit distinct banks.
template <int D>
__device__ __forceinline__ int ring_swz(int t, int c) {
  if constexpr (D == 128) return c ^ (((t & 7) << 1) | ((t >> 3) & 1));
  else return c ^ ((((t >> 1) & 3) << 1) | ((t >> 3) & 1));
}

__device__ __forceinline__ unsigned lds_addr32(const unsigned char *p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p)));
}

// acc + the sum of the eight bf16 values of v (pairwise against (1, 1)).
__device__ __forceinline__ float add_bf16_pairs(const bf16x8_t &v, float acc) {
  const bf16x2_t one2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, acc, false);
}

// OFF32: every byte of a pool tensor lies within 4 GiB of its base, so a tile
// load addresses the tensor base (scalar) plus one 32-bit vector offset.
template <int D, bool OFF32>
__global__ __launch_bounds__(256, Ring<D>::kMinWaves) void chunk_kernel(AttendArgs a, int G) {
  constexpr int T = Ring<D>::kTok;            // tokens per ring stage
  constexpr int S = Ring<D>::kStages;
  constexpr int kRowBytes = D * 2;
  constexpr int kCPR = kRowBytes / 16;
  constexpr int kStageBytes = T * kRowBytes;
  constexpr int kPer = T * kCPR / (kWaves * kWave);
  constexpr int kTT = T / 32;                 // 32-token MFMA tiles per stage
  constexpr int kPS = T / 16;                 // 16-key PV steps per stage
  constexpr int kQS = D / 16;                 // 16-dim q . k steps
  constexpr int kDT = D / 32;                 // 32-wide output dimension tiles
  static_assert(kPer >= 1 && T % 32 == 0 && 64 % T == 0, "ring geometry");
  __shared__ __align__(16) unsigned char lds[S * 2 * kStageBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const auto map = make_unit_map(a, [&](const SegInfo &s) { return chunk_units_of<D>(s, G); },
                                 [&](const SegInfo &s) { return chunk_partial_slots_of<D>(s, G); });
  const int hkv = a.num_kv_heads;
  if (static_cast<int64_t>(blockIdx.x) >= static_cast<int64_t>(map.total) * hkv) return;
  const int unit = blockIdx.x / hkv;
  const int g = blockIdx.x - unit * hkv;
  const UnitPlace place = map.place(unit);
  const int u = place.rest;
  const SegInfo si = place.si;
  if (!si.ok) return;
  const int n = si.n, L = si.L;
  const int mtot = n * G;
  const ChunkShape cs = chunk_shape<D>(n, L, G);
  const int mt = cs.mtiles - 1 - u / cs.splits;      // heaviest (latest) rows first
  const int split = u - (cs.mtiles - 1 - mt) * cs.splits;
  const int m0 = mt * kMTile;
  const int mw = m0 + wave * kRowsPerWave;
  const int m_last = min(m0 + kMTile, mtot) - 1;
  const int kv_end = L - n + m_last / G + 1;         // keys any row of the tile sees
  const int rt_begin = split * cs.tps * (kKV / T);
  const int rt_end = min(rt_begin + cs.tps * (kKV / T), (kv_end + T - 1) / T);
  if (rt_begin >= rt_end) return;
  const bool partial_out = cs.splits > 1;
  // tiles nobody else reads in this launch stream past the caches
  const bool stream_tiles = PKV_CHUNK_STREAM_LOADS == 1 || (PKV_CHUNK_STREAM_LOADS == 2 && cs.mtiles == 1);
  // first partial slot of this segment (uniform over the workgroup)
  int64_t part_base = 0;
  if (partial_out) {
    if (a.chunk_part == nullptr) return;
    part_base = place.slots_before;
    if (part_base + static_cast<int64_t>(mtot) * cs.splits > a.chunk_slots) return;   // bounds understated
  }
  const int wave_pos0 = mw < mtot ? L - n + mw / G : -1;
  const bool wave_live = mw < mtot;                  // the wavefront has M-rows of the segment

  // Q operand (B of S^T = K Q^T): lane holds dims 16 ks + 8 hh .. + 7 of
  // its M-row, the query's own bf16 values: the score accumulators hold the
  // raw q . k, and the scale is applied in fp32 to each score.
  const float c_log2 = a.scale_log2;
  const float slack_raw = PKV_CHUNK_RESCALE_SLACK / c_log2;    // the slack in raw score units
  const int m = mw + l32;
  const bool valid = m < mtot;
  const int qi = valid ? m / G : 0;
  const int qh = valid ? m - qi * G : 0;
  const int pos = valid ? L - n + qi : -1;
  const int row = si.row0 + qi;
  const int hq = g * G + qh;
  bf16x8_t qv[kQS];
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                      (static_cast<int64_t>(row) * a.num_q_heads + hq) * D);
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) {
      const uint4 w = valid ? qp[2 * ks + hh] : make_uint4(0, 0, 0, 0);
      qv[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // Online softmax state of the lane's M-row: running max m_run (raw q . k
  // units) and the reference the weights are taken against, ref = m_run x
  // scale log2(e) as one fp32 value (0 before the row has seen a key): a
  // score s weighs exp2(fma(s, scale log2(e), -ref)).  The score
  // accumulators start from zero (the MFMA's inline constant).  lsum: this
  // half's row sum.
  float m_run = -FLT_MAX, ref = 0.f, lsum = 0.f;
  const floatx16_t zero16 = {};
  floatx16_t o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  // Direct-to-LDS staging.  Wavefront w fills token rows w R .. w R + R - 1
  // of each K and V stage (R = T / 4: 16 at D = 64, 8 at D = 128), all inside
  // one pool block: load x covers kRowsW of them, lane l row
  // t = w R + x kRowsW + l / kCPR, position p = l % kCPR, taking chunk
  // ring_swz(t, p) of that row.  So one block lookup per tile serves the
  // wavefront, the 64-bit base is wave-uniform (scalar registers) and each
  // lane adds a fixed 32-bit offset.  Tokens past the sequence read the last
  // token (finite data; their scores are masked and their weights are
  // exactly zero).
  constexpr int kRowsW = kWave / kCPR;              // token rows per load
  constexpr int kR = T / kWaves;                    // token rows per wavefront
  constexpr int kBlockBytes = kBlockTokens * kRowBytes;
  static_assert(kR == kPer * kRowsW && kBlockTokens % kR == 0 && T % kBlockTokens == 0,
                "a wavefront's rows stay inside one block");
  const int32_t *bt = a.block_tables + static_cast<int64_t>(si.slot) * a.max_blocks;
  const char *kbase = static_cast<const char *>(a.k);
  const char *vbase = static_cast<const char *>(a.v);
  const int lane_row = lane / kCPR;
  // voff: a tile's offsets within its block; toff: those of the tile that
  // holds the sequence's last token (rows past it read the last token).
  unsigned voff[kPer], toff[kPer];
  {
    const int rt_last = (L - 1) / T;
    const int row0 = rt_last * T + wave * kR;
    const int blk = static_cast<int>(static_cast<unsigned>(min(row0, L - 1)) / kBlockTokens);
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const int t = wave * kR + x * kRowsW + lane_row;            // row within the stage
      const unsigned col_off = static_cast<unsigned>(ring_swz<D>(t, lane - lane_row * kCPR) * 16);
      voff[x] = static_cast<unsigned>((t % kBlockTokens) * kRowBytes) + col_off;
      toff[x] = static_cast<unsigned>((min(row0 + x * kRowsW + lane_row, L - 1) - blk * kBlockTokens) * kRowBytes) +
                col_off;
    }
  }
  const int64_t head_off = static_cast<int64_t>(g) * kBlockBytes;
  const int64_t blk_stride = static_cast<int64_t>(hkv) * kBlockBytes;
  // The tile loads are inline assembly (M0 takes the LDS destination; nothing
  // else here uses M0): the compiler does not wait on them, the explicit
  // vmcnt waits below do.  The block-table entries they need come from a
  // slice staged in LDS per pass, so no other vector load sits in the loop.
  __shared__ int bt_lds[kTableWindow];
  int blk0 = 0;
  // Block-table entry (from the staged slice) of the block holding tile rt's
  // rows that this wavefront loads; read one iteration before the loads that
  // use it.
  auto lookup = [&](int rt) {
    return __builtin_amdgcn_readfirstlane(bt_lds[static_cast<int>(static_cast<unsigned>(min(rt * T + wave * kR, L - 1)) / kBlockTokens) - blk0]);
  };
  // One tile's loads, with or without the streaming hint (a compile-time
  // string in the instruction): the choice is one uniform branch per tile.
  // `parts`: 1 = K only, 2 = V only, 3 = both.
  auto issue_loads = [&](int stage, int rt, int phys, auto stream_tag, auto parts) {
    constexpr int kParts = decltype(parts)::value;
    unsigned char *kd = lds + stage * 2 * kStageBytes;
    unsigned char *vd = kd + kStageBytes;
    const bool tail = rt * T + T > L;                // uniform; only the tile that holds token L - 1
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      unsigned off = tail ? toff[x] : voff[x];
      const unsigned dst = lds_addr32(kd) + (wave * kR + x * kRowsW) * kRowBytes;
      const unsigned dstv = lds_addr32(vd) + (wave * kR + x * kRowsW) * kRowBytes;
      const char *gk, *gv;
      if constexpr (OFF32) {
        off += static_cast<unsigned>(phys) * static_cast<unsigned>(blk_stride) + static_cast<unsigned>(head_off);
        gk = kbase;
        gv = vbase;
      } else {
        const int64_t boff = phys * blk_stride + head_off;
        gk = kbase + boff;
        gv = vbase + boff;
      }
      if constexpr (decltype(stream_tag)::value) {
        if constexpr (kParts & 1)
          asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(dst), "v"(off), "s"(gk) : "memory");
        if constexpr (kParts & 2)
          asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(dstv), "v"(off), "s"(gv) : "memory");
      } else {
        if constexpr (kParts & 1)
          asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dst), "v"(off), "s"(gk) : "memory");
        if constexpr (kParts & 2)
          asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dstv), "v"(off), "s"(gv) : "memory");
      }
    }
  };
  using kOnlyK = std::integral_constant<int, 1>;
  using kOnlyV = std::integral_constant<int, 2>;
  using kBoth = std::integral_constant<int, 3>;
  auto issue_ph = [&](int stage, int rt, int phys, auto parts) {
    if (stream_tiles) issue_loads(stage, rt, phys, std::true_type{}, parts);
    else issue_loads(stage, rt, phys, std::false_type{}, parts);
  };
  auto issue = [&](int stage, int rt, auto parts) { issue_ph(stage, rt, lookup(rt), parts); };
  const int last_blk = (L - 1) / kBlockTokens;
  constexpr int kPassTiles = kTableWindow * kBlockTokens / T;
  static_assert(S >= 3, "V of tile t and K of tile t + 1 are resident together");

  // K operand of q . k step ks for token tile tt of stage st: key tt*32 + l32,
  // dims 16 ks + 8 hh .. + 7 (16-byte chunk 2 ks + hh of the row).
  auto k_operand = [&](const unsigned char *kl, int tt, int ks) {
    const int kr = tt * 32 + l32;
    return *reinterpret_cast<const bf16x8_t *>(kl + kr * kRowBytes + ring_swz<D>(kr, 2 * ks + hh) * 16);
  };
  auto qk = [&](int st, floatx16_t(&sc)[kTT]) {
    const unsigned char *kl = lds + st * 2 * kStageBytes;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
      for (int ks = 0; ks < kQS; ++ks)
        sc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kl, tt, ks), qv[ks], ks == 0 ? zero16 : sc[tt],
                                                         0, 0, 0);
    }
  };
  // Causal mask of tile rt; only tiles reaching past the wave's first row.
  auto mask = [&](int rt, floatx16_t(&sc)[kTT]) {
    if (rt * T + T - 1 > wave_pos0) {
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (rt * T + tt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) > pos) sc[tt][i] = -INFINITY;
    }
  };
  // Row max of a tile (accumulator units) over both halves: the candidate new
  // running max, and whether it exceeds the current one by more than the
  // allowed slack (the rescale vote).
  auto finish_max = [&](float part, float &mnew) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float mx = vmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    mnew = vmaxf(m_run, mx);
    return mx > m_run + slack_raw;
  };
  auto rowmax = [&](const floatx16_t(&sc)[kTT], float &mnew) {
    float acc = vmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int w = 2; w < 16 * kTT; w += 2) acc = vmaxf(vmaxf(acc, sc[w / 16][w % 16]), sc[w / 16][w % 16 + 1]);
    return finish_max(acc, mnew);
  };
  // Move O and l to the new reference when any row of the wave asked (a row
  // that has seen no key yet holds O = l = 0: factor 0).
  auto rescale = [&](float mnew, bool raise) {
    if (__ballot(raise) != 0) {
      const float nref = mnew > -FLT_MAX ? mnew * c_log2 : ref;
      const float alpha = m_run > -FLT_MAX ? fast_exp2(ref - nref) : 0.f;
      m_run = mnew;
      ref = nref;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) o[dt] *= alpha;
    }
  };
  // V^T operand of PV step ps, dimension tile dt: lane (16-lane group
  // 2 hh + g2, j) receives keys 16 ps + 4 hh + {0..3} then 16 ps + 8 + 4 hh +
  // {0..3} of dimension dt*32 + 16 g2 + j (two transposed reads).
  auto load_v = [&](int st, bf16x8_t(&va)[kDT][kPS]) {
    const unsigned char *vl = lds + st * 2 * kStageBytes + kStageBytes;
    const int i16 = lane & 15;
    const int g2 = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const int dd = dt * 32 + 16 * g2 + 4 * (i16 & 3);
#pragma unroll
      for (int ps = 0; ps < kPS; ++ps) {
        const int r1 = ps * 16 + 4 * hh + (i16 >> 2);
        const int r2 = r1 + 8;
        const shortx4_t v1 = lds_read_tr16(vl + r1 * kRowBytes + ring_swz<D>(r1, dd >> 3) * 16 + (dd & 7) * 2);
        const shortx4_t v2 = lds_read_tr16(vl + r2 * kRowBytes + ring_swz<D>(r2, dd >> 3) * 16 + (dd & 7) * 2);
        va[dt][ps] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // Phase A: the scores of the next tile (stage st_next) on the matrix
  // cores; the weights of the current tile on the vector ALU.
  auto phase_a = [&](const floatx16_t(&cur)[kTT], int st, int st_next, floatx16_t(&nxt)[kTT], bf16x8_t(&pb)[kPS],
                     bf16x8_t(&va)[kDT][kPS]) {
    const unsigned char *kl = lds + st_next * 2 * kStageBytes;
    constexpr int kLead = 2;
    constexpr int kPairs = kTT * kQS;
    constexpr int kSteps = kPairs + kLead;
    constexpr int kScores = 16 * kTT;
    bf16x8_t ka[kPairs];
    float p[kScores];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if (Ring<D>::kEarlyV && i == kSteps / 2) load_v(st, va);
      if (i < kPairs) ka[i] = k_operand(kl, i / kQS, i % kQS);
      if (i >= kLead) {
        const int j = i - kLead;
        nxt[j / kQS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], qv[j % kQS],
                                                               j % kQS == 0 ? zero16 : nxt[j / kQS], 0, 0, 0);
      }
#pragma unroll
      for (int w = i * kScores / kSteps; w < (i + 1) * kScores / kSteps; ++w) {
        p[w] = fast_exp2(fmaf(cur[w / 16][w % 16], c_log2, -ref));
        if (w % 8 == 7) {
          const float *q8 = p + (w - 7);
          pb[w / 8] = bf16x8_t{static_cast<__bf16>(q8[0]), static_cast<__bf16>(q8[1]), static_cast<__bf16>(q8[2]),
                               static_cast<__bf16>(q8[3]), static_cast<__bf16>(q8[4]), static_cast<__bf16>(q8[5]),
                               static_cast<__bf16>(q8[6]), static_cast<__bf16>(q8[7])};
        }
      }
      if constexpr (PKV_CHUNK_INTERLEAVE) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Phase B: O^T += V^T P^T of the current tile; the vector ALU adds the
  // row sums and takes the next tile's row max.
  auto phase_b = [&](const bf16x8_t(&pb)[kPS], bf16x8_t(&va)[kDT][kPS], int st, const floatx16_t(&nxt)[kTT],
                     float &mnew) {
    if constexpr (!Ring<D>::kEarlyV) load_v(st, va);
    constexpr int kPairs = kDT * kPS;
    constexpr int kMax = 8 * kTT;              // max steps over the next tile's scores
    float acc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int dt = i / kPS, ps = i % kPS;
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][ps], pb[ps], o[dt], 0, 0, 0);
      if (i % kDT == 0) lsum = add_bf16_pairs(pb[i / kDT], lsum);
#pragma unroll
      for (int w = i * kMax / kPairs; w < (i + 1) * kMax / kPairs; ++w)
        acc = vmaxf(vmaxf(acc, nxt[w / 8][(w % 8) * 2]), nxt[w / 8][(w % 8) * 2 + 1]);
      if constexpr (PKV_CHUNK_INTERLEAVE) __builtin_amdgcn_sched_barrier(0);
    }
    return finish_max(acc, mnew);
  };

  for (int pass0 = rt_begin; pass0 < rt_end; pass0 += kPassTiles) {
    const int pass1 = min(rt_end, pass0 + kPassTiles);
    blk0 = pass0 * T / kBlockTokens;
    const int nblk = min((pass1 * T - 1) / kBlockTokens, last_blk) - blk0 + 1;
    __syncthreads();             // the previous pass is done with bt_lds
    for (int i = tid; i < nblk; i += kWaves * kWave) bt_lds[i] = min(max(bt[blk0 + i], 0), a.num_blocks - 1);
    __syncthreads();
    // Q, the metadata and the table slice have landed before any tile load
    // (vmcnt(0); expcnt and lgkmcnt left at their maxima).
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Tile t of the pass sits in stage (t - pass0) % S.  Every iteration
    // issues exactly one tile's loads (the last ones repeat the final tile),
    // so "tile t has landed" is "at most k newer tiles are outstanding".
    // Split ring: K of tiles pass0 .. pass0 + S - 1 and V of pass0 .. pass0
    // + S - 2, issued as [K(p0)], then [K(p0 + i), V(p0 + i - 1)] per i, the
    // grouping of the iterations' own loads.
    if constexpr (PKV_CHUNK_SPLIT_RING) {
      issue(0, pass0, kOnlyK{});
#pragma unroll
      for (int i = 1; i < S; ++i) {
        issue(i, min(pass0 + i, pass1 - 1), kOnlyK{});
        issue(i - 1, min(pass0 + i - 1, pass1 - 1), kOnlyV{});
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 1)) : "memory");
    } else {
#pragma unroll
      for (int i = 0; i < S - 1; ++i) issue(i, min(pass0 + i, pass1 - 1), kBoth{});
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 2)) : "memory");
    }
    __syncthreads();
    floatx16_t s0[kTT], s1[kTT];
    float mnew;
    qk(0, s0);
    mask(pass0, s0);
    bool raise = rowmax(s0, mnew);
    // Block of the next iteration's K refill (tile rt + S with the split
    // ring, rt + S - 1 otherwise) and of its V refill (tile rt + S - 1: the
    // K refill of the iteration before).
    int ph_next = lookup(min(pass0 + (PKV_CHUNK_SPLIT_RING ? S : S - 1), pass1 - 1));
    int ph_v = PKV_CHUNK_SPLIT_RING ? lookup(min(pass0 + S - 1, pass1 - 1)) : 0;

    // One iteration: tile rt's scores are in `cur`, tile rt + 1's go to `nxt`.
    // `stage_tag`: tile rt's ring stage when known at compile time (the LDS
    // addresses then fold into the instructions' offsets), else -1.
    auto iter = [&](int rt, floatx16_t(&cur)[kTT], floatx16_t(&nxt)[kTT], auto masked_next, auto stage_tag) {
      constexpr int kSt = decltype(stage_tag)::value;
      const int st = kSt >= 0 ? kSt : static_cast<int>(static_cast<unsigned>(rt - pass0) % S);
      const int st_next = kSt >= 0 ? (kSt + 1) % S : static_cast<int>(static_cast<unsigned>(rt + 1 - pass0) % S);
      const int st_fill = kSt >= 0 ? (kSt + S - 1) % S : static_cast<int>(static_cast<unsigned>(rt - pass0 + S - 1) % S);
      // Tile rt + 1 has landed (at most S - 3 newer tiles outstanding); past
      // the barrier every wave is done with tile rt - 1, whose stage refills.
      // Split ring: K of tile rt + 1 and V of tile rt were issued S - 1
      // iterations ago (S - 2 newer groups outstanding); past the barrier
      // every wave is done with K of tile rt (its slot takes K of rt + S) and
      // with V of tile rt - 1 (its slot takes V of rt + S - 1).
      if constexpr (PKV_CHUNK_SPLIT_RING) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 2)) : "memory");
        __syncthreads();
        issue_ph(st, min(rt + S, pass1 - 1), ph_next, kOnlyK{});
        issue_ph(st_fill, min(rt + S - 1, pass1 - 1), ph_v, kOnlyV{});
      } else {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 3)) : "memory");
        __syncthreads();
        issue_ph(st_fill, min(rt + S - 1, pass1 - 1), ph_next, kBoth{});
      }
      rescale(mnew, raise);
      // A wavefront whose M-rows all lie past the segment only loads its
      // share of the tiles.
      if (wave_live) {
        bf16x8_t pb[kPS];
        bf16x8_t va[kDT][kPS];
        // Phase A: the weights of tile rt while the matrix cores form the
        // scores of tile rt + 1 (of a repeat of tile rt on the last
        // iteration: computed, never used).
        phase_a(cur, st, st_next, nxt, pb, va);
        if constexpr (decltype(masked_next)::value) mask(rt + 1, nxt);
        // Phase B: O += V P of tile rt, the row sums, and the row max of
        // tile rt + 1.
        raise = phase_b(pb, va, st, nxt, mnew) && rt + 1 < pass1;
      }
      if constexpr (PKV_CHUNK_SPLIT_RING) {
        ph_v = ph_next;
        ph_next = lookup(min(rt + 1 + S, pass1 - 1));
      } else {
        ph_next = lookup(min(rt + S, pass1 - 1));
      }
    };
    // Tiles before `unmasked_end` need no causal mask for any row of this
    // wave.  Iterations whose next tile is among them run branch-free, two at
    // a time so the score buffers swap roles; the rest mask the next tile.
    // Trip counts differ between waves, but every iteration has one barrier
    // and every wave runs pass1 - pass0 of them.
    const int unmasked_end = wave_pos0 >= 0 ? (wave_pos0 + 1) / T : 0;
    const int split_at = max(pass0, min(pass1, unmasked_end - 1));
    using dyn = std::integral_constant<int, -1>;
    int rt = pass0;
    if constexpr (PKV_CHUNK_STATIC_STAGES && S == 4) {
      // a whole turn of the ring per trip: every stage index is a constant
      for (; rt + 3 < split_at; rt += 4) {
        iter(rt, s0, s1, std::false_type{}, std::integral_constant<int, 0>{});
        iter(rt + 1, s1, s0, std::false_type{}, std::integral_constant<int, 1>{});
        iter(rt + 2, s0, s1, std::false_type{}, std::integral_constant<int, 2>{});
        iter(rt + 3, s1, s0, std::false_type{}, std::integral_constant<int, 3>{});
      }
    }
    for (; rt + 1 < split_at; rt += 2) {
      iter(rt, s0, s1, std::false_type{}, dyn{});
      iter(rt + 1, s1, s0, std::false_type{}, dyn{});
    }
    if (rt < split_at) {
      iter(rt, s0, s1, std::false_type{}, dyn{});
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) s0[tt] = s1[tt];
      ++rt;
    }
    for (; rt < pass1; ++rt) {
      iter(rt, s0, s1, std::true_type{}, dyn{});
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) s0[tt] = s1[tt];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain before the ring is reused
  }

  // Normalise and store (or store the unnormalised partial of this key range
  // for the merge).  Both halves' sums; lane (hh, l32) stores dims dt*32 + 8 r + 4 hh .. + 3.
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
  const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (!valid) return;
  if (partial_out) {
    const int64_t pidx = static_cast<int64_t>(g) * a.chunk_slots + part_base + m * cs.splits + split;
    float *pa = a.chunk_part + pidx * kChunkSlotFloats<D>;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4 *>(pa + dt * 32 + 8 * r + 4 * hh) =
            make_float4(o[dt][4 * r], o[dt][4 * r + 1], o[dt][4 * r + 2], o[dt][4 * r + 3]);
    // the merge takes the reference in log2 units
    if (hh == 0) *reinterpret_cast<float2 *>(pa + D) = make_float2(ref, lt);
    return;
  }
  const float inv = 1.f / lt;
  const int64_t ob = (static_cast<int64_t>(row) * a.num_q_heads + hq) * D + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v0 = o[dt][4 * r] * inv, v1 = o[dt][4 * r + 1] * inv;
      const float v2 = o[dt][4 * r + 2] * inv, v3 = o[dt][4 * r + 3] * inv;
      const int64_t off = ob + dt * 32 + 8 * r;
      if (a.out_bf16) {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + off) =
            make_uint2(f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16), f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16));
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + off) = make_float4(v0, v1, v2, v3);
      }
    }
}

// ------------------------------------------------------------ 8-bit pools
// Multi-row segments over an 8-bit pool (int8 codes with one float32 scale
// per token and KV head, for K and for V; the format pagedkv.h defines):
// the work split, row tiles, key ranges and partials of chunk_kernel, with
// each staged tile converted once per workgroup into fp16 tiles, exactly.
// Code c becomes the fp16 value 1152 + c (the pattern 0x6400 | (c + 128), one
// byte permute per two codes) and then c itself (one packed fp16 subtract of
// 1152 per two codes, exact), so the products run on v_mfma_f32_32x32x16_f16
// with Q in fp16 (exact inside fp16's range):
//   * a score is S x k_scale of its key, formed before the row max;
//   * P' = fp16(p x v_scale) multiplies the V codes, so O weights the stored
//     value code x v_scale by P' / v_scale; the row sum adds exactly that
//     weight (P' times the reciprocal of v_scale).  A zero V row (scale 0,
//     codes 0) takes scale 1.
// (With PKV_CHUNK_Q8_EXACT_CODES=0 the tiles keep 1152 + c: a score is then
// (S - 1152 sum(q)) x k_scale and O loses 1152 x sum(P') at the end.)
// Three raw stages (the tile's codes and its blocks' scale lines, direct to
// LDS) feed three converted stages (fp16 K and V tiles and per-token scale
// factors): while the scores of tile rt + 1 and the weights of tile rt are
// formed, tile rt + 2 is converted, so one barrier per tile orders it all.
typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2_t __attribute__((ext_vector_type(2)));

// Four int8 codes (one dword) -> two dwords of fp16 (1152 + code, or the
// code itself).
__device__ __forceinline__ uint2 q8c_codes_to_f16x4(unsigned w) {
  const unsigned u = w ^ 0x80808080u;       // code + 128 as unsigned bytes
  uint2 r = make_uint2(__builtin_amdgcn_perm(0x64646464u, u, 0x05010400u),
                       __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u));
  if constexpr (PKV_CHUNK_Q8_EXACT_CODES) {
    const halfx2_t bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
    r.x = __builtin_bit_cast(unsigned, __builtin_bit_cast(halfx2_t, r.x) - bias);
    r.y = __builtin_bit_cast(unsigned, __builtin_bit_cast(halfx2_t, r.y) - bias);
  }
  return r;
}

template <int D>
struct Q8Geo {
  static constexpr int T = Ring<D>::kTok;              // tokens per tile
  static constexpr int kRaw = 3, kConv = 3;            // raw and converted stages
  static constexpr int kCodeTile = T * D;              // K (or V) code bytes per tile
  static constexpr int kScaleSlot = 256;               // per wavefront: its block's 32 floats, twice
  static constexpr int kRawBytes = 2 * kCodeTile + kWaves * kScaleSlot;
  static constexpr int kRowBytes = 2 * D;              // fp16 row
  static constexpr int kCPR = kRowBytes / 16;          // 16-byte chunks per fp16 row
  static constexpr int kTileBytes = T * kRowBytes;     // fp16 K (or V) tile
  static constexpr int kFacBytes = 3 * T * 4;          // k_scale, v_scale, 1 / v_scale per token
  static constexpr int kConvBytes = 2 * kTileBytes + kFacBytes;
  static constexpr int kCodeCPR = D / 16;              // 16-byte code chunks per row
  static constexpr int kR = T / kWaves;                // token rows per wavefront
  static_assert(kCodeTile / 16 == kWaves * kWave, "one code chunk per thread per K or V tile");
  static_assert(kBlockTokens % kR == 0, "a wavefront's rows stay inside one block");
};

// Multi-row segments of an 8-bit pool: all of them (no verify kernel here).
template <int D>
__device__ __forceinline__ int chunk_q8_units_of(const SegInfo &s, int G) {
  if (!s.ok || s.n < 2) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.mtiles * c.splits;
}
template <int D>
__device__ __forceinline__ int chunk_q8_partial_slots_of(const SegInfo &s, int G) {
  if (!s.ok || s.n < 2) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.splits > 1 ? s.n * G * c.splits : 0;
}

template <int D, bool OFF32>
__global__ __launch_bounds__(256, 2) void chunk_q8_kernel(AttendArgs a, int G) {
  using M = Q8Geo<D>;
  constexpr int T = M::T;
  constexpr int kTT = T / 32;                 // 32-token MFMA tiles per tile
  constexpr int kPS = T / 16;                 // 16-key PV steps per tile
  constexpr int kQS = D / 16;                 // 16-dim q . k steps
  constexpr int kDT = D / 32;                 // 32-wide output dimension tiles
  constexpr int kPerIssue = 3;                // VMEM ops per wavefront per tile (K, V codes, scales)
  __shared__ __align__(16) unsigned char raw[M::kRaw * M::kRawBytes];
  __shared__ __align__(16) unsigned char conv[M::kConv * M::kConvBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const auto map = make_unit_map(a, [&](const SegInfo &s) { return chunk_q8_units_of<D>(s, G); },
                                 [&](const SegInfo &s) { return chunk_q8_partial_slots_of<D>(s, G); });
  const int hkv = a.num_kv_heads;
  if (static_cast<int64_t>(blockIdx.x) >= static_cast<int64_t>(map.total) * hkv) return;
  const int unit = blockIdx.x / hkv;
  const int g = blockIdx.x - unit * hkv;
  const UnitPlace place = map.place(unit);
  const int u = place.rest;
  const SegInfo si = place.si;
  if (!si.ok) return;
  const int n = si.n, L = si.L;
  const int mtot = n * G;
  const ChunkShape cs = chunk_shape<D>(n, L, G);
  const int mt = cs.mtiles - 1 - u / cs.splits;      // heaviest (latest) rows first
  const int split = u - (cs.mtiles - 1 - mt) * cs.splits;
  const int m0 = mt * kMTile;
  const int mw = m0 + wave * kRowsPerWave;
  const int m_last = min(m0 + kMTile, mtot) - 1;
  const int kv_end = L - n + m_last / G + 1;         // keys any row of the tile sees
  const int rt_begin = split * cs.tps * (kKV / T);
  const int rt_end = min(rt_begin + cs.tps * (kKV / T), (kv_end + T - 1) / T);
  if (rt_begin >= rt_end) return;
  const bool partial_out = cs.splits > 1;
  const bool stream_tiles = PKV_CHUNK_STREAM_LOADS == 1 || (PKV_CHUNK_STREAM_LOADS == 2 && cs.mtiles == 1);
  int64_t part_base = 0;
  if (partial_out) {
    if (a.chunk_part == nullptr) return;
    part_base = place.slots_before;
    if (part_base + static_cast<int64_t>(mtot) * cs.splits > a.chunk_slots) return;   // bounds understated
  }
  const int wave_pos0 = mw < mtot ? L - n + mw / G : -1;
  const bool wave_live = mw < mtot;                  // the wavefront has M-rows of the segment

  // Q operand in fp16: lane holds dims 16 ks + 8 hh .. + 7 of its M-row;
  // with biased codes, qbias = 1152 x the sum of the row's fp16 values (both halves).
  const float c_log2 = a.scale_log2;
  const float slack_raw = PKV_CHUNK_RESCALE_SLACK / c_log2;
  const int m = mw + l32;
  const bool valid = m < mtot;
  const int qi = valid ? m / G : 0;
  const int qh = valid ? m - qi * G : 0;
  const int pos = valid ? L - n + qi : -1;
  const int row = si.row0 + qi;
  const int hq = g * G + qh;
  halfx8_t qv[kQS];
  float qbias = 0.f;
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                      (static_cast<int64_t>(row) * a.num_q_heads + hq) * D);
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) {
      const uint4 w = valid ? qp[2 * ks + hh] : make_uint4(0, 0, 0, 0);
      const unsigned ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 h0 = static_cast<_Float16>(__uint_as_float(ww[i] << 16));
        const _Float16 h1 = static_cast<_Float16>(__uint_as_float(ww[i] & 0xFFFF0000u));
        qv[ks][2 * i] = h0;
        qv[ks][2 * i + 1] = h1;
        if constexpr (!PKV_CHUNK_Q8_EXACT_CODES) qbias += static_cast<float>(h0) + static_cast<float>(h1);
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(qbias), __float_as_uint(qbias), false, false);
    qbias = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * 1152.f;
  }

  // Softmax state as in chunk_kernel; csum: this half's sum of the fp16 P' (biased codes only).
  float m_run = -FLT_MAX, ref = 0.f, lsum = 0.f, csum = 0.f;
  const floatx16_t zero16 = {};
  floatx16_t o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  // Raw staging: thread tid loads code chunk tid of the K and of the V tile
  // (row r = tid / kCodeCPR, 16 codes at dims 16 c ..), a wavefront's rows
  // inside one block; each wavefront also loads its block's scale line (32
  // floats: K's 16 then V's 16) into its own slot (lanes 32-63 repeat it).
  // Rows past the sequence read the last token.
  constexpr int kBlockCodes = kBlockTokens * D;        // code bytes of one (block, head)
  const int r_own = tid / M::kCodeCPR;
  const int c_own = tid - r_own * M::kCodeCPR;
  const int32_t *bt = a.block_tables + static_cast<int64_t>(si.slot) * a.max_blocks;
  const char *kbase = static_cast<const char *>(a.k);
  const char *vbase = static_cast<const char *>(a.v);
  unsigned voff, toff;
  {
    const int rt_last = (L - 1) / T;
    const int row0 = rt_last * T + wave * M::kR;
    const int blk = static_cast<int>(static_cast<unsigned>(min(row0, L - 1)) / kBlockTokens);
    voff = static_cast<unsigned>(((r_own) % kBlockTokens) * D + c_own * 16);
    toff = static_cast<unsigned>((min(rt_last * T + r_own, L - 1) - blk * kBlockTokens) * D + c_own * 16);
  }
  const int64_t head_codes = static_cast<int64_t>(g) * kBlockCodes;
  const int64_t blk_codes = static_cast<int64_t>(hkv) * kBlockCodes;
  __shared__ int bt_lds[kTableWindow];
  int blk0 = 0;
  auto lookup = [&](int rt) {
    return __builtin_amdgcn_readfirstlane(bt_lds[static_cast<int>(static_cast<unsigned>(min(rt * T + wave * M::kR, L - 1)) / kBlockTokens) - blk0]);
  };
  auto issue_loads = [&](int slot, int rt, int phys, auto stream_tag) {
    unsigned char *rs = raw + slot * M::kRawBytes;
    const bool tail = rt * T + T > L;                // uniform; only the tile that holds token L - 1
    unsigned off = tail ? toff : voff;
    const char *gk, *gv;
    if constexpr (OFF32) {
      off += static_cast<unsigned>(phys) * static_cast<unsigned>(blk_codes) + static_cast<unsigned>(head_codes);
      gk = kbase;
      gv = vbase;
    } else {
      const int64_t boff = phys * blk_codes + head_codes;
      gk = kbase + boff;
      gv = vbase + boff;
    }
    const unsigned dk = lds_addr32(rs) + wave * kWave * 16;
    const unsigned dv = lds_addr32(rs + M::kCodeTile) + wave * kWave * 16;
    const unsigned ds = lds_addr32(rs + 2 * M::kCodeTile) + wave * M::kScaleSlot;
    const float *gs = a.scales + (static_cast<int64_t>(phys) * hkv + g) * (2 * kBlockTokens) + (lane & 31);
    if constexpr (decltype(stream_tag)::value) {
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(dk), "v"(off), "s"(gk) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(dv), "v"(off), "s"(gv) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off nt" ::"s"(ds), "v"(gs) : "memory");
    } else {
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dk), "v"(off), "s"(gk) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dv), "v"(off), "s"(gv) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(ds), "v"(gs) : "memory");
    }
  };
  auto issue = [&](int slot, int rt) {
    const int phys = lookup(rt);
    if (stream_tiles) issue_loads(slot, rt, phys, std::true_type{});
    else issue_loads(slot, rt, phys, std::false_type{});
  };
  const int last_blk = (L - 1) / kBlockTokens;
  constexpr int kPassTiles = kTableWindow * kBlockTokens / T;

  // Raw tile rt (in raw stage rslot) -> converted stage cslot: fp16 K and V
  // rows at the bf16 kernel's chunk positions, and the tile's per-token
  // factors (token L - 1's for rows past the sequence).
  auto convert = [&](int rslot, int cslot, int rt) {
    const unsigned char *rs = raw + rslot * M::kRawBytes;
    unsigned char *cv = conv + cslot * M::kConvBytes;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint4 w = *reinterpret_cast<const uint4 *>(rs + kv * M::kCodeTile + tid * 16);
      const uint2 a0 = q8c_codes_to_f16x4(w.x), a1 = q8c_codes_to_f16x4(w.y);
      const uint2 a2 = q8c_codes_to_f16x4(w.z), a3 = q8c_codes_to_f16x4(w.w);
      unsigned char *tile = cv + kv * M::kTileBytes + r_own * M::kRowBytes;
      *reinterpret_cast<uint4 *>(tile + ring_swz<D>(r_own, 2 * c_own) * 16) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *reinterpret_cast<uint4 *>(tile + ring_swz<D>(r_own, 2 * c_own + 1) * 16) = make_uint4(a2.x, a2.y, a3.x, a3.y);
    }
    if (tid < T) {
      const int te = min(rt * T + tid, L - 1) - rt * T;             // row within the tile
      const int bw = (te / kBlockTokens) * (kBlockTokens / M::kR);   // first wavefront of its block
      const float *line = reinterpret_cast<const float *>(rs + 2 * M::kCodeTile + bw * M::kScaleSlot);
      const int e = (rt * T + te) % kBlockTokens;
      const float ks = line[e], vs = line[kBlockTokens + e];
      const float vse = vs != 0.f ? vs : 1.f;
      float *fac = reinterpret_cast<float *>(cv + 2 * M::kTileBytes);
      fac[tid] = ks;
      fac[T + tid] = vse;
      fac[2 * T + tid] = __builtin_amdgcn_rcpf(vse);
    }
  };
  // Factor `which` (0 k_scale, 1 v_scale, 2 1 / v_scale) of the lane's keys
  // 8 j + 4 hh .. + 3 of 32-key tile tt.
  auto factor4 = [&](int cslot, int which, int tt, int j) {
    const float *fac = reinterpret_cast<const float *>(conv + cslot * M::kConvBytes + 2 * M::kTileBytes);
    return *reinterpret_cast<const float4 *>(fac + which * T + tt * 32 + 8 * j + 4 * hh);
  };
  auto k_operand = [&](const unsigned char *kl, int tt, int ks) {
    const int kr = tt * 32 + l32;
    return *reinterpret_cast<const halfx8_t *>(kl + kr * M::kRowBytes + ring_swz<D>(kr, 2 * ks + hh) * 16);
  };
  auto qk = [&](int cslot, floatx16_t(&sc)[kTT]) {
    const unsigned char *kl = conv + cslot * M::kConvBytes;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int ks = 0; ks < kQS; ++ks)
        sc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k_operand(kl, tt, ks), qv[ks], ks == 0 ? zero16 : sc[tt],
                                                        0, 0, 0);
  };
  // Raw sums -> scores: (S - qbias) x k_scale of each key; then the causal
  // mask (after the scaling: a zero K row has scale 0).
  auto scale_mask = [&](int cslot, int rt, floatx16_t(&sc)[kTT], bool masked) {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 k4 = factor4(cslot, 0, tt, j);
        if constexpr (PKV_CHUNK_Q8_EXACT_CODES) {
          sc[tt][4 * j] *= k4.x;
          sc[tt][4 * j + 1] *= k4.y;
          sc[tt][4 * j + 2] *= k4.z;
          sc[tt][4 * j + 3] *= k4.w;
        } else {
          sc[tt][4 * j] = (sc[tt][4 * j] - qbias) * k4.x;
          sc[tt][4 * j + 1] = (sc[tt][4 * j + 1] - qbias) * k4.y;
          sc[tt][4 * j + 2] = (sc[tt][4 * j + 2] - qbias) * k4.z;
          sc[tt][4 * j + 3] = (sc[tt][4 * j + 3] - qbias) * k4.w;
        }
      }
    if (masked && rt * T + T - 1 > wave_pos0) {
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (rt * T + tt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) > pos) sc[tt][i] = -INFINITY;
    }
  };
  auto finish_max = [&](float part, float &mnew) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float mx = vmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    mnew = vmaxf(m_run, mx);
    return mx > m_run + slack_raw;
  };
  auto rowmax = [&](const floatx16_t(&sc)[kTT], float &mnew) {
    float acc = vmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int w = 2; w < 16 * kTT; w += 2) acc = vmaxf(vmaxf(acc, sc[w / 16][w % 16]), sc[w / 16][w % 16 + 1]);
    return finish_max(acc, mnew);
  };
  auto rescale = [&](float mnew, bool raise) {
    if (__ballot(raise) != 0) {
      const float nref = mnew > -FLT_MAX ? mnew * c_log2 : ref;
      const float alpha = m_run > -FLT_MAX ? fast_exp2(ref - nref) : 0.f;
      m_run = mnew;
      ref = nref;
      lsum *= alpha;
      csum *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) o[dt] *= alpha;
    }
  };
  auto load_v = [&](int cslot, halfx8_t(&va)[kDT][kPS]) {
    const unsigned char *vl = conv + cslot * M::kConvBytes + M::kTileBytes;
    const int i16 = lane & 15;
    const int g2 = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const int dd = dt * 32 + 16 * g2 + 4 * (i16 & 3);
#pragma unroll
      for (int ps = 0; ps < kPS; ++ps) {
        const int r1 = ps * 16 + 4 * hh + (i16 >> 2);
        const int r2 = r1 + 8;
        const shortx4_t v1 = lds_read_tr16(vl + r1 * M::kRowBytes + ring_swz<D>(r1, dd >> 3) * 16 + (dd & 7) * 2);
        const shortx4_t v2 = lds_read_tr16(vl + r2 * M::kRowBytes + ring_swz<D>(r2, dd >> 3) * 16 + (dd & 7) * 2);
        va[dt][ps] = __builtin_bit_cast(halfx8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // Phase A: scores of the next tile on the matrix cores; the fp16 weights
  // P' = fp16(p v_scale) of the current tile, their row sum (P' / v_scale)
  // and their plain sum (for the code bias) on the vector ALU.
  auto phase_a = [&](const floatx16_t(&cur)[kTT], int cs_cur, int cs_next, floatx16_t(&nxt)[kTT],
                     halfx8_t(&pb)[kPS]) {
    const unsigned char *kl = conv + cs_next * M::kConvBytes;
    constexpr int kLead = 2;
    constexpr int kPairs = kTT * kQS;
    constexpr int kSteps = kPairs + kLead;
    constexpr int kScores = 16 * kTT;
    halfx8_t ka[kPairs];
    _Float16 hp[kScores];
    float4 vs4 = {}, rv4 = {};
    const halfx2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if (i < kPairs) ka[i] = k_operand(kl, i / kQS, i % kQS);
      if (i >= kLead) {
        const int j = i - kLead;
        nxt[j / kQS] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[j], qv[j % kQS],
                                                              j % kQS == 0 ? zero16 : nxt[j / kQS], 0, 0, 0);
      }
#pragma unroll
      for (int w = i * kScores / kSteps; w < (i + 1) * kScores / kSteps; ++w) {
        if (w % 4 == 0) {
          vs4 = factor4(cs_cur, 1, w / 16, (w % 16) / 4);
          rv4 = factor4(cs_cur, 2, w / 16, (w % 16) / 4);
        }
        const float vsk = w % 4 == 0 ? vs4.x : w % 4 == 1 ? vs4.y : w % 4 == 2 ? vs4.z : vs4.w;
        const float rvk = w % 4 == 0 ? rv4.x : w % 4 == 1 ? rv4.y : w % 4 == 2 ? rv4.z : rv4.w;
        const _Float16 ph = static_cast<_Float16>(fast_exp2(fmaf(cur[w / 16][w % 16], c_log2, -ref)) * vsk);
        hp[w] = ph;
        lsum = fmaf(static_cast<float>(ph), rvk, lsum);           // the weight P' / v_scale
        if (!PKV_CHUNK_Q8_EXACT_CODES && w % 2 == 1)
          csum = __builtin_amdgcn_fdot2(halfx2_t{hp[w - 1], ph}, one2, csum, false);
        if (w % 8 == 7)
          pb[w / 8] = halfx8_t{hp[w - 7], hp[w - 6], hp[w - 5], hp[w - 4], hp[w - 3], hp[w - 2], hp[w - 1], ph};
      }
    }
  };
  // Phase B: O^T += V^T P'^T of the current tile; the row max of the next.
  auto phase_b = [&](const halfx8_t(&pb)[kPS], int cs_cur, const floatx16_t(&nxt)[kTT], float &mnew) {
    halfx8_t va[kDT][kPS];
    load_v(cs_cur, va);
    constexpr int kPairs = kDT * kPS;
    constexpr int kMax = 8 * kTT;
    float acc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int dt = i / kPS, ps = i % kPS;
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[dt][ps], pb[ps], o[dt], 0, 0, 0);
#pragma unroll
      for (int w = i * kMax / kPairs; w < (i + 1) * kMax / kPairs; ++w)
        acc = vmaxf(vmaxf(acc, nxt[w / 8][(w % 8) * 2]), nxt[w / 8][(w % 8) * 2 + 1]);
    }
    return finish_max(acc, mnew);
  };

  for (int pass0 = rt_begin; pass0 < rt_end; pass0 += kPassTiles) {
    const int pass1 = min(rt_end, pass0 + kPassTiles);
    blk0 = pass0 * T / kBlockTokens;
    const int nblk = min((pass1 * T - 1) / kBlockTokens, last_blk) - blk0 + 1;
    __syncthreads();             // the previous pass is done with bt_lds and the stages
    for (int i = tid; i < nblk; i += kWaves * kWave) bt_lds[i] = min(max(bt[blk0 + i], 0), a.num_blocks - 1);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // Q and the table slice have landed (vmcnt(0))

    // Tile t sits in raw stage and converted stage (t - pass0) % 3.  Every
    // iteration issues exactly one tile (the last ones repeat the final
    // tile), so "tile t has landed" is "at most k newer tiles outstanding".
    auto slot = [&](int t) { return static_cast<int>(static_cast<unsigned>(t - pass0) % 3u); };
    auto clampt = [&](int t) { return min(t, pass1 - 1); };
    issue(0, clampt(pass0));
    issue(1, clampt(pass0 + 1));
    issue(2, clampt(pass0 + 2));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPerIssue) : "memory");
    __syncthreads();
    convert(0, 0, clampt(pass0));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPerIssue) : "memory");
    __syncthreads();
    convert(1, 1, clampt(pass0 + 1));
    __syncthreads();             // both converted; raw stage 0 may be refilled
    issue(0, clampt(pass0 + 3));
    floatx16_t s0[kTT], s1[kTT];
    float mnew;
    qk(0, s0);
    scale_mask(0, pass0, s0, true);
    bool raise = rowmax(s0, mnew);

    // One iteration: tile rt's scores are in `cur`, tile rt + 1's go to `nxt`.
    auto iter = [&](int rt, floatx16_t(&cur)[kTT], floatx16_t(&nxt)[kTT], auto masked_next) {
      // Tile rt + 2 has landed (tile rt + 3 may be outstanding); past the
      // barrier every wave is done with iteration rt - 1, so converted
      // stage (rt + 2) % 3 and raw stage (rt + 1) % 3 are free.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPerIssue) : "memory");
      __syncthreads();
      issue(slot(rt + 1), clampt(rt + 4));
      rescale(mnew, raise);
      convert(slot(rt + 2), slot(rt + 2), clampt(rt + 2));
      if (!wave_live) return;                           // no M-row of the segment: staging only
      halfx8_t pb[kPS];
      phase_a(cur, slot(rt), slot(rt + 1), nxt, pb);
      scale_mask(slot(rt + 1), rt + 1, nxt, decltype(masked_next)::value);
      raise = phase_b(pb, slot(rt), nxt, mnew) && rt + 1 < pass1;
    };
    const int unmasked_end = wave_pos0 >= 0 ? (wave_pos0 + 1) / T : 0;
    const int split_at = max(pass0, min(pass1, unmasked_end - 1));
    int rt = pass0;
    for (; rt + 1 < split_at; rt += 2) {
      iter(rt, s0, s1, std::false_type{});
      iter(rt + 1, s1, s0, std::false_type{});
    }
    if (rt < split_at) {
      iter(rt, s0, s1, std::false_type{});
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) s0[tt] = s1[tt];
      ++rt;
    }
    for (; rt < pass1; ++rt) {
      iter(rt, s0, s1, std::true_type{});
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) s0[tt] = s1[tt];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain before the stages are reused
  }

  // Both halves' sums (and, with the biased codes, O loses 1152 x sum(P')); then normalise or store the
  // partial of this key range.
  const auto swl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
  const float lt = __uint_as_float(swl[0]) + __uint_as_float(swl[1]);
  if constexpr (!PKV_CHUNK_Q8_EXACT_CODES) {
    const auto swc = __builtin_amdgcn_permlane32_swap(__float_as_uint(csum), __float_as_uint(csum), false, false);
    const float ct = (__uint_as_float(swc[0]) + __uint_as_float(swc[1])) * 1152.f;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) o[dt] -= ct;
  }
  if (!valid) return;
  if (partial_out) {
    const int64_t pidx = static_cast<int64_t>(g) * a.chunk_slots + part_base + m * cs.splits + split;
    float *pa = a.chunk_part + pidx * kChunkSlotFloats<D>;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4 *>(pa + dt * 32 + 8 * r + 4 * hh) =
            make_float4(o[dt][4 * r], o[dt][4 * r + 1], o[dt][4 * r + 2], o[dt][4 * r + 3]);
    if (hh == 0) *reinterpret_cast<float2 *>(pa + D) = make_float2(ref, lt);
    return;
  }
  const float inv = 1.f / lt;
  const int64_t ob = (static_cast<int64_t>(row) * a.num_q_heads + hq) * D + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v0 = o[dt][4 * r] * inv, v1 = o[dt][4 * r + 1] * inv;
      const float v2 = o[dt][4 * r + 2] * inv, v3 = o[dt][4 * r + 3] * inv;
      const int64_t off = ob + dt * 32 + 8 * r;
      if (a.out_bf16) {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + off) =
            make_uint2(f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16), f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16));
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + off) = make_float4(v0, v1, v2, v3);
      }
    }
}

// Merge the key-range partials of split segments: for M-row m (query row
// i = m / G, head g * G + m % G), ranges 0 .. min(splits - 1, pos / (tps*64))
// hold keys it sees; combine them in range order.  A unit is 4 consecutive
// M-rows of one split segment and is one wavefront: a 16-lane group per
// M-row, each lane owning D / 16 output dimensions.
constexpr int kMergeRowsPerWave = 4;
constexpr int kMergeWaves = 4;

// Q8: an 8-bit pool's launch (every multi-row segment on the chunk kernel).
template <int D, bool Q8>
__device__ __forceinline__ int merge_units_of(const SegInfo &s, int G) {
  if (!s.ok || s.n < 2 || (!Q8 && verify_segment(s.n, G, D))) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.splits > 1 ? (s.n * G + kMergeRowsPerWave - 1) / kMergeRowsPerWave : 0;
}

template <int D, bool Q8>
__global__ __launch_bounds__(kMergeWaves * kWave) void chunk_merge_kernel(AttendArgs a, int G) {
  constexpr int DPL = D / 16;                         // dimensions per lane
  constexpr int SF = kChunkSlotFloats<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int hkv = a.num_kv_heads;
  const int wg = blockIdx.x / hkv;
  const int g = blockIdx.x - wg * hkv;                // same head-to-workgroup order as the chunk kernel
  const auto map = make_unit_map(a, [&](const SegInfo &s) { return merge_units_of<D, Q8>(s, G); },
                                 [&](const SegInfo &s) {
                                   return Q8 ? chunk_q8_partial_slots_of<D>(s, G) : chunk_partial_slots_of<D>(s, G);
                                 });
  const int unit = wg * kMergeWaves + wave;
  if (unit >= map.total) return;
  const UnitPlace place = map.place(unit);
  const int u = place.rest;
  const SegInfo si = place.si;
  if (!si.ok) return;
  const ChunkShape cs = chunk_shape<D>(si.n, si.L, G);
  const int64_t part_base = place.slots_before;
  if (part_base + static_cast<int64_t>(si.n) * G * cs.splits > a.chunk_slots) return;
  const int m = u * kMergeRowsPerWave + (lane >> 4);
  if (m >= si.n * G) return;                          // no cross-group exchange below
  const int i = m / G;
  const int h = m - i * G;
  const int pos = si.L - si.n + i;
  const int last = min(cs.splits - 1, pos / (cs.tps * kKV));
  const float *pp = a.chunk_part + (static_cast<int64_t>(g) * a.chunk_slots + part_base +
                                    static_cast<int64_t>(m) * cs.splits) * SF;
  // Row max over the ranges: lane li reads ranges li, li + 16, ...
  float mx = -FLT_MAX;
  for (int sp = li; sp <= last; sp += 16) mx = fmaxf(mx, pp[sp * SF + D]);
  mx = group16_max(mx);
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;
  float lsum = 0.f;
#pragma unroll 4
  for (int sp = 0; sp <= last; ++sp) {
    const float *q = pp + sp * SF;
    const float2 ml = *reinterpret_cast<const float2 *>(q + D);
    const float w = fast_exp2(ml.x - mx);
    lsum = fmaf(w, ml.y, lsum);
#pragma unroll
    for (int k = 0; k < DPL; k += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(q + li * DPL + k);
      o[k] = fmaf(w, v.x, o[k]);
      o[k + 1] = fmaf(w, v.y, o[k + 1]);
      o[k + 2] = fmaf(w, v.z, o[k + 2]);
      o[k + 3] = fmaf(w, v.w, o[k + 3]);
    }
  }
  const float inv = 1.f / lsum;
  const int64_t ob = (static_cast<int64_t>(si.row0 + i) * a.num_q_heads + g * G + h) * D + li * DPL;
  if (a.out_bf16) {
    uint32_t w[DPL / 2];
#pragma unroll
    for (int k = 0; k < DPL; k += 2) w[k / 2] = f32_to_bf16_rne(o[k] * inv) | (f32_to_bf16_rne(o[k + 1] * inv) << 16);
    uint16_t *op = static_cast<uint16_t *>(a.out) + ob;
    if constexpr (DPL == 8) *reinterpret_cast<uint4 *>(op) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2 *>(op) = make_uint2(w[0], w[1]);
  } else {
    float *op = static_cast<float *>(a.out) + ob;
#pragma unroll
    for (int k = 0; k < DPL; k += 4)
      *reinterpret_cast<float4 *>(op + k) = make_float4(o[k] * inv, o[k + 1] * inv, o[k + 2] * inv, o[k + 3] * inv);
  }
}

}  // namespace

bool chunk_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return (dtype == PKV_BF16 || (dtype == PKV_I8 && PKV_CHUNK_Q8)) && (head_dim == 64 || head_dim == 128) &&
         group >= 1 && group <= 8;
}

bool chunk_segment_splits(int32_t n, int32_t L, int32_t G, int32_t head_dim) {
  if (n < 2 || L < n || G < 1) return false;
  const ChunkShape c = head_dim == 128 ? chunk_shape<128>(n, L, G) : chunk_shape<64>(n, L, G);
  return c.splits > 1;
}

int launch_chunk(const AttendArgs &a, int32_t dtype, int32_t head_dim, int32_t max_query_len,
                 int32_t max_context_len, bool need_merge, hipStream_t stream) {
  const bool q8 = dtype == PKV_I8;
  const int G = a.num_q_heads / a.num_kv_heads;
  // Upper bound on workgroups: per segment, row tiles x splits is at most
  // max(row tiles, the split target) and row tiles <= n G / 128 + 1; the
  // splits are also at most ceil(K/V tiles / the range floor) for the
  // longest context.  Surplus workgroups exit at once.
  const int64_t row_tiles = static_cast<int64_t>(a.total_q) * G / kMTile + a.num_segments;
  const int64_t kv_tiles = (static_cast<int64_t>(max_context_len > 0 ? max_context_len : 1) + kKV - 1) / kKV;
  const int64_t max_splits = (kv_tiles + PKV_CHUNK_MIN_TILES_PER_SPLIT - 1) / PKV_CHUNK_MIN_TILES_PER_SPLIT;
  const int64_t by_target =
      static_cast<int64_t>(a.total_q) * G / kMTile + static_cast<int64_t>(a.num_segments) * (chunk_split_row_tiles(head_dim) + 1);
  const int64_t by_splits = row_tiles * (max_splits > 1 ? max_splits : 1);
  const int64_t bound = (by_target < by_splits ? by_target : by_splits) * a.num_kv_heads;
  if (bound <= 0) return PKV_OK;
  if (bound > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(bound)), block(kWaves * kWave);
  const uint64_t tensor_bytes =
      static_cast<uint64_t>(a.num_blocks) * a.num_kv_heads * kBlockTokens * head_dim * (q8 ? 1 : 2);
  const bool off32 = tensor_bytes <= 0xFFFFFFFFull;
  if (q8) {
    if (head_dim == 128) {
      if (off32) chunk_q8_kernel<128, true><<<grid, block, 0, stream>>>(a, G);
      else chunk_q8_kernel<128, false><<<grid, block, 0, stream>>>(a, G);
    } else {
      if (off32) chunk_q8_kernel<64, true><<<grid, block, 0, stream>>>(a, G);
      else chunk_q8_kernel<64, false><<<grid, block, 0, stream>>>(a, G);
    }
  } else if (head_dim == 128) {
    if (off32) chunk_kernel<128, true><<<grid, block, 0, stream>>>(a, G);
    else chunk_kernel<128, false><<<grid, block, 0, stream>>>(a, G);
  } else {
    if (off32) chunk_kernel<64, true><<<grid, block, 0, stream>>>(a, G);
    else chunk_kernel<64, false><<<grid, block, 0, stream>>>(a, G);
  }
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (a.chunk_part == nullptr || !need_merge) return PKV_OK;
  // Merge: at most total_q * G M-rows in split segments, padded to whole
  // units per segment.
  const int64_t units = (static_cast<int64_t>(a.total_q) * G) / kMergeRowsPerWave + a.num_segments;
  const int64_t mgrid = (units + kMergeWaves - 1) / kMergeWaves * a.num_kv_heads;
  if (mgrid <= 0) return PKV_OK;
  if (mgrid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const dim3 mg(static_cast<unsigned>(mgrid)), mb(kMergeWaves * kWave);
  if (head_dim == 128) {
    if (q8) chunk_merge_kernel<128, true><<<mg, mb, 0, stream>>>(a, G);
    else chunk_merge_kernel<128, false><<<mg, mb, 0, stream>>>(a, G);
  } else {
    if (q8) chunk_merge_kernel<64, true><<<mg, mb, 0, stream>>>(a, G);
    else chunk_merge_kernel<64, false><<<mg, mb, 0, stream>>>(a, G);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
