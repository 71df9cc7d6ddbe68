// Multi-row segments (prompt chunks, speculative drafts) on bf16 MFMA tiles.
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
// runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   * "M-rows" are (query row, head of the GQA group) pairs, m = i * G + h;
//     a workgroup of 4 wavefronts takes 128 consecutive M-rows of one
//     segment and one KV head, so all G query heads share every K/V tile;
//   * K/V tiles of 64 tokens (4 pool blocks, fetched through the block table)
//     are staged in LDS once per workgroup;
//   * scores are formed transposed, S^T = K Q^T, so each lane owns one M-row
//     (lane % 16) and the softmax max/sum need only two cross-row shuffles;
//   * the output is formed as O^T += V^T P^T: P^T comes straight from the
//     S^T accumulator layout, and V^T from the natural [token][dim] tile with
//     ds_read_b64_tr_b16 (lane j of each 16-lane group receives 4 consecutive
//     tokens of dimension j);
//   * the causal mask is applied per element only on tiles that reach past a
//     wavefront's first row; rows of a segment never see past their position.
#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef short shortx8_t __attribute__((ext_vector_type(8)));

// Transposed LDS read: with lane i of a 16-lane group pointing at
// tile[t0 + i / 4][d0 + 4 (i % 4)], lane j receives tile[t0 .. t0 + 3][d0 + j].
__device__ __forceinline__ shortx4_t lds_read_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t *)(p));
}


// IEEE-754 maximum (NaN-propagating): lowers to v_maximum3_f32 / v_maximum_f32
// with no canonicalisation of matrix-core results, unlike fmaxf.
__device__ __forceinline__ float vmaxf(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <int N>
__device__ __forceinline__ float max_of(const float (&v)[N]) {
  float m = vmaxf(v[0], v[1]);
#pragma unroll
  for (int i = 2; i + 1 < N; i += 2) m = vmaxf(m, vmaxf(v[i], v[i + 1]));
  if constexpr (N % 2 == 1) m = vmaxf(m, v[N - 1]);
  return m;
}

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups) with the
// lane-swap instructions: each swap leaves x[l] and x[l ^ 32] (then
// x[l ^ 16]) in the two returned registers of every lane.
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;                 // two 16-row MFMA column tiles
constexpr int kMTile = kWaves * kRowsPerWave;    // M-rows per workgroup
constexpr int kKV = 64;                          // tokens per K/V tile
constexpr int kPad = 32;                         // LDS row padding (bytes)
constexpr int kTableWindow = PKV_CHUNK_TABLE_WINDOW;   // block-table entries staged per pass

template <int D>
struct ChunkGeo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kStride = kRowBytes + kPad;         // LDS bytes per token row
  static constexpr int kCPR = kRowBytes / 16;              // 16-byte chunks per row
  static constexpr int kPerThread = kKV * kCPR / (kWaves * kWave);
  static constexpr int kKSteps = D / 32;                   // MFMA k-steps of q . k
  static constexpr int kDTiles = D / 16;                   // 16-wide output column tiles
  static constexpr int kTileLds = kKV * kStride;
};

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
__device__ __forceinline__ ChunkShape chunk_shape(int n, int L, int G) {
  ChunkShape c;
  c.mtiles = (n * G + kMTile - 1) / kMTile;
  const int kv_tiles = (L + kKV - 1) / kKV;
  constexpr int kRT = chunk_split_row_tiles(D);
  int splits = c.mtiles >= kRT ? 1 : kRT / c.mtiles;
  constexpr int kMin = PKV_CHUNK_MIN_TILES_PER_SPLIT;
  splits = max(1, min(splits, (kv_tiles + kMin - 1) / kMin));   // at least kMin K/V tiles per range
  c.tps = (kv_tiles + splits - 1) / splits;
  c.splits = (kv_tiles + c.tps - 1) / c.tps;
  return c;
}

template <int D>
__device__ __forceinline__ int chunk_units(const AttendArgs &a, int b, int G) {
  const SegInfo s = seg_info(a, b);
  if (!s.ok || s.n < 2 || verify_segment(s.n, G, D)) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.mtiles * c.splits;
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
// K operand reads (16 rows, one chunk) and the transposed V reads (4 rows,
// two chunks) hit distinct banks.
template <int D>
__device__ __forceinline__ int ring_swz(int t, int c) {
  if constexpr (D == 128) return c ^ (((t & 7) << 1) | ((t >> 3) & 1));
  else return c ^ ((((t >> 1) & 3) << 1) | ((t >> 3) & 1));
}

__device__ __forceinline__ unsigned lds_addr32(const unsigned char *p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p)));
}

// OFF32: every byte of a pool tensor lies within 4 GiB of its base, so a tile
// load addresses the tensor base (scalar) plus one 32-bit vector offset.
template <int D, bool OFF32>
__global__ __launch_bounds__(256, Ring<D>::kMinWaves) void chunk_kernel(AttendArgs a, int G) {
  using C = ChunkGeo<D>;
  constexpr int T = Ring<D>::kTok;            // tokens per ring stage
  constexpr int S = Ring<D>::kStages;
  constexpr int kRowBytes = D * 2;
  constexpr int kCPR = kRowBytes / 16;
  constexpr int kStageBytes = T * kRowBytes;  // K (or V) bytes per stage
  constexpr int kPer = T * kCPR / (kWaves * kWave);   // 16-byte chunks per thread per tile
  constexpr int kTT = T / 16;                 // 16-token MFMA tiles per stage
  constexpr int kKS = T / 32;                 // 32-key MFMA steps per stage
  static_assert(kPer >= 1 && T % 32 == 0 && 64 % T == 0, "ring geometry");
  __shared__ __align__(16) unsigned char lds[S * 2 * kStageBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  auto units_fn = [&](int b) { return chunk_units<D>(a, b, G); };
  const int hkv = a.num_kv_heads;
  const int total = __builtin_amdgcn_readfirstlane(count_units(a.num_segments, units_fn));
  if (static_cast<int64_t>(blockIdx.x) >= static_cast<int64_t>(total) * hkv) return;
  const int unit = blockIdx.x / hkv;
  const int g = blockIdx.x - unit * hkv;
  int u;
  const int b = __builtin_amdgcn_readfirstlane(find_unit(a.num_segments, unit, units_fn, &u));
  u = __builtin_amdgcn_readfirstlane(u);
  const SegInfo si = seg_info_uniform(a, b);
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
  if (rt_begin >= rt_end) return;                     // no row of this tile reaches this key range
  const bool partial_out = cs.splits > 1;
  if (partial_out && a.chunk_part == nullptr) return;
  // first position among this wave's rows (rows past the segment see nothing)
  const int wave_pos0 = mw < mtot ? L - n + mw / G : -1;

  // Q operands (B of S^T = K Q^T): lane holds 8 dims of its M-row per k-step,
  // pre-multiplied by scale * log2(e) (rounded to bf16) so that the matrix
  // cores produce scores in log2 units.
  const float c_log2 = a.scale_log2;
  int pos[2], row[2], hq[2];
  bool valid[2];
  bf16x8_t qv[2][C::kKSteps];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int m = mw + qt * 16 + l16;
    valid[qt] = m < mtot;
    const int i = valid[qt] ? m / G : 0;
    const int h = valid[qt] ? m - i * G : 0;
    pos[qt] = valid[qt] ? L - n + i : -1;
    row[qt] = si.row0 + i;
    hq[qt] = g * G + h;
    const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                      (static_cast<int64_t>(row[qt]) * a.num_q_heads + hq[qt]) * D);
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      const uint4 w = valid[qt] ? qp[kk * 4 + lg] : make_uint4(0, 0, 0, 0);
      const bf16x8_t raw = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[qt][kk][j] = static_cast<__bf16>(static_cast<float>(raw[j]) * c_log2);
    }
  }

  // Online softmax state per M-row (log2 units): running max m_run, and the
  // reference r_ref that the score accumulators start from (-r_ref), so that
  // a tile's accumulators hold score - r_ref and its weights are exp2 of them
  // directly.  r_ref follows m_run once the row has seen an unmasked key (0
  // before).  The row sums are one more output tile, lsum: the matrix cores
  // multiply the bf16 weights by an all-ones V^T tile, so every lane holds
  // its own row's sum of exactly the weights the products used.
  float m_run[2] = {-FLT_MAX, -FLT_MAX};
  floatx4_t lsum[2] = {floatx4_t{0.f, 0.f, 0.f, 0.f}, floatx4_t{0.f, 0.f, 0.f, 0.f}};
  float r_ref[2] = {0.f, 0.f};
  floatx4_t negr[2] = {floatx4_t{0.f, 0.f, 0.f, 0.f}, floatx4_t{0.f, 0.f, 0.f, 0.f}};
  floatx4_t o[C::kDTiles][2];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt) o[dt][0] = o[dt][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // Direct-to-LDS staging.  Thread tid fills 16-byte chunks q = x * 256 + tid
  // of each K and V stage: token row t = q / kCPR, position p = q % kCPR,
  // taking chunk ring_swz(t, p) of that row.  One wavefront's 64 chunks of a
  // step x are kRowsW consecutive token rows (8 for D = 64, 4 for D = 128)
  // inside a single pool block, so the block lookup and the 64-bit base are
  // wave-uniform (scalar registers) and each lane adds a fixed 32-bit offset.
  // Tokens past the sequence read the last token (finite data; their scores
  // are masked and their weights are exactly zero).
  constexpr int kRowsX = kWaves * kWave / kCPR;     // token rows per step x
  constexpr int kRowsW = kWave / kCPR;              // of which one wavefront's
  constexpr int kBlockBytes = kBlockTokens * kRowBytes;
  static_assert(kBlockTokens % kRowsW == 0 && T % kBlockTokens == 0, "a wavefront's rows stay inside one block");
  const int32_t *bt = a.block_tables + static_cast<int64_t>(si.slot) * a.max_blocks;
  const char *kbase = static_cast<const char *>(a.k);
  const char *vbase = static_cast<const char *>(a.v);
  const int lane_row = lane / kCPR;
  unsigned voff[kPer], col_off[kPer];
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    const int t = x * kRowsX + wave * kRowsW + lane_row;          // row within the stage
    col_off[x] = static_cast<unsigned>(ring_swz<D>(t, lane - lane_row * kCPR) * 16);
    voff[x] = static_cast<unsigned>((t % kBlockTokens) * kRowBytes) + col_off[x];
  }
  const int64_t head_off = static_cast<int64_t>(g) * kBlockBytes;
  const int64_t blk_stride = static_cast<int64_t>(hkv) * kBlockBytes;
  // The tile loads are inline assembly (M0 takes the LDS destination; nothing
  // else here uses M0): the compiler does not wait on them, the explicit
  // vmcnt waits below do.  The block-table entries they need come from a
  // slice staged in LDS per pass, so no other vector load sits in the loop.
  __shared__ int bt_lds[kTableWindow];
  int blk0 = 0;
  // Block-table entries (from the staged slice) of tile rt's rows that this
  // wavefront loads; read one iteration before the loads that use them.
  auto lookup = [&](int rt, int(&ph)[kPer]) {
#pragma unroll
    for (int x = 0; x < kPer; ++x)
      ph[x] = __builtin_amdgcn_readfirstlane(bt_lds[min(rt * T + x * kRowsX + wave * kRowsW, L - 1) / kBlockTokens - blk0]);
  };
  auto issue_ph = [&](int stage, int rt, const int(&ph)[kPer]) {
    unsigned char *kd = lds + stage * 2 * kStageBytes;
    unsigned char *vd = kd + kStageBytes;
    const bool tail = rt * T + T > L;                // uniform
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const int tok0 = rt * T + x * kRowsX + wave * kRowsW;       // wavefront's first row
      const int blk = min(tok0, L - 1) / kBlockTokens;
      const int phys = ph[x];
      unsigned off = voff[x];
      if (tail)
        off = static_cast<unsigned>((min(tok0 + lane_row, L - 1) - blk * kBlockTokens) * kRowBytes) + col_off[x];
      const unsigned dst = lds_addr32(kd) + (x * (kWaves * kWave) + wave * kWave) * 16;
      const unsigned dstv = lds_addr32(vd) + (x * (kWaves * kWave) + wave * kWave) * 16;
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
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 " PKV_CHUNK_DMA_HINT ::"s"(dst), "v"(off),
                   "s"(gk)
                   : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 " PKV_CHUNK_DMA_HINT ::"s"(dstv), "v"(off),
                   "s"(gv)
                   : "memory");
    }
  };
  auto issue = [&](int stage, int rt) {
    int ph[kPer];
    lookup(rt, ph);
    issue_ph(stage, rt, ph);
  };
  const int last_blk = (L - 1) / kBlockTokens;
  constexpr int kPassTiles = kTableWindow * kBlockTokens / T;
  static_assert(S >= 3, "V of tile t and K of tile t + 1 are resident together");

  // S^T = K Q^T for the tile in stage st: kTT token tiles x 2 row tiles.
  // Lane holds keys tt*16 + 4*lg + e of the tile for its M-rows (qt, l16).
  auto qk = [&](int st, floatx4_t(&sc)[kTT][2]) {
    const unsigned char *kl = lds + st * 2 * kStageBytes;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      sc[tt][0] = negr[0];
      sc[tt][1] = negr[1];
      const int kr = tt * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t *>(kl + kr * kRowBytes + ring_swz<D>(kr, kk * 4 + lg) * 16);
        sc[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[0][kk], sc[tt][0], 0, 0, 0);
        sc[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[1][kk], sc[tt][1], 0, 0, 0);
      }
    }
  };
  // Causal mask of tile rt; only tiles reaching past the wave's first row.
  auto mask = [&](int rt, floatx4_t(&sc)[kTT][2]) {
    if (rt * T + T - 1 > wave_pos0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (rt * T + tt * 16 + lg * 4 + e > pos[qt]) sc[tt][qt][e] = -INFINITY;
    }
  };
  // Row max of a tile (log2 units): the candidate new running max, and
  // whether it exceeds the current one by more than the allowed slack.
  auto rowmax = [&](const floatx4_t(&sc)[kTT][2], float(&mnew)[2]) {
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float v[4 * kTT];
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[tt * 4 + e] = sc[tt][qt][e];
      const float mx = r_ref[qt] + group4_max(max_of<4 * kTT>(v));
      mnew[qt] = vmaxf(m_run[qt], mx);
      raise |= mx > m_run[qt] + PKV_CHUNK_RESCALE_SLACK;
    }
    return raise;
  };
  // Move O and l to the new running max when any row of the wave asked.
  // Move O and l to the new running max when any row of the wave asked, and
  // re-base the pending tile's accumulators `cur` to the new reference.
  auto rescale = [&](const float(&mnew)[2], bool raise, floatx4_t(&cur)[kTT][2]) {
    if (__ballot(raise) != 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float alpha = fast_exp2(m_run[qt] - mnew[qt]);
        m_run[qt] = mnew[qt];
        lsum[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) o[dt][qt] *= alpha;
        const float nr = mnew[qt] > -FLT_MAX ? mnew[qt] : r_ref[qt];
        const float d = nr - r_ref[qt];
        r_ref[qt] = nr;
        negr[qt] = floatx4_t{-nr, -nr, -nr, -nr};
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) cur[tt][qt] -= d;
      }
    }
  };
  // V^T operands of tile stage st for phase B: keys 4*lg .. 4*lg+3 and
  // 16 + 4*lg .. of each 32-key step, dimension dt*16 + l16, read transposed
  // from the swizzled tile.
  auto load_v = [&](int st, bf16x8_t(&va)[C::kDTiles][kKS]) {
    const unsigned char *vl = lds + st * 2 * kStageBytes + kStageBytes;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
      const int dd = dt * 16 + 4 * (l16 & 3);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const int r1 = ks * 32 + lg * 4 + (l16 >> 2);
        const int r2 = r1 + 16;
        const shortx4_t v1 = lds_read_tr16(vl + r1 * kRowBytes + ring_swz<D>(r1, dd >> 3) * 16 + (dd & 7) * 2);
        const shortx4_t v2 = lds_read_tr16(vl + r2 * kRowBytes + ring_swz<D>(r2, dd >> 3) * 16 + (dd & 7) * 2);
        va[dt][ks] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // Phase A of an iteration: the matrix cores form the scores of the next
  // tile (S^T = K Q^T from stage st_next) while the vector ALU turns the
  // current tile's scores into bf16 weights and row sums.  The two streams
  // are interleaved by hand, one matrix-core pair per step, each step fenced
  // so that the scheduler keeps them side by side.
  auto phase_a = [&](const floatx4_t(&cur)[kTT][2], int st, int st_next, floatx4_t(&nxt)[kTT][2],
                     bf16x8_t(&pb)[kKS][2], bf16x8_t(&va)[C::kDTiles][kKS]) {
    const unsigned char *kl = lds + st_next * 2 * kStageBytes;
    // K operand of matrix-core pair j (token tile j / kKSteps, k-step
    // j % kKSteps): read at step j, used kLead steps later.
    bf16x8_t ka[kTT * C::kKSteps];
    auto load_k = [&](int j) {
      const int kr = (j / C::kKSteps) * 16 + l16;
      ka[j] = *reinterpret_cast<const bf16x8_t *>(kl + kr * kRowBytes + ring_swz<D>(kr, (j % C::kKSteps) * 4 + lg) * 16);
    };
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      nxt[tt][0] = negr[0];
      nxt[tt][1] = negr[1];
    }
    // The first kLead steps are weights only, covering the operand reads.
    constexpr int kLead = 2;
    constexpr int kPairs = kTT * C::kKSteps;
    constexpr int kSteps = kPairs + kLead;
    constexpr int kScores = 2 * kKS * 8;
    float p[2][kKS][8];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if (Ring<D>::kEarlyV && i == kSteps / 2) load_v(st, va);   // V reads of the current tile, midway
      if (i < kPairs) load_k(i);
      if (i >= kLead) {
        const int j = i - kLead, tt = j / C::kKSteps, kk = j % C::kKSteps;
        nxt[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qv[0][kk], nxt[tt][0], 0, 0, 0);
        nxt[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qv[1][kk], nxt[tt][1], 0, 0, 0);
      }
#pragma unroll
      for (int w = i * kScores / kSteps; w < (i + 1) * kScores / kSteps; ++w) {
        const int qt = w / (kKS * 8), ks = (w / 8) % kKS, e8 = w % 8;
        p[qt][ks][e8] = fast_exp2(cur[2 * ks + e8 / 4][qt][e8 % 4]);
        if (e8 == 7) {
          const float *q8 = p[qt][ks];
          pb[ks][qt] = bf16x8_t{static_cast<__bf16>(q8[0]), static_cast<__bf16>(q8[1]), static_cast<__bf16>(q8[2]),
                                static_cast<__bf16>(q8[3]), static_cast<__bf16>(q8[4]), static_cast<__bf16>(q8[5]),
                                static_cast<__bf16>(q8[6]), static_cast<__bf16>(q8[7])};
        }
      }
      if constexpr (PKV_CHUNK_INTERLEAVE) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Phase B: O^T += V^T P^T of the current tile (stage st) on the matrix
  // cores while the vector ALU takes the row max of the next tile.  Returns
  // the rescale vote, as rowmax.
  auto phase_b = [&](const bf16x8_t(&pb)[kKS][2], bf16x8_t(&va)[C::kDTiles][kKS], int st,
                     const floatx4_t(&nxt)[kTT][2], float(&mnew)[2]) {
    if constexpr (!Ring<D>::kEarlyV) load_v(st, va);
    // the last kKS pairs are the row sums (all-ones V^T operand)
    constexpr int kPairs = C::kDTiles * kKS + kKS;
    constexpr int kItems = 2 * kTT;
    const bf16x8_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f), static_cast<__bf16>(1.f),
                           static_cast<__bf16>(1.f), static_cast<__bf16>(1.f), static_cast<__bf16>(1.f),
                           static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    float acc[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int dt = i / kKS, ks = i % kKS;
      if (dt < C::kDTiles) {
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt][ks], pb[ks][0], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt][ks], pb[ks][1], o[dt][1], 0, 0, 0);
      } else {
        lsum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[ks][0], lsum[0], 0, 0, 0);
        lsum[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[ks][1], lsum[1], 0, 0, 0);
      }
#pragma unroll
      for (int w = i * kItems / kPairs; w < (i + 1) * kItems / kPairs; ++w) {
        const int qt = w / kTT, tt = w % kTT;
        const floatx4_t &x = nxt[tt][qt];
        acc[qt] = vmaxf(acc[qt], vmaxf(vmaxf(x[0], x[1]), vmaxf(x[2], x[3])));
      }
      if constexpr (PKV_CHUNK_INTERLEAVE) __builtin_amdgcn_sched_barrier(0);
    }
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float mx = r_ref[qt] + group4_max(acc[qt]);
      mnew[qt] = vmaxf(m_run[qt], mx);
      raise |= mx > m_run[qt] + PKV_CHUNK_RESCALE_SLACK;
    }
    return raise;
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
#pragma unroll
    for (int i = 0; i < S - 1; ++i) issue(i, min(pass0 + i, pass1 - 1));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 2)) : "memory");
    __syncthreads();
    floatx4_t s0[kTT][2], s1[kTT][2];
    float mnew[2];
    qk(0, s0);
    mask(pass0, s0);
    bool raise = rowmax(s0, mnew);
    int ph_next[kPer];
    lookup(min(pass0 + S - 1, pass1 - 1), ph_next);

    // One iteration: tile rt's scores are in `cur`, tile rt + 1's go to `nxt`.
    auto iter = [&](int rt, floatx4_t(&cur)[kTT][2], floatx4_t(&nxt)[kTT][2], auto masked_next) {
      const int st = (rt - pass0) % S;
      const int st_next = (rt + 1 - pass0) % S;
      // Tile rt + 1 has landed (at most S - 3 newer tiles outstanding); past
      // the barrier every wave is done with tile rt - 1, whose stage refills.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer * (S - 3)) : "memory");
      __syncthreads();
      issue_ph((rt - pass0 + S - 1) % S, min(rt + S - 1, pass1 - 1), ph_next);
      rescale(mnew, raise, cur);
      // Phase A: the weights of tile rt on the vector ALU while the matrix
      // cores form the scores of tile rt + 1 (of a repeat of tile rt on the
      // last iteration: computed, never used).
      bf16x8_t pb[kKS][2];
      bf16x8_t va[C::kDTiles][kKS];
      phase_a(cur, st, st_next, nxt, pb, va);
      if constexpr (decltype(masked_next)::value) mask(rt + 1, nxt);
      // Phase B: O += V P of tile rt on the matrix cores while the vector
      // ALU takes the row max of tile rt + 1.
      raise = phase_b(pb, va, st, nxt, mnew) && rt + 1 < pass1;
      lookup(min(rt + S, pass1 - 1), ph_next);
    };
    // Tiles before `unmasked_end` need no causal mask for any row of this
    // wave.  Iterations whose next tile is among them run branch-free, two at
    // a time so the score buffers swap roles; the rest mask the next tile.
    // Trip counts differ between waves, but every iteration has one barrier
    // and every wave runs pass1 - pass0 of them.
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
      for (int tt = 0; tt < kTT; ++tt) {
        s0[tt][0] = s1[tt][0];
        s0[tt][1] = s1[tt][1];
      }
      ++rt;
    }
    for (; rt < pass1; ++rt) {
      iter(rt, s0, s1, std::true_type{});
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
        s0[tt][0] = s1[tt][0];
        s0[tt][1] = s1[tt][1];
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain before the ring is reused
  }

  // Normalise and store (or store the unnormalised partial of this key range
  // for the merge); every lane already holds its row's sum.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = lsum[qt][0];
    if (!valid[qt]) continue;
    if (partial_out) {
      const int m = mw + qt * 16 + l16;
      const int64_t pidx = (static_cast<int64_t>(b) * hkv + g) * chunk_split_slots(D) + m * cs.splits + split;
      float *pa = a.chunk_part + pidx * kChunkSlotFloats<D>;
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        *reinterpret_cast<float4 *>(pa + dt * 16 + lg * 4) =
            make_float4(o[dt][qt][0], o[dt][qt][1], o[dt][qt][2], o[dt][qt][3]);
      if (lg == 0) *reinterpret_cast<float2 *>(pa + D) = make_float2(m_run[qt], lt);
      continue;
    }
    const float inv = 1.f / lt;
    const int64_t ob = (static_cast<int64_t>(row[qt]) * a.num_q_heads + hq[qt]) * D + lg * 4;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
      const floatx4_t v = o[dt][qt] * inv;
      if (a.out_bf16) {
        uint16_t *op = static_cast<uint16_t *>(a.out) + ob + dt * 16;
        *reinterpret_cast<uint2 *>(op) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                    f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + ob + dt * 16) = make_float4(v[0], v[1], v[2], v[3]);
      }
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

template <int D>
__device__ __forceinline__ int merge_units(const AttendArgs &a, int b, int G) {
  const SegInfo s = seg_info(a, b);
  if (!s.ok || s.n < 2 || verify_segment(s.n, G, D)) return 0;
  const ChunkShape c = chunk_shape<D>(s.n, s.L, G);
  return c.splits > 1 ? (s.n * G + kMergeRowsPerWave - 1) / kMergeRowsPerWave : 0;
}

template <int D>
__global__ __launch_bounds__(kMergeWaves * kWave) void chunk_merge_kernel(AttendArgs a, int G) {
  constexpr int DPL = D / 16;                         // dimensions per lane
  constexpr int SF = kChunkSlotFloats<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int hkv = a.num_kv_heads;
  const int wg = blockIdx.x / hkv;
  const int g = blockIdx.x - wg * hkv;                // same head-to-workgroup order as the chunk kernel
  auto units_fn = [&](int b) { return merge_units<D>(a, b, G); };
  const int total = __builtin_amdgcn_readfirstlane(count_units(a.num_segments, units_fn));
  const int unit = wg * kMergeWaves + wave;
  if (unit >= total) return;
  int u;
  const int b = __builtin_amdgcn_readfirstlane(find_unit(a.num_segments, unit, units_fn, &u));
  u = __builtin_amdgcn_readfirstlane(u);
  const SegInfo si = seg_info_uniform(a, b);
  if (!si.ok) return;
  const ChunkShape cs = chunk_shape<D>(si.n, si.L, G);
  const int m = u * kMergeRowsPerWave + (lane >> 4);
  if (m >= si.n * G) return;                          // no cross-group exchange below
  const int i = m / G;
  const int h = m - i * G;
  const int pos = si.L - si.n + i;
  const int last = min(cs.splits - 1, pos / (cs.tps * kKV));
  const float *pp = a.chunk_part + ((static_cast<int64_t>(b) * hkv + g) * chunk_split_slots(D) +
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
  return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8;
}

int launch_chunk(const AttendArgs &a, int32_t head_dim, int32_t max_query_len, int32_t max_context_len,
                 hipStream_t stream) {
  (void)max_context_len;
  const int G = a.num_q_heads / a.num_kv_heads;
  // Upper bound on workgroups: per segment, row tiles x splits is at most
  // max(row tiles, the split target) and row tiles <= n G / 128 + 1;
  // surplus workgroups exit at once.
  const int64_t bound =
      (static_cast<int64_t>(a.total_q) * G / kMTile + static_cast<int64_t>(a.num_segments) * (chunk_split_row_tiles(head_dim) + 1)) *
      a.num_kv_heads;
  if (bound <= 0) return PKV_OK;
  if (bound > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(bound)), block(kWaves * kWave);
  const uint64_t tensor_bytes =
      static_cast<uint64_t>(a.num_blocks) * a.num_kv_heads * kBlockTokens * head_dim * 2;   // bf16
  const bool off32 = tensor_bytes <= 0xFFFFFFFFull;
  if (head_dim == 128) {
    if (off32) chunk_kernel<128, true><<<grid, block, 0, stream>>>(a, G);
    else chunk_kernel<128, false><<<grid, block, 0, stream>>>(a, G);
  } else {
    if (off32) chunk_kernel<64, true><<<grid, block, 0, stream>>>(a, G);
    else chunk_kernel<64, false><<<grid, block, 0, stream>>>(a, G);
  }
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (a.chunk_part == nullptr) return PKV_OK;
  // Merge: at most total_q * G M-rows in split segments, padded to whole
  // units per segment.
  const int64_t units = (static_cast<int64_t>(a.total_q) * G) / kMergeRowsPerWave + a.num_segments;
  const int64_t mgrid = (units + kMergeWaves - 1) / kMergeWaves * a.num_kv_heads;
  if (mgrid <= 0) return PKV_OK;
  if (mgrid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  if (head_dim == 128)
    chunk_merge_kernel<128><<<dim3(static_cast<unsigned>(mgrid)), dim3(kMergeWaves * kWave), 0, stream>>>(a, G);
  else
    chunk_merge_kernel<64><<<dim3(static_cast<unsigned>(mgrid)), dim3(kMergeWaves * kWave), 0, stream>>>(a, G);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
