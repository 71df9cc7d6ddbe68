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

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;                 // two 16-row MFMA column tiles
constexpr int kMTile = kWaves * kRowsPerWave;    // M-rows per workgroup
constexpr int kKV = 64;                          // tokens per K/V tile
constexpr int kPad = 32;                         // LDS row padding (bytes)
constexpr int kTableWindow = 2048;               // block-table entries staged per pass

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

__device__ __forceinline__ ChunkShape chunk_shape(int n, int L, int G) {
  ChunkShape c;
  c.mtiles = (n * G + kMTile - 1) / kMTile;
  const int kv_tiles = (L + kKV - 1) / kKV;
  int splits = c.mtiles >= kChunkSplitRowTiles ? 1 : kChunkSplitRowTiles / c.mtiles;
  splits = max(1, min(splits, (kv_tiles + 1) / 2));   // at least two K/V tiles per range
  c.tps = (kv_tiles + splits - 1) / splits;
  c.splits = (kv_tiles + c.tps - 1) / c.tps;
  return c;
}

__device__ __forceinline__ int chunk_units(const AttendArgs &a, int b, int G) {
  const SegInfo s = seg_info(a, b);
  if (!s.ok || s.n < 2) return 0;
  const ChunkShape c = chunk_shape(s.n, s.L, G);
  return c.mtiles * c.splits;
}

// LDS ring of K/V tiles fed by direct-to-LDS loads: kRingTok tokens per
// stage, kRingStages stages (64 KiB or less per workgroup so two fit a CU).
template <int D>
struct Ring;
template <>
struct Ring<64> {
  static constexpr int kTok = PKV_CHUNK_RING_TOK_D64, kStages = PKV_CHUNK_RING_STAGES_D64;
};
template <>
struct Ring<128> {
  static constexpr int kTok = PKV_CHUNK_RING_TOK_D128, kStages = PKV_CHUNK_RING_STAGES_D128;
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

template <int D>
__global__ __launch_bounds__(256, 2) void chunk_kernel(AttendArgs a, int G) {
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

  auto units_fn = [&](int b) { return chunk_units(a, b, G); };
  const int hkv = a.num_kv_heads;
  const int total = count_units(a.num_segments, units_fn);
  if (static_cast<int64_t>(blockIdx.x) >= static_cast<int64_t>(total) * hkv) return;
  const int unit = blockIdx.x / hkv;
  const int g = blockIdx.x - unit * hkv;
  int u;
  const int b = find_unit(a.num_segments, unit, units_fn, &u);
  const SegInfo si = seg_info(a, b);
  if (!si.ok) return;
  const int n = si.n, L = si.L;
  const int mtot = n * G;
  const ChunkShape cs = chunk_shape(n, L, G);
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

  // Q operands (B of S^T = K Q^T): lane holds 8 dims of its M-row per k-step.
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
      qv[qt][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  float m_run[2] = {-FLT_MAX, -FLT_MAX};
  float l_run[2] = {0.f, 0.f};
  floatx4_t o[C::kDTiles][2];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt) o[dt][0] = o[dt][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const float c_log2 = a.scale_log2;

  // Direct-to-LDS staging.  Thread tid fills 16-byte chunks q = x * 256 + tid
  // of each K and V stage: token row t = q / kCPR, position p = q % kCPR,
  // taking chunk ring_swz(t, p) of that row.  Tokens past the sequence read
  // the last token (finite data; their scores are masked and their weights
  // are exactly zero).
  const int32_t *bt = a.block_tables + static_cast<int64_t>(si.slot) * a.max_blocks;
  const char *kbase = static_cast<const char *>(a.k);
  const char *vbase = static_cast<const char *>(a.v);
  int row_of[kPer], col_off[kPer];
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    const int q = x * (kWaves * kWave) + tid;
    row_of[x] = q / kCPR;
    col_off[x] = ring_swz<D>(row_of[x], q - row_of[x] * kCPR) * 16;
  }
  // The tile loads are inline assembly (M0 takes the LDS destination; nothing
  // else here uses M0): the compiler does not wait on them, the explicit
  // vmcnt waits below do.  The block-table entries they need come from a
  // slice staged in LDS per pass, so no other vector load sits in the loop.
  __shared__ int bt_lds[kTableWindow];
  int blk0 = 0;
  auto issue = [&](int stage, int rt) {
    unsigned char *kd = lds + stage * 2 * kStageBytes;
    unsigned char *vd = kd + kStageBytes;
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const int tok = min(rt * T + row_of[x], L - 1);
      const int phys = bt_lds[tok / kBlockTokens - blk0];
      const int64_t off = ((static_cast<int64_t>(phys) * hkv + g) * kBlockTokens + (tok % kBlockTokens)) * kRowBytes +
                          col_off[x];
      const unsigned dst = lds_addr32(kd) + (x * (kWaves * kWave) + wave * kWave) * 16;
      const unsigned dstv = lds_addr32(vd) + (x * (kWaves * kWave) + wave * kWave) * 16;
      const void *gk = kbase + off;
      const void *gv = vbase + off;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT ::"s"(dst), "v"(gk)
                   : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT ::"s"(dstv), "v"(gv)
                   : "memory");
    }
  };
  const int last_blk = (L - 1) / kBlockTokens;
  constexpr int kPassTiles = kTableWindow * kBlockTokens / T;

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

#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i, min(pass0 + i, pass1 - 1));
  for (int rt = pass0; rt < pass1; ++rt) {
    const int stage = (rt - pass0) % S;
    // this wave's loads of tile rt have landed once at most S - 2 newer
    // tiles' loads are outstanding; the barrier makes everyone's visible and
    // retires every read of the stage refilled below
    if constexpr (S == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (S == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer) : "memory");
    if constexpr (S == 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kPer) : "memory");
    __syncthreads();
    issue((rt - pass0 + S - 1) % S, min(rt + S - 1, pass1 - 1));
    const unsigned char *kl = lds + stage * 2 * kStageBytes;
    const unsigned char *vl = kl + kStageBytes;

    // S^T tiles: kTT token tiles x 2 row tiles.
    floatx4_t s[kTT][2];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      s[tt][0] = s[tt][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = tt * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t *>(kl + kr * kRowBytes + ring_swz<D>(kr, kk * 4 + lg) * 16);
        s[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[0][kk], s[tt][0], 0, 0, 0);
        s[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[1][kk], s[tt][1], 0, 0, 0);
      }
    }
    // Lane holds keys rt*T + tt*16 + 4*lg + e of its M-rows (qt, l16).
    const bool need_mask = rt * T + T - 1 > wave_pos0;
    if (need_mask) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (rt * T + tt * 16 + lg * 4 + e > pos[qt]) s[tt][qt][e] = -INFINITY;
    }
    float mnew[2];
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = s[0][qt][0];
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[tt][qt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mnew[qt] = fmaxf(m_run[qt], mx * c_log2);
      raise |= mnew[qt] > m_run[qt];
    }
    if (__ballot(raise) != 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float alpha = fast_exp2(m_run[qt] - mnew[qt]);
        m_run[qt] = mnew[qt];
        l_run[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) o[dt][qt] *= alpha;
      }
    }
    // P^T as the B operand of O^T += V^T P^T, one per 32-key step.
    bf16x8_t pb[kKS][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = fast_exp2(fmaf(s[2 * ks][qt][e], c_log2, -m_run[qt]));
          p[4 + e] = fast_exp2(fmaf(s[2 * ks + 1][qt][e], c_log2, -m_run[qt]));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run[qt] += p[e];
        pb[ks][qt] = bf16x8_t{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]), static_cast<__bf16>(p[2]),
                              static_cast<__bf16>(p[3]), static_cast<__bf16>(p[4]), static_cast<__bf16>(p[5]),
                              static_cast<__bf16>(p[6]), static_cast<__bf16>(p[7])};
      }
    }
    // V^T operand: keys 4*lg .. 4*lg+3 and 16 + 4*lg .. of each 32-key step,
    // dimension dt*16 + l16, read transposed from the swizzled tile.
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
      const int dd = dt * 16 + 4 * (l16 & 3);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const int r1 = ks * 32 + lg * 4 + (l16 >> 2);
        const int r2 = r1 + 16;
        const shortx4_t v1 = lds_read_tr16(vl + r1 * kRowBytes + ring_swz<D>(r1, dd >> 3) * 16 + (dd & 7) * 2);
        const shortx4_t v2 = lds_read_tr16(vl + r2 * kRowBytes + ring_swz<D>(r2, dd >> 3) * 16 + (dd & 7) * 2);
        const shortx8_t rr = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, rr);
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks][0], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks][1], o[dt][1], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain before the ring is reused
  }

  // Row sums live spread over the 4 lane groups; combine, normalise, store
  // (or store the unnormalised partial of this key range for the merge).
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float lt = l_run[qt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (!valid[qt]) continue;
    if (partial_out) {
      const int m = mw + qt * 16 + l16;
      const int64_t pidx = (static_cast<int64_t>(b) * hkv + g) * kChunkSplitSlots + m * cs.splits + split;
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
// hold keys it sees; combine them in range order.  One wavefront per row.
template <int D>
__global__ __launch_bounds__(256) void chunk_merge_kernel(AttendArgs a, int G, int rows_per_block) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hkv = a.num_kv_heads;
  (void)rows_per_block;
  // blockIdx.x = (b * hkv + g) * row_blocks + rb
  const int row_blocks = gridDim.x / (a.num_segments * hkv);
  const int bg = blockIdx.x / row_blocks;
  const int rb = blockIdx.x - bg * row_blocks;
  const int b = bg / hkv;
  const int g = bg - b * hkv;
  const SegInfo si = seg_info(a, b);
  if (!si.ok || si.n < 2) return;
  const ChunkShape cs = chunk_shape(si.n, si.L, G);
  if (cs.splits <= 1 || a.chunk_part == nullptr) return;
  const int mtot = si.n * G;
  constexpr int DPL = D / kWave;
  for (int m = rb * 4 + wave; m < mtot; m += row_blocks * 4) {
    const int i = m / G;
    const int h = m - i * G;
    const int pos = si.L - si.n + i;
    const int last = min(cs.splits - 1, pos / (cs.tps * kKV));
    const int64_t base = ((static_cast<int64_t>(b) * hkv + g) * kChunkSplitSlots + static_cast<int64_t>(m) * cs.splits);
    float mx = -FLT_MAX;
    for (int sp = 0; sp <= last; ++sp) mx = fmaxf(mx, a.chunk_part[(base + sp) * kChunkSlotFloats<D> + D]);
    float lsum = 0.f;
    float o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int sp = 0; sp <= last; ++sp) {
      const float *pp = a.chunk_part + (base + sp) * kChunkSlotFloats<D>;
      const float w = fast_exp2(pp[D] - mx);
      lsum += w * pp[D + 1];
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = fmaf(w, pp[lane + k * kWave], o[k]);
    }
    const float inv = 1.f / lsum;
    const int64_t ob = (static_cast<int64_t>(si.row0 + i) * a.num_q_heads + g * G + h) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const float val = o[k] * inv;
      if (a.out_bf16)
        static_cast<uint16_t *>(a.out)[ob + lane + k * kWave] = static_cast<uint16_t>(f32_to_bf16_rne(val));
      else
        static_cast<float *>(a.out)[ob + lane + k * kWave] = val;
    }
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
  // max(row tiles, kChunkSplitRowTiles) and row tiles <= n G / 128 + 1;
  // surplus workgroups exit at once.
  const int64_t bound =
      (static_cast<int64_t>(a.total_q) * G / kMTile + static_cast<int64_t>(a.num_segments) * (kChunkSplitRowTiles + 1)) *
      a.num_kv_heads;
  if (bound <= 0) return PKV_OK;
  if (bound > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(bound)), block(kWaves * kWave);
  if (head_dim == 128)
    chunk_kernel<128><<<grid, block, 0, stream>>>(a, G);
  else
    chunk_kernel<64><<<grid, block, 0, stream>>>(a, G);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (a.chunk_part == nullptr) return PKV_OK;
  // Merge: split segments have at most kChunkSplitRowTiles * 128 / G rows x G heads.
  const int rows_cap = max_query_len * G;
  const int row_blocks = static_cast<int>((static_cast<int64_t>(min(rows_cap, kChunkSplitRowTiles * kMTile)) + 3) / 4);
  const int64_t mgrid = static_cast<int64_t>(a.num_segments) * a.num_kv_heads * row_blocks;
  if (mgrid <= 0) return PKV_OK;
  if (mgrid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  if (head_dim == 128)
    chunk_merge_kernel<128><<<dim3(static_cast<unsigned>(mgrid)), dim3(256), 0, stream>>>(a, G, 4);
  else
    chunk_merge_kernel<64><<<dim3(static_cast<unsigned>(mgrid)), dim3(256), 0, stream>>>(a, G, 4);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
