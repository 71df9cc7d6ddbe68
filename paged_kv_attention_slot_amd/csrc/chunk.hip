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

__device__ __forceinline__ int chunk_units(const AttendArgs &a, int b, int G) {
  const SegInfo s = seg_info(a, b);
  if (!s.ok || s.n < 2) return 0;
  return (s.n * G + kMTile - 1) / kMTile;
}

template <int D>
__global__ __launch_bounds__(256, 2) void chunk_kernel(AttendArgs a, int G) {
  using C = ChunkGeo<D>;
  __shared__ __align__(16) unsigned char lds[2 * C::kTileLds];
  unsigned char *kl = lds;
  unsigned char *vl = lds + C::kTileLds;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
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
  const int units = (mtot + kMTile - 1) / kMTile;
  const int m0 = (units - 1 - u) * kMTile;          // heaviest (latest) rows first
  const int mw = m0 + wave * kRowsPerWave;
  const int m_last = min(m0 + kMTile, mtot) - 1;
  const int kv_end = L - n + m_last / G + 1;         // keys any row of the tile sees
  const int ntiles = (kv_end + kKV - 1) / kKV;
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

  // Staging: thread tid copies chunks tid + 256 x of the K and V tiles.
  const int32_t *bt = a.block_tables + static_cast<int64_t>(si.slot) * a.max_blocks;
  const char *kbase = static_cast<const char *>(a.k);
  const char *vbase = static_cast<const char *>(a.v);
  uint4 kr[C::kPerThread], vr[C::kPerThread];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int x = 0; x < C::kPerThread; ++x) {
      const int q = tid + x * (kWaves * kWave);
      const int t = q / C::kCPR;
      const int col = q - t * C::kCPR;
      const int tok = kt * kKV + t;
      if (tok < L) {
        int phys = bt[tok / kBlockTokens];
        phys = min(max(phys, 0), a.num_blocks - 1);
        const int64_t off = ((static_cast<int64_t>(phys) * hkv + g) * kBlockTokens + (tok % kBlockTokens)) *
                                C::kRowBytes + col * 16;
        kr[x] = stream_load(reinterpret_cast<const uint4 *>(kbase + off));
        vr[x] = stream_load(reinterpret_cast<const uint4 *>(vbase + off));
      } else {
        kr[x] = make_uint4(0, 0, 0, 0);   // past the sequence: zeros, never the pool's contents
        vr[x] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int x = 0; x < C::kPerThread; ++x) {
      const int q = tid + x * (kWaves * kWave);
      const int t = q / C::kCPR;
      const int col = q - t * C::kCPR;
      *reinterpret_cast<uint4 *>(kl + t * C::kStride + col * 16) = kr[x];
      *reinterpret_cast<uint4 *>(vl + t * C::kStride + col * 16) = vr[x];
    }
  };

  fetch(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();           // every wave is done with the previous tile
    stash();
    __syncthreads();
    if (kt + 1 < ntiles) fetch(kt + 1);   // in flight while this tile is used

    // S^T tiles: 4 token tiles x 2 row tiles.
    floatx4_t s[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt][0] = s[tt][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t *>(kl + (tt * 16 + l16) * C::kStride + (kk * 32 + lg * 8) * 2);
        s[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[0][kk], s[tt][0], 0, 0, 0);
        s[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv[1][kk], s[tt][1], 0, 0, 0);
      }
    }
    // Lane holds keys kt*64 + tt*16 + 4*lg + e of its M-rows (qt, l16).
    const bool need_mask = kt * kKV + kKV - 1 > wave_pos0;
    if (need_mask) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kt * kKV + tt * 16 + lg * 4 + e > pos[qt]) s[tt][qt][e] = -INFINITY;
    }
    float mnew[2];
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = s[0][qt][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
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
    bf16x8_t pb[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
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
    // V^T operand: keys 4*lg .. 4*lg+3 and 16 + 4*lg .. of the 32-key step,
    // dimension dt*16 + l16, read transposed from the [token][dim] tile.
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const unsigned char *p1 = vl + (ks * 32 + lg * 4 + (l16 >> 2)) * C::kStride + (dt * 16 + 4 * (l16 & 3)) * 2;
        const shortx4_t r1 = lds_read_tr16(p1);
        const shortx4_t r2 = lds_read_tr16(p1 + 16 * C::kStride);
        const shortx8_t rr = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, rr);
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks][0], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks][1], o[dt][1], 0, 0, 0);
      }
    }
  }

  // Row sums live spread over the 4 lane groups; combine, normalise, store.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float lt = l_run[qt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (!valid[qt]) continue;
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

}  // namespace

bool chunk_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8;
}

int launch_chunk(const AttendArgs &a, int32_t head_dim, int32_t max_query_len, int32_t max_context_len,
                 hipStream_t stream) {
  (void)max_context_len;
  (void)max_query_len;
  const int G = a.num_q_heads / a.num_kv_heads;
  // Upper bound on workgroups: sum over segments of ceil(n G / 128) is at
  // most total_q G / 128 + num_segments; surplus workgroups exit at once.
  const int64_t bound = (static_cast<int64_t>(a.total_q) * G / kMTile + a.num_segments) * a.num_kv_heads;
  if (bound <= 0) return PKV_OK;
  if (bound > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(bound)), block(kWaves * kWave);
  if (head_dim == 128)
    chunk_kernel<128><<<grid, block, 0, stream>>>(a, G);
  else
    chunk_kernel<64><<<grid, block, 0, stream>>>(a, G);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
