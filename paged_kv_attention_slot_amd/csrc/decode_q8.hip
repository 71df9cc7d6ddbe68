// Decode rows over an 8-bit pool: int8 codes with one float32 scale per
// (token, KV head); a stored row stands for code * scale (the lucebox blog's
// R9700 DFlash2 section runs an 8-bit KV cache; the format itself is this
// library's, defined in pagedkv.h).
//
// The work and its split are those of the bf16 MFMA decode kernel - one
// wavefront per (decode row, KV head g, split-context partition), all G query
// heads of the group sharing every tile, online softmax, partition partials
// merged by the reduce kernel - with half the tile bytes.  The 16 MFMA
// columns are a segment's (row, head) pairs: G heads of one row for a decode
// row; for a multi-row segment (prompt chunk, drafts) up to 16 pairs of
// consecutive rows per wavefront, each column with its own causal limit
// (row i sees keys 0 .. L - n + i), so the codes are read once per column
// group rather than once per row.  Multi-row segments run PKV_DECODE_Q8_GROUP_W
// column groups of one partition per workgroup, one per wavefront: a tile is
// staged and its V codes converted once for all of them (two barriers per
// tile), and each wavefront stops at its own rows' last key.  A row keeps
// partials only for the partitions up to its own position.  (Default builds
// give multi-row segments to chunk_q8_kernel in chunk.hip, which shares one
// converted tile among 128 (row, head) pairs; this form serves them only
// with PKV_CHUNK_Q8=0.)
//   * the K and V code tiles (16 x head_dim bytes each) and their 2 x 16
//     scales go from HBM straight into LDS staging (global_load_lds_dwordx4
//     for codes, one global_load_lds_dword for the scales), S tiles in
//     flight; the K code rows are XOR-swizzled in 16-byte chunks;
//   * a code c becomes an fp16 operand with one byte permute per two codes:
//     the fp16 pattern 0x6400 | (c + 128) is exactly 1152 + c, so the
//     products run on fp16 MFMA and the constant is taken out afterwards,
//     exactly: 1152 * sum(q) from every score, 1152 * sum(p) from O (sums of
//     the fp16 operands actually used);
//   * S^T[token][head] = K Q^T on v_mfma_f32_16x16x32_f16 (Q converted from
//     bf16 once per item, exact inside fp16's range), then times the token's
//     K scale;
//   * the V codes become an fp16 [token][dim] tile in LDS, read transposed
//     with ds_read_b64_tr_b16; the V scale is folded into P, so
//     O^T += V^T fp16(P * v_scale)^T on v_mfma_f32_16x16x16_f16.  That
//     weights the stored value code * v_scale by fp16(P v_scale) / v_scale,
//     and the softmax sum adds exactly those weights (one reciprocal per
//     token), so the normalisation matches the numerator.
#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));

// fp16 value of the pattern 0x6400 | (code + 128).
constexpr float kCodeBias = 1152.f;

// Column groups per workgroup for multi-row segments, and their tiles in
// flight (one wavefront issues a workgroup's loads).
#ifndef PKV_DECODE_Q8_GROUP_W
#define PKV_DECODE_Q8_GROUP_W 2
#endif
#ifndef PKV_DECODE_Q8_GROUP_STAGES
#define PKV_DECODE_Q8_GROUP_STAGES 3
#endif
constexpr int kQ8GroupW = PKV_DECODE_Q8_GROUP_W;

__device__ __forceinline__ unsigned q8_lds_addr(const unsigned char *p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)(p)));
}

__device__ __forceinline__ shortx4_t q8_lds_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t *)(p));
}

// Four int8 codes (one dword) -> two dwords of fp16 (1152 + code): the
// byte c + 128 under an exponent byte 0x64.
__device__ __forceinline__ uint2 codes_to_f16x4(unsigned w) {
  const unsigned u = w ^ 0x80808080u;       // code + 128 as unsigned bytes
  return make_uint2(__builtin_amdgcn_perm(0x64646464u, u, 0x05010400u),
                    __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u));
}

template <int D>
struct QGeo {
  static constexpr int kRowBytes = D * 2;                  // fp16 row of the converted V tile
  static constexpr int kTile = kBlockTokens * kRowBytes;   // fp16 V tile bytes
  static constexpr int kCodeCPR = D / 16;                  // 16-byte chunks per code row
  static constexpr int kCodeTile = kBlockTokens * D;       // bytes of a K (or V) code tile
  static constexpr int kCodeLoads = kCodeTile / 1024;      // direct-to-LDS loads per code tile
  static constexpr int kChunksPerLane = kCodeTile / 16 / kWave;
  static constexpr int kPerIssue = 2 * kCodeLoads + 1;     // VMEM ops per tile (codes + scales)
  static constexpr int kKSteps = D / 32;
  static constexpr int kDTiles = D / 16;
  static constexpr int kScaleBytes = 256;                  // one dword per lane: K then V scales
  // fp16 V tile chunk position (the bf16 kernel's: conflict-free
  // transposed reads).
  static __device__ __forceinline__ int swz(int t, int c) {
    if constexpr (D == 128) return c ^ (((t & 7) << 1) | ((t >> 3) & 1));
    else return c ^ ((((t >> 1) & 3) << 1) | ((t >> 3) & 1));
  }
  // K code tile chunk position.
  static __device__ __forceinline__ int kswz(int t, int c) { return c ^ (t & (kCodeCPR - 1)); }
};

__device__ __forceinline__ int q8_parts(int L) {
  return (L + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
}

// 16-wide MFMA column groups of a segment's (row, head) pairs.
__device__ __forceinline__ int q8_groups(int n, int G) { return (n * G + 15) / 16; }

// Work units of a segment.  One wavefront per workgroup (W = 1): its column
// groups times its partitions (a decode row: one group of its G heads), for
// every segment the launch serves (decode rows; in multi-row mode every
// segment, or with SINGLE only the decode rows).  W wavefronts per
// workgroup (multi-row segments only): W consecutive column groups of one
// partition per unit, so the partition's tiles are staged once for them.
template <int W, bool SINGLE>
__device__ __forceinline__ int q8_units(const SegInfo &s, bool multirow, int G) {
  if constexpr (W == 1) {
    if (!s.ok || (SINGLE ? s.n != 1 : (!multirow && s.n != 1))) return 0;
    return q8_groups(s.n, G) * q8_parts(s.L);
  } else {
    if (!s.ok || !multirow || s.n < 2) return 0;
    return (q8_groups(s.n, G) + W - 1) / W * q8_parts(s.L);
  }
}

template <int D, int S, int W, bool SINGLE>
__global__ __launch_bounds__(64 * W, PKV_DECODE_Q8_MIN_WAVES) void decode_q8_kernel(AttendArgs a, int G) {
  using M = QGeo<D>;
  static_assert(S >= 1 && S <= 3, "1 to 3 tiles in flight");
  static_assert(W == 1 || !SINGLE, "decode rows take one wavefront per workgroup");
  constexpr int PT = kDecodePartitionTokens;
  constexpr int kStage = 2 * M::kCodeTile + M::kScaleBytes;   // K codes | V codes | scales
  // V code chunks (16 bytes) of a tile, and per lane: W = 1 converts them
  // all, W > 1 spreads them over the workgroup's first wavefronts.
  constexpr int kVChunks = M::kCodeTile / 16;
  constexpr int kCPL = W == 1 ? M::kChunksPerLane : (kVChunks + kWave * W - 1) / (kWave * W);
  __shared__ __align__(16) unsigned char stg[S * kStage];
  __shared__ __align__(16) unsigned char vt[M::kTile];
  const int lane = W == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x & (kWave - 1));
  const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const bool loader = W == 1 || wave == 0;              // issues the tile loads
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const SegInfo mine = seg_info(a, lane);
  const int u0 = q8_units<W, SINGLE>(mine, a.multirow, G);
  const int incl0 = wave_inclusive_scan(u0);
  int total = __shfl(incl0, kWave - 1);
  if (a.num_segments > kWave)
    total = count_units(a.num_segments, [&](int b) { return q8_units<W, SINGLE>(seg_info(a, b), a.multirow, G); });
  const int64_t items = static_cast<int64_t>(total) * a.num_kv_heads;
  const float c_log2 = a.scale_log2;

  for (int64_t f = blockIdx.x; f < items; f += gridDim.x) {
    const int unit = static_cast<int>(f / a.num_kv_heads);
    const int g = static_cast<int>(f - static_cast<int64_t>(unit) * a.num_kv_heads);
    int b, rest;
    SegInfo si;
    if (unit < __shfl(incl0, kWave - 1)) {
      const unsigned long long mask = __ballot(incl0 > unit);
      b = __ffsll(static_cast<long long>(mask)) - 1;
      rest = unit - (__shfl(incl0, b) - __shfl(u0, b));
      si.slot = __builtin_amdgcn_readlane(mine.slot, b);
      si.L = __builtin_amdgcn_readlane(mine.L, b);
      si.n = __builtin_amdgcn_readlane(mine.n, b);
      si.row0 = __builtin_amdgcn_readlane(mine.row0, b);
      si.ok = true;
    } else {
      b = find_unit(a.num_segments, unit, [&](int bb) { return q8_units<W, SINGLE>(seg_info(a, bb), a.multirow, G); },
                    &rest);
      si = seg_info(a, b);
      if (!si.ok) continue;
    }
    // A partition's column groups are consecutive units, so they run side
    // by side on one XCD and share its L2 for the partition's tiles.
    const int ngroups = q8_groups(si.n, G);
    int part, cg, cg_last;                             // this wavefront's column group; the workgroup's last
    if constexpr (W == 1) {
      part = rest / ngroups;
      cg = rest - part * ngroups;
      cg_last = cg;
    } else {
      const int nblk = (ngroups + W - 1) / W;
      part = rest / nblk;
      const int cb = rest - part * nblk;
      cg = cb * W + wave;
      cg_last = min(cb * W + W - 1, ngroups - 1);
    }
    const bool wave_cols = W == 1 || cg < ngroups;     // the wavefront has a column group
    // MFMA column l16 = (row, head) pair cg * 16 + l16 of the segment
    const int pair = cg * 16 + l16;
    const bool hv = wave_cols && pair < si.n * G;
    const int ri = hv ? pair / G : 0;
    const int hq = g * G + (hv ? pair - ri * G : 0);
    const int row = si.row0 + ri;
    const int prow = a.multirow ? row : b;             // partials index
    const int limit = si.L - si.n + ri + 1;            // keys visible to this column's row
    // wave-uniform bounds: keys the group's last and first rows see
    const int ri_hi = min(si.n - 1, (cg * 16 + 15) / G);
    const int ri_lo = min(si.n - 1, (cg * 16) / G);
    const int tok0 = part * PT;
    const int tok1 = wave_cols ? min(si.L - si.n + ri_hi + 1, tok0 + PT) : tok0;   // tok0 >= tok1: nothing here
    const int tok_full = min(si.L - si.n + ri_lo + 1, tok1);    // every column sees keys below this
    const int lim = hv ? min(limit, tok1) : tok1;
    // Keys the workgroup stages: those its last column group sees.
    int tok1_wg = tok1;
    if constexpr (W > 1) tok1_wg = min(si.L - si.n + min(si.n - 1, (cg_last * 16 + 15) / G) + 1, tok0 + PT);
    // No column reaches this partition: nothing to do (a column's row has
    // partials only for the partitions up to its position).
    if (tok0 >= tok1_wg) continue;
    const int j0 = tok0 / kBlockTokens;
    const int nb = (tok1_wg + kBlockTokens - 1) / kBlockTokens - j0;               // tiles staged
    const int nb_w = tok1 > tok0 ? (tok1 + kBlockTokens - 1) / kBlockTokens - j0 : 0;   // tiles this wavefront uses

    int phys_lane = 0;
    if (loader && lane < nb) {
      phys_lane = a.block_tables[static_cast<int64_t>(si.slot) * a.max_blocks + j0 + lane];
      phys_lane = min(max(phys_lane, 0), a.num_blocks - 1);
    }
    // Q^T operand: lane holds dims 32 kk + 8 lg .. + 7 of its head, as fp16;
    // qsum: 1152 x the sum of its head's fp16 values (all lane groups).
    halfx8_t qh[M::kKSteps];
    float qsum = 0.f;
    {
      const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                        (static_cast<int64_t>(row) * a.num_q_heads + hq) * D);
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) {
        const uint4 w = hv ? qp[kk * 4 + lg] : make_uint4(0, 0, 0, 0);
        const unsigned ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const _Float16 h0 = static_cast<_Float16>(__uint_as_float(ww[i] << 16));
          const _Float16 h1 = static_cast<_Float16>(__uint_as_float(ww[i] & 0xFFFF0000u));
          qh[kk][2 * i] = h0;
          qh[kk][2 * i + 1] = h1;
          qsum += static_cast<float>(h0) + static_cast<float>(h1);
        }
      }
      qsum += __shfl_xor(qsum, 16);
      qsum += __shfl_xor(qsum, 32);
      qsum *= kCodeBias;
    }
    // Direct-to-LDS sources: load x fills staging chunk x * 64 + lane.  K
    // chunk position (t, p) holds code chunk kswz(t, p) of row t; V chunks
    // stay in order.  Scales: the tile's 32-float run (K scales of tokens
    // 0-15, then the V scales), one 128-byte line; lanes 32-63 load the same
    // run again into the stage's unused upper half.
    int ksrc[M::kCodeLoads];
#pragma unroll
    for (int x = 0; x < M::kCodeLoads; ++x) {
      const int P = x * kWave + lane;
      const int t = P / M::kCodeCPR;
      const int p = P - t * M::kCodeCPR;
      ksrc[x] = t * D + M::kswz(t, p) * 16;
    }
    const char *kbase = static_cast<const char *>(a.k);
    const char *vbase = static_cast<const char *>(a.v);
    const float *sbase = a.scales + (lane & 31);
    // The loads are issued as inline assembly (M0 takes the LDS destination;
    // nothing else here uses M0); the explicit s_waitcnt counts below wait
    // on them.
    auto issue = [&](int stage, int jj) {
      const int phys = __builtin_amdgcn_readlane(phys_lane, jj);
      const int64_t th = static_cast<int64_t>(phys) * a.num_kv_heads + g;
      const int64_t off = th * M::kCodeTile;
      unsigned char *st = stg + stage * kStage;
#pragma unroll
      for (int x = 0; x < M::kCodeLoads; ++x) {
        const unsigned ldsk = q8_lds_addr(st + x * 1024);
        const unsigned ldsv = q8_lds_addr(st + M::kCodeTile + x * 1024);
        const void *gk = kbase + off + ksrc[x];
        const void *gv = vbase + off + x * 1024 + lane * 16;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT
                     ::"s"(ldsk), "v"(gk) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off " PKV_LDS_DMA_HINT
                     ::"s"(ldsv), "v"(gv) : "memory");
      }
      const unsigned ldss = q8_lds_addr(st + 2 * M::kCodeTile);
      const void *gs = sbase + th * (2 * kBlockTokens);
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off " PKV_LDS_DMA_HINT
                   ::"s"(ldss), "v"(gs) : "memory");
    };

    // Q and the table slice must have landed before the tile loads start.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    float m_run = -FLT_MAX, l_run = 0.f, c_run = 0.f;   // c_run: sum of the fp16 P * v_scale used
    floatx4_t o[M::kDTiles];
#pragma unroll
    for (int dt = 0; dt < M::kDTiles; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // Staged codes of one tile -> K operands (registers), this lane's V code
    // chunks (registers, for the fp16 V tile) and its four K and V scales
    // (tokens 4 lg .. + 3).  Reads only: once they have landed the stage can
    // be refilled.
    auto read_stage = [&](int stage, halfx8_t (&ka)[M::kKSteps], uint4 (&vraw)[kCPL], floatx4_t &ks,
                          floatx4_t &vs) {
      const unsigned char *st = stg + stage * kStage;
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) {
        const int c = 2 * kk + (lg >> 1);
        const uint2 w = *reinterpret_cast<const uint2 *>(st + l16 * D + M::kswz(l16, c) * 16 + (lg & 1) * 8);
        const uint2 h0 = codes_to_f16x4(w.x), h1 = codes_to_f16x4(w.y);
        ka[kk] = __builtin_bit_cast(halfx8_t, make_uint4(h0.x, h0.y, h1.x, h1.y));
      }
#pragma unroll
      for (int i = 0; i < kCPL; ++i) {
        const int P = (i * W + wave) * kWave + lane;
        if (W == 1 || P < kVChunks) vraw[i] = *reinterpret_cast<const uint4 *>(st + M::kCodeTile + P * 16);
      }
      ks = *reinterpret_cast<const floatx4_t *>(st + 2 * M::kCodeTile + lg * 16);
      vs = *reinterpret_cast<const floatx4_t *>(st + 2 * M::kCodeTile + 64 + lg * 16);
    };
    // The V code chunks -> the fp16 V tile in LDS (the transposed reads'
    // layout).  The wave's earlier reads of the previous tile are ordered
    // before these writes.
    auto write_vt = [&](const uint4 (&vraw)[kCPL]) {
#pragma unroll
      for (int i = 0; i < kCPL; ++i) {
        const int P = (i * W + wave) * kWave + lane;
        if (W > 1 && P >= kVChunks) continue;
        const int t = P / M::kCodeCPR;
        const int p = P - t * M::kCodeCPR;
        const uint4 w = vraw[i];
        const uint2 a0 = codes_to_f16x4(w.x), a1 = codes_to_f16x4(w.y);
        const uint2 a2 = codes_to_f16x4(w.z), a3 = codes_to_f16x4(w.w);
        const uint4 lo = make_uint4(a0.x, a0.y, a1.x, a1.y);
        const uint4 hi = make_uint4(a2.x, a2.y, a3.x, a3.y);
        *reinterpret_cast<uint4 *>(vt + t * M::kRowBytes + M::swz(t, 2 * p) * 16) = lo;
        *reinterpret_cast<uint4 *>(vt + t * M::kRowBytes + M::swz(t, 2 * p + 1) * 16) = hi;
      }
    };

    auto compute = [&](const halfx8_t (&ka)[M::kKSteps], const floatx4_t &ks, const floatx4_t &vs, int jj,
                       auto partial_tag) {
      constexpr bool PARTIAL = decltype(partial_tag)::value;
      const int tokbase = (j0 + jj) * kBlockTokens;
      const int valid = lim - tokbase;        // this column's tokens of the tile (< 16 only if PARTIAL)
      floatx4_t s = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < M::kKSteps; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[kk], qh[kk], s, 0, 0, 0);
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ok[e] = !PARTIAL || lg * 4 + e < valid;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = ok[e] ? (s[e] - qsum) * ks[e] : -INFINITY;   // select: unwritten scales may be NaN
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run, mx * c_log2);
      if (__ballot(mnew > m_run) != 0) {
        const float alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
        c_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < M::kDTiles; ++dt) o[dt] *= alpha;
      }
      float p[4], w[4];
      halfx4_t ph;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(fmaf(s[e], c_log2, -m_run));
        ph[e] = static_cast<_Float16>(ok[e] ? p[e] * vs[e] : 0.f);
        // The product weights the stored value code * vs by fp16(p vs) / vs;
        // the row sum adds that weight (p itself for a zero row, scale 0,
        // whose value is 0 whatever its weight; nothing for masked tokens,
        // whose scales may be unwritten).
        w[e] = ok[e] ? (vs[e] != 0.f ? static_cast<float>(ph[e]) * __builtin_amdgcn_rcpf(vs[e]) : p[e]) : 0.f;
      }
      l_run += (w[0] + w[1]) + (w[2] + w[3]);
      c_run += (static_cast<float>(ph[0]) + static_cast<float>(ph[1])) +
               (static_cast<float>(ph[2]) + static_cast<float>(ph[3]));
      const int vt_row = lg * 4 + (l16 >> 2);
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt) {
        const int dd = dt * 16 + 4 * (l16 & 3);
        const shortx4_t va = q8_lds_tr16(vt + vt_row * M::kRowBytes + M::swz(vt_row, dd >> 3) * 16 + (dd & 7) * 2);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(halfx4_t, va), ph, o[dt], 0, 0, 0);
      }
    };

    // S tiles in flight.  Past the last tile the prefetch re-reads the last
    // tile (a cache hit) so every wait below has a static count.  An empty
    // partition loads nothing and leaves m = -FLT_MAX, l = 0, O = 0.
    if (nb > 0 && loader) {
      issue(0, 0);
      if constexpr (S > 1) issue(1, min(1, nb - 1));
      if constexpr (S > 2) issue(2, min(2, nb - 1));
    }
    // W > 1: the loader waits for a tile, and a barrier hands it to every
    // wavefront (which by then are done with the previous V tile); they read
    // the stage and convert their share of the V codes; a second barrier
    // marks the stage read and the V tile whole, and the loader refills the
    // stage.  nb and the trip counts are uniform over the workgroup.
    for (int jj = 0; jj < nb; jj += S) {
#pragma unroll
      for (int st = 0; st < S; ++st) {
        if (jj + st >= nb) break;
        // tile jj + st sits in stage st; wait until its loads have landed
        if constexpr (S == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if constexpr (S == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(M::kPerIssue) : "memory");
        if constexpr (S == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * M::kPerIssue) : "memory");
        if constexpr (W > 1) __syncthreads();
        halfx8_t ka[M::kKSteps];
        uint4 vraw[kCPL];
        floatx4_t ks, vs;
        read_stage(st, ka, vraw, ks, vs);
        if constexpr (W == 1) {
          // every read of the stage has completed: it can be refilled while
          // the V tile is converted and the tile's arithmetic runs
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if constexpr (S > 1) issue(st, min(jj + st + S, nb - 1));
          else if (jj + 1 < nb) issue(0, jj + 1);
          write_vt(vraw);
        } else {
          write_vt(vraw);
          __syncthreads();
          if (loader) {
            if constexpr (S > 1) issue(st, min(jj + st + S, nb - 1));
            else if (jj + 1 < nb) issue(0, jj + 1);
          }
        }
        if (W == 1 || jj + st < nb_w) {
          if ((j0 + jj + st + 1) * kBlockTokens > tok_full)
            compute(ka, ks, vs, jj + st, std::true_type{});
          else
            compute(ka, ks, vs, jj + st, std::false_type{});
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Lane groups hold disjoint tokens: combine their sums, then take the
    // code bias out of O.
    float lt = l_run, ct = c_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    ct += __shfl_xor(ct, 16);
    ct += __shfl_xor(ct, 32);
    ct *= kCodeBias;
#pragma unroll
    for (int dt = 0; dt < M::kDTiles; ++dt) o[dt] -= ct;
    if (!hv) continue;
    const int np_row = q8_parts(limit);               // partitions this column's row sees
    if (part >= np_row) continue;
    const bool direct = (np_row == 1);
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
      const int64_t pidx = (static_cast<int64_t>(prow) * a.num_q_heads + hq) * a.part_max + part;
      float *pa = a.part_acc + pidx * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < M::kDTiles; ++dt)
        *reinterpret_cast<float4 *>(pa + dt * 16) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (lg == 0) *reinterpret_cast<float2 *>(a.part_ml + pidx * 2) = make_float2(m_run, lt);
    }
  }
}

template <int D, int W, bool SINGLE>
int launch_q8_w(const AttendArgs &a, int G, int64_t grid, int stages, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(kWave * W);
  if (stages >= 3) decode_q8_kernel<D, 3, W, SINGLE><<<g, b, 0, stream>>>(a, G);
  else if (stages == 2) decode_q8_kernel<D, 2, W, SINGLE><<<g, b, 0, stream>>>(a, G);
  else decode_q8_kernel<D, 1, W, SINGLE><<<g, b, 0, stream>>>(a, G);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <int D>
int launch_q8_d(const AttendArgs &a, int G, int64_t parts, int stages, int32_t decode_rows, hipStream_t stream) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * kDecodeWavesPerCU;
  const int64_t hkv = a.num_kv_heads;
  if (!a.multirow) {
    const int64_t items_bound = static_cast<int64_t>(a.num_segments) * parts * hkv;
    const int64_t grid = items_bound < cap ? items_bound : cap;
    return grid > 0 ? launch_q8_w<D, 1, false>(a, G, grid, stages, stream) : PKV_OK;
  }
  // Multi-row mode: decode rows (unless the host knows there are none) one
  // wavefront per item, multi-row segments kQ8GroupW column groups per
  // workgroup.  Both write the same partials; one reduce follows.
  int st = PKV_OK;
  if (decode_rows != 0) {
    const int64_t items_bound = static_cast<int64_t>(a.num_segments) * parts * hkv;
    const int64_t grid = items_bound < cap ? items_bound : cap;
    if (grid > 0) st = launch_q8_w<D, 1, true>(a, G, grid, stages, stream);
  }
  constexpr int W = kQ8GroupW;
  const int64_t groups_bound = (static_cast<int64_t>(a.total_q) * G + 15) / 16 + a.num_segments;
  const int64_t items_bound = ((groups_bound + W - 1) / W + a.num_segments) * parts * hkv;
  const int64_t cap_w = cap / W > 0 ? cap / W : 1;
  const int64_t grid = items_bound < cap_w ? items_bound : cap_w;
  if (st == PKV_OK && grid > 0) st = launch_q8_w<D, W, false>(a, G, grid, PKV_DECODE_Q8_GROUP_STAGES, stream);
  return st;
}

}  // namespace

int launch_decode_q8(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, int stages, int32_t decode_rows,
                     hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  int64_t parts = (static_cast<int64_t>(max_context_len) + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
  if (parts < 1) parts = 1;
  return head_dim == 128 ? launch_q8_d<128>(a, G, parts, stages, decode_rows, stream)
                         : launch_q8_d<64>(a, G, parts, stages, decode_rows, stream);
}

}  // namespace pkv
