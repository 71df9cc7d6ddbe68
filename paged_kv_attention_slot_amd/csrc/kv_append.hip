// KV append: scatter this step's new K/V rows into the shared block pool.
//
// "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog),
// §Chunked prefill is a slot phase: each selected chunk appends directly to
// its slot's paged KV.  The flat pool token slot s = slot_mapping[t] names
// position s % block_size of physical block s / block_size.
//
// The work is a pure byte copy in 16-byte units.  Thread c handles unit c of
// the packed source [T][Hkv][row16] (row16 = head_dim * elem_bytes / 16), so
// reads are perfectly coalesced; each (token, head) destination row is one
// contiguous head_dim * elem_bytes span of a (block, head) tile, so writes
// coalesce per row.  Entries outside the pool are skipped.
#include "pagedkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct AppendArgs {
  const int32_t *slot_mapping;
  const uint4 *k_new;
  const uint4 *v_new;
  uint4 *pool_k;
  uint4 *pool_v;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t heads_shift;         // log2(num_kv_heads) when it is a power of two, else -1
  int64_t pool_slots;
  // Optional: copy stage_len int32 of step metadata from stage_src (pinned
  // host memory the device can read) to stage_dst (device) in the same pass.
  const int32_t *stage_src;
  int32_t *stage_dst;
  int32_t stage_len;
};

// (token, head) of source row r: a shift for power-of-two head counts, else
// one 32-bit division (the host keeps T x Hkv x row units below 2^31).
__device__ __forceinline__ uint32_t token_of_row(uint32_t r, int32_t heads, int32_t heads_shift) {
  return heads_shift >= 0 ? r >> heads_shift : r / static_cast<uint32_t>(heads);
}

template <int ROW16>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t nthreads = gridDim.x * blockDim.x;
  for (uint32_t i = tid; i < static_cast<uint32_t>(a.stage_len); i += nthreads) a.stage_dst[i] = a.stage_src[i];
  const uint32_t total = static_cast<uint32_t>(a.num_tokens) * static_cast<uint32_t>(a.num_kv_heads) * ROW16;
  for (uint32_t c = tid; c < total; c += nthreads) {
    const uint32_t r = c / ROW16;                                // (token, head) row
    const uint32_t w = c - r * ROW16;
    const uint32_t t = token_of_row(r, a.num_kv_heads, a.heads_shift);
    const uint32_t h = r - t * static_cast<uint32_t>(a.num_kv_heads);
    const int64_t s = a.slot_mapping[t];
    if (s < 0 || s >= a.pool_slots) continue;
    const int64_t blk = s / kBlockTokens;
    const int64_t off = s - blk * kBlockTokens;
    const int64_t dst = ((blk * a.num_kv_heads + h) * kBlockTokens + off) * ROW16 + w;
    a.pool_k[dst] = a.k_new[c];
    a.pool_v[dst] = a.v_new[c];
  }
}

// 8-bit pools: each (token, KV head) row of bf16 input becomes head_dim int8
// codes plus one float32 scale (the format stated at pkv_pool in pagedkv.h):
// amax over the row, inv = 127 / amax and scale = amax / 127 as correctly
// rounded divisions, code = rint(x * inv) (the float32 product, ties to even)
// clamped to +-127; a zero row gives codes 0 and scale 0.  R = D / 8 lanes
// share a row, 8 values each: a 16-byte load of bf16, an R-lane max, an
// 8-byte store of codes; the row's first lane stores the scale.
struct Q8AppendArgs {
  const int32_t *slot_mapping;
  const uint4 *k_new;          // [T][Hkv][D] bf16, as 16-byte units
  const uint4 *v_new;
  uint2 *codes_k;              // [blocks][Hkv][16][D] int8, as 8-byte units
  uint2 *codes_v;
  float *scales;               // [blocks][Hkv][2][16]: K's 16 scales, then V's
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t heads_shift;         // log2(num_kv_heads) when it is a power of two, else -1
  int64_t pool_slots;
  const int32_t *stage_src;
  int32_t *stage_dst;
  int32_t stage_len;
};

template <int R>
__device__ __forceinline__ void quantize_row8(const uint4 in, int li, uint2 *codes, float *scale) {
  float x[8];
  const unsigned w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 1; m < R; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  unsigned lo = 0, hi = 0;
  float sc = 0.f;
  if (amax > 0.f) {
    const float inv = __fdiv_rn(127.f, amax);
    sc = __fdiv_rn(amax, 127.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float prod = x[i] * inv;
      const int c = static_cast<int>(fminf(fmaxf(rintf(prod), -127.f), 127.f));
      const unsigned byte = static_cast<unsigned>(c) & 0xFFu;
      if (i < 4) lo |= byte << (8 * i);
      else hi |= byte << (8 * (i - 4));
    }
  }
  *codes = make_uint2(lo, hi);
  if (li == 0) *scale = sc;
}

template <int D>
__global__ __launch_bounds__(256) void kv_append_q8_kernel(Q8AppendArgs a) {
  constexpr int R = D / 8;                    // lanes per row
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t nthreads = gridDim.x * blockDim.x;
  for (uint32_t i = tid; i < static_cast<uint32_t>(a.stage_len); i += nthreads) a.stage_dst[i] = a.stage_src[i];
  const int li = static_cast<int>(tid % R);
  const uint32_t rows = static_cast<uint32_t>(a.num_tokens) * static_cast<uint32_t>(a.num_kv_heads);
  for (uint32_t r = tid / R; r < rows; r += nthreads / R) {
    const uint32_t t = token_of_row(r, a.num_kv_heads, a.heads_shift);
    const int64_t h = r - t * static_cast<uint32_t>(a.num_kv_heads);
    const int64_t s = a.slot_mapping[t];
    if (s < 0 || s >= a.pool_slots) continue;   // the whole row's lanes skip together
    const int64_t blk = s / kBlockTokens;
    const int64_t off = s - blk * kBlockTokens;
    const int64_t tile = blk * a.num_kv_heads + h;
    const int64_t drow = tile * kBlockTokens + off;
    const int64_t srow = tile * (2 * kBlockTokens) + off;
    const int64_t src = static_cast<int64_t>(r) * R + li;
    quantize_row8<R>(a.k_new[src], li, a.codes_k + drow * R + li, a.scales + srow);
    quantize_row8<R>(a.v_new[src], li, a.codes_v + drow * R + li, a.scales + srow + kBlockTokens);
  }
}

static int32_t heads_shift(int32_t heads) {
  return heads > 0 && (heads & (heads - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(heads)) : -1;
}

int launch_kv_append(const int32_t *slot_mapping, const void *k_new, const void *v_new, int32_t num_tokens,
                     const pkv_pool &pool, hipStream_t stream, const int32_t *stage_src, int32_t *stage_dst,
                     int32_t stage_len) {
  if (pool.dtype == PKV_I8) {
    Q8AppendArgs a;
    a.slot_mapping = slot_mapping;
    a.k_new = static_cast<const uint4 *>(k_new);
    a.v_new = static_cast<const uint4 *>(v_new);
    a.codes_k = static_cast<uint2 *>(pool.k);
    a.codes_v = static_cast<uint2 *>(pool.v);
    a.scales = pool.scales;
    a.num_tokens = num_tokens;
    a.num_kv_heads = pool.num_kv_heads;
    a.heads_shift = heads_shift(pool.num_kv_heads);
    a.pool_slots = static_cast<int64_t>(pool.num_blocks) * pool.block_size;
    a.stage_src = stage_src;
    a.stage_dst = stage_dst;
    a.stage_len = stage_src && stage_dst ? stage_len : 0;
    const int64_t lanes = static_cast<int64_t>(num_tokens) * pool.num_kv_heads * (pool.head_dim / 8);
    if (lanes >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
    int64_t blocks = ((lanes > a.stage_len ? lanes : a.stage_len) + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    if (pool.head_dim == 128)
      kv_append_q8_kernel<128><<<dim3(blocks), dim3(256), 0, stream>>>(a);
    else if (pool.head_dim == 64)
      kv_append_q8_kernel<64><<<dim3(blocks), dim3(256), 0, stream>>>(a);
    else
      return PKV_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  const int row16 = pool.head_dim * (pool.dtype == PKV_F32 ? 4 : 2) / 16;
  const int64_t units = static_cast<int64_t>(num_tokens) * pool.num_kv_heads * row16;
  if (units >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;   // 32-bit unit indices
  const int threads = 256;
  int64_t blocks = ((units > stage_len ? units : stage_len) + threads - 1) / threads;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  AppendArgs a;
  a.slot_mapping = slot_mapping;
  a.k_new = static_cast<const uint4 *>(k_new);
  a.v_new = static_cast<const uint4 *>(v_new);
  a.pool_k = static_cast<uint4 *>(pool.k);
  a.pool_v = static_cast<uint4 *>(pool.v);
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool.num_kv_heads;
  a.heads_shift = heads_shift(pool.num_kv_heads);
  a.pool_slots = static_cast<int64_t>(pool.num_blocks) * pool.block_size;
  a.stage_src = stage_src;
  a.stage_dst = stage_dst;
  a.stage_len = stage_src && stage_dst ? stage_len : 0;
  switch (row16) {
    case 8: kv_append_kernel<8><<<dim3(blocks), dim3(threads), 0, stream>>>(a); break;
    case 16: kv_append_kernel<16><<<dim3(blocks), dim3(threads), 0, stream>>>(a); break;
    case 32: kv_append_kernel<32><<<dim3(blocks), dim3(threads), 0, stream>>>(a); break;
    default: return PKV_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// Copy-on-write block copies (mlxcel user guide "연속 배칭" §Paged KV 캐시와
// 프리픽스 공유): pair c copies the whole K and V tile set of block src[c]
// into block dst[c].  Workgroup (x, c) copies 256 16-byte units of pair c's
// [Hkv][block][row16] span; both sides are contiguous, so every access is
// coalesced.  The ids may live in pinned host memory (read once per thread).
// An 8-bit pool's scales ([Hkv][2][16] floats per block) travel with the codes.
template <int ROW16>
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(const int32_t *src, const int32_t *dst, uint4 *pool_k,
                                                             uint4 *pool_v, float *scales, int32_t num_blocks,
                                                             int32_t num_kv_heads) {
  const int64_t per_block = static_cast<int64_t>(num_kv_heads) * kBlockTokens * ROW16;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (u >= per_block) return;
  const int64_t s = src[blockIdx.y], d = dst[blockIdx.y];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  pool_k[d * per_block + u] = pool_k[s * per_block + u];
  pool_v[d * per_block + u] = pool_v[s * per_block + u];
  const int64_t per_scales = static_cast<int64_t>(num_kv_heads) * 2 * kBlockTokens;
  if (scales && u < per_scales) scales[d * per_scales + u] = scales[s * per_scales + u];
}

int pool_row16(const pkv_pool &pool) {
  const int elem = pool.dtype == PKV_F32 ? 4 : (pool.dtype == PKV_I8 ? 1 : 2);
  return pool.head_dim * elem / 16;
}

int launch_copy_blocks(const int32_t *src, const int32_t *dst, int32_t num_copies, const pkv_pool &pool,
                       hipStream_t stream) {
  if (num_copies <= 0) return PKV_OK;
  if (num_copies > 65535) return PKV_ERR_INVALID_ARG;
  const int row16 = pool_row16(pool);
  const int64_t per_block = static_cast<int64_t>(pool.num_kv_heads) * kBlockTokens * row16;
  const dim3 grid(static_cast<unsigned>((per_block + 255) / 256), static_cast<unsigned>(num_copies));
  uint4 *k = static_cast<uint4 *>(pool.k), *v = static_cast<uint4 *>(pool.v);
  float *sc = pool.dtype == PKV_I8 ? pool.scales : nullptr;
  const int nb = pool.num_blocks, hkv = pool.num_kv_heads;
  switch (row16) {
    case 4: kv_copy_blocks_kernel<4><<<grid, dim3(256), 0, stream>>>(src, dst, k, v, sc, nb, hkv); break;
    case 8: kv_copy_blocks_kernel<8><<<grid, dim3(256), 0, stream>>>(src, dst, k, v, sc, nb, hkv); break;
    case 16: kv_copy_blocks_kernel<16><<<grid, dim3(256), 0, stream>>>(src, dst, k, v, sc, nb, hkv); break;
    case 32: kv_copy_blocks_kernel<32><<<grid, dim3(256), 0, stream>>>(src, dst, k, v, sc, nb, hkv); break;
    default: return PKV_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
