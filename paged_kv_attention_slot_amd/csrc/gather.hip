// Gather of each sequence's visible KV window into contiguous blocks.
//
// mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유 compares its
// native block-table decode kernel with a gather path that rebuilds every
// sequence's visible window before attending, on every step, and reports the
// gap widening with context length.  This kernel is that rebuild, kept as an
// ablation: the block-table kernels never need it.  Segment b's logical
// blocks 0 .. ceil(L / 16) - 1 (L = context_lens[row_to_slot[b]]) are copied,
// whole, from the source pool through the slot's block table to blocks
// dst_block_start[b] + j of the destination pool, so the window is contiguous
// there and an identity table reads it.
//
// A block's K (and V) tile set is one contiguous [Hkv][16][row16] span on
// both sides, so each 16-byte unit moves with coalesced loads and stores,
// several in flight per lane.  Work is spread evenly over the flat list of
// (segment, block) pairs: a persistent grid of about 8 workgroups per CU
// builds the exclusive prefix of the segments' block counts in LDS and walks
// the list with a grid stride, so a long window is shared by as many
// workgroups as a short one and no workgroup is launched without work.
// Beyond kGatherLdsSegments segments (prefix too large for LDS) workgroup
// (b, y) takes blocks y, y + gridDim.y, ... of segment b instead.
#include "pagedkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct GatherArgs {
  const int32_t *row_to_slot;
  const int32_t *context_lens;
  const int32_t *block_tables;
  const int32_t *dst_block_start;
  const uint4 *src_k;
  const uint4 *src_v;
  uint4 *dst_k;
  uint4 *dst_v;
  const float *src_scales;  // 8-bit pools: per-row scales, [blocks][Hkv][2][16] (else null)
  float *dst_scales;
  int32_t num_slots;
  int32_t max_blocks;
  int32_t src_blocks;
  int32_t dst_blocks;
  int32_t num_kv_heads;
};

constexpr int kGatherLdsSegments = 4096;

#ifndef PKV_GATHER_NT
#define PKV_GATHER_NT 0  // 1: non-temporal stores; 2: non-temporal loads and stores
#endif
#ifndef PKV_GATHER_WGS
#define PKV_GATHER_WGS 2048  // persistent grid size
#endif

typedef unsigned int gather_u32x4 __attribute__((ext_vector_type(4)));

__device__ inline gather_u32x4 gather_load(const gather_u32x4 *p) {
  if constexpr (PKV_GATHER_NT >= 2) return __builtin_nontemporal_load(p);
  return *p;
}
__device__ inline void gather_store(gather_u32x4 *p, gather_u32x4 v) {
  if constexpr (PKV_GATHER_NT >= 1) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Segment b's block count (0 when its slot is out of range).
__device__ inline int gather_blocks(const GatherArgs &g, int b) {
  const int s = g.row_to_slot[b];
  if (s < 0 || s >= g.num_slots) return 0;
  int nb = (g.context_lens[s] + kBlockTokens - 1) / kBlockTokens;
  return nb < 0 ? 0 : (nb > g.max_blocks ? g.max_blocks : nb);
}

// Copy logical block j of segment b (slot s) to its place in the dst pool.
template <int ROW16>
__device__ inline void gather_one(const GatherArgs &g, int b, int s, int j) {
  constexpr int kBatch = 8;  // 16-byte units per array in flight per lane
  const int64_t per_block = static_cast<int64_t>(g.num_kv_heads) * kBlockTokens * ROW16;
  const int64_t phys = g.block_tables[static_cast<int64_t>(s) * g.max_blocks + j];
  const int64_t dst = static_cast<int64_t>(g.dst_block_start[b]) + j;
  if (phys < 0 || phys >= g.src_blocks || dst < 0 || dst >= g.dst_blocks) return;
  using V4 = gather_u32x4;
  const V4 *__restrict__ sk = reinterpret_cast<const V4 *>(g.src_k + phys * per_block);
  const V4 *__restrict__ sv = reinterpret_cast<const V4 *>(g.src_v + phys * per_block);
  V4 *__restrict__ dk = reinterpret_cast<V4 *>(g.dst_k + dst * per_block);
  V4 *__restrict__ dv = reinterpret_cast<V4 *>(g.dst_v + dst * per_block);
  for (int64_t u0 = threadIdx.x; u0 < per_block; u0 += 256 * kBatch) {
    V4 rk[kBatch], rv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t u = u0 + 256 * i;
      if (u < per_block) {
        rk[i] = gather_load(sk + u);
        rv[i] = gather_load(sv + u);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t u = u0 + 256 * i;
      if (u < per_block) {
        gather_store(dk + u, rk[i]);
        gather_store(dv + u, rv[i]);
      }
    }
  }
  if (g.src_scales) {
    const int64_t per_scales = static_cast<int64_t>(g.num_kv_heads) * 2 * kBlockTokens;
    for (int64_t u = threadIdx.x; u < per_scales; u += 256)
      g.dst_scales[dst * per_scales + u] = g.src_scales[phys * per_scales + u];
  }
}

template <int ROW16>
__global__ __launch_bounds__(256) void gather_flat_kernel(GatherArgs g, int num_segments) {
  __shared__ int32_t pre[kGatherLdsSegments + 1];  // exclusive prefix of block counts
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int per_t = (num_segments + 255) / 256;
  const int lo = tid * per_t;
  const int hi = lo + per_t < num_segments ? lo + per_t : num_segments;
  int sum = 0;
  for (int i = lo; i < hi; ++i) {
    pre[i] = sum;
    sum += gather_blocks(g, i);
  }
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 256 partial sums (Hillis-Steele)
  for (int d = 1; d < 256; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int before = part[tid] - sum;
  for (int i = lo; i < hi; ++i) pre[i] += before;
  if (tid == 255) pre[num_segments] = part[255];
  __syncthreads();
  const int total = pre[num_segments];
  for (int f = blockIdx.x; f < total; f += gridDim.x) {
    // the last segment whose first flat index is <= f (it has >= 1 block)
    int a = 0, z = num_segments - 1;
    while (a < z) {
      const int m = (a + z + 1) >> 1;
      if (pre[m] <= f) a = m; else z = m - 1;
    }
    gather_one<ROW16>(g, a, g.row_to_slot[a], f - pre[a]);
  }
}

template <int ROW16>
__global__ __launch_bounds__(256) void gather_window_kernel(GatherArgs g) {
  const int b = blockIdx.x;
  const int nb = gather_blocks(g, b);
  for (int j = blockIdx.y; j < nb; j += gridDim.y) gather_one<ROW16>(g, b, g.row_to_slot[b], j);
}

int launch_gather_window(const int32_t *row_to_slot, int32_t num_segments, const int32_t *context_lens,
                         const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq,
                         int32_t max_context_len, const int32_t *dst_block_start, const pkv_pool &src,
                         const pkv_pool &dst, hipStream_t stream) {
  if (num_segments == 0 || max_context_len == 0) return PKV_OK;
  const int row16 = pool_row16(src);
  const int64_t max_nb = (static_cast<int64_t>(max_context_len) + kBlockTokens - 1) / kBlockTokens;
  GatherArgs g;
  g.row_to_slot = row_to_slot;
  g.context_lens = context_lens;
  g.block_tables = block_tables;
  g.dst_block_start = dst_block_start;
  g.src_k = static_cast<const uint4 *>(src.k);
  g.src_v = static_cast<const uint4 *>(src.v);
  g.dst_k = static_cast<uint4 *>(dst.k);
  g.dst_v = static_cast<uint4 *>(dst.v);
  g.num_slots = num_slots;
  g.max_blocks = max_blocks_per_seq;
  g.src_blocks = src.num_blocks;
  g.dst_blocks = dst.num_blocks;
  g.num_kv_heads = src.num_kv_heads;
  const bool q8 = src.dtype == PKV_I8;
  g.src_scales = q8 ? src.scales : nullptr;
  g.dst_scales = q8 ? dst.scales : nullptr;
  if (row16 != 4 && row16 != 8 && row16 != 16 && row16 != 32) return PKV_ERR_UNSUPPORTED;
  if (num_segments <= kGatherLdsSegments) {
    // a persistent grid, never more workgroups than blocks
    int64_t wg = static_cast<int64_t>(num_segments) * max_nb;
    if (wg > PKV_GATHER_WGS) wg = PKV_GATHER_WGS;
    const dim3 grid(static_cast<unsigned>(wg));
    switch (row16) {
      case 4: gather_flat_kernel<4><<<grid, dim3(256), 0, stream>>>(g, num_segments); break;
      case 8: gather_flat_kernel<8><<<grid, dim3(256), 0, stream>>>(g, num_segments); break;
      case 16: gather_flat_kernel<16><<<grid, dim3(256), 0, stream>>>(g, num_segments); break;
      default: gather_flat_kernel<32><<<grid, dim3(256), 0, stream>>>(g, num_segments); break;
    }
  } else {
    const int64_t per = (static_cast<int64_t>(num_segments) * max_nb + 65535) / 65536;
    int64_t gy = (max_nb + per - 1) / per;
    if (gy > 65535) gy = 65535;
    if (gy < 1) gy = 1;
    const dim3 grid(static_cast<unsigned>(num_segments), static_cast<unsigned>(gy));
    switch (row16) {
      case 4: gather_window_kernel<4><<<grid, dim3(256), 0, stream>>>(g); break;
      case 8: gather_window_kernel<8><<<grid, dim3(256), 0, stream>>>(g); break;
      case 16: gather_window_kernel<16><<<grid, dim3(256), 0, stream>>>(g); break;
      default: gather_window_kernel<32><<<grid, dim3(256), 0, stream>>>(g); break;
    }
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
