// Internal launch interfaces between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

constexpr int kBlockTokens = 16;  // tokens per pool block (the only block size built)

// Tokens per split-context partition of the decode path.  A multiple of the
// block size and at most 64 blocks (one block-table entry per lane).
#ifndef PKV_DECODE_PARTITION_TOKENS
#define PKV_DECODE_PARTITION_TOKENS 512
#endif
constexpr int32_t kDecodePartitionTokens = PKV_DECODE_PARTITION_TOKENS;

// K/V tiles each decode wavefront keeps in flight, and the decode grid size
// in wavefronts per compute unit.
#ifndef PKV_DECODE_STAGES
#define PKV_DECODE_STAGES 1
#endif
#ifndef PKV_DECODE_WAVES_PER_CU
#define PKV_DECODE_WAVES_PER_CU 16
#endif
// bf16 decode rows on MFMA tiles (decode_mfma.hip) instead of the vector-ALU
// decode kernel (decode.hip, always used for fp32 pools).
#ifndef PKV_DECODE_MFMA
#define PKV_DECODE_MFMA 1
#endif
// Minimum wavefronts per SIMD the MFMA decode kernel is compiled for (caps
// its registers so that many waves stay resident to hide memory latency).
#ifndef PKV_DECODE_MFMA_MIN_WAVES
#define PKV_DECODE_MFMA_MIN_WAVES 3
#endif
constexpr int kDecodeMfmaMinWaves = PKV_DECODE_MFMA_MIN_WAVES;
// Ablation knobs of the MFMA decode kernel (measurement builds only): one
// wavefront per query head instead of per GQA group, and one wavefront per
// row's whole context instead of split-context partitions.
#ifndef PKV_DECODE_NO_GQA_SHARE
#define PKV_DECODE_NO_GQA_SHARE 0
#endif
#ifndef PKV_DECODE_WHOLE_CONTEXT
#define PKV_DECODE_WHOLE_CONTEXT 0
#endif
#ifndef PKV_STREAM_LOADS
#define PKV_STREAM_LOADS 1
#endif
#if PKV_STREAM_LOADS
#define PKV_LDS_DMA_HINT "nt"
#else
#define PKV_LDS_DMA_HINT ""
#endif
// Chunk kernel tile loads: 0 cached, 1 nontemporal, 2 nontemporal for
// segments with one row tile (each K/V byte read by one workgroup per KV
// head) and cached for longer ones (row tiles re-read the same tiles).
#ifndef PKV_CHUNK_STREAM_LOADS
#define PKV_CHUNK_STREAM_LOADS 2
#endif
// Fence the chunk kernel's hand-interleaved matrix-core / vector-ALU steps
// so that the scheduler keeps them side by side (1), or leave the order of
// each phase to the compiler (0; measured faster with 32x32x16 tiles).
#ifndef PKV_CHUNK_INTERLEAVE
#define PKV_CHUNK_INTERLEAVE 0
#endif
// The chunk kernel's running row max may lag the true max by up to this much
// (log2 units) before O and l are rescaled: weights stay below 2^slack.
#ifndef PKV_CHUNK_RESCALE_SLACK
#define PKV_CHUNK_RESCALE_SLACK 8.0f
#endif
constexpr int kDecodeStages = PKV_DECODE_STAGES;
// K/V tiles in flight per wavefront in the MFMA decode kernel (1 to 3): the
// default, and the depth used when a launch has fewer than
// PKV_DECODE_FEW_WAVES wavefronts of work (each must then pull more bytes
// in flight).  Neither changes the arithmetic.
#ifndef PKV_DECODE_MFMA_STAGES
#define PKV_DECODE_MFMA_STAGES 1
#endif
#ifndef PKV_DECODE_MFMA_STAGES_FEW
#define PKV_DECODE_MFMA_STAGES_FEW 3
#endif
#ifndef PKV_DECODE_FEW_WAVES
#define PKV_DECODE_FEW_WAVES 400
#endif
constexpr int kDecodeMfmaStages = PKV_DECODE_MFMA_STAGES;

// 8-bit pools: tiles in flight per decode wavefront (half the bytes of a
// bf16 tile, so more of them), and when the launch has few waves.
#ifndef PKV_DECODE_Q8_STAGES
#define PKV_DECODE_Q8_STAGES 1
#endif
#ifndef PKV_DECODE_Q8_MIN_WAVES
#define PKV_DECODE_Q8_MIN_WAVES 3   // waves per SIMD the register budget must allow
#endif
#ifndef PKV_DECODE_Q8_STAGES_FEW
#define PKV_DECODE_Q8_STAGES_FEW 3
#endif

// Multi-row segments with fewer than this many 128-row tiles split their
// key range so that (row tiles x splits) reaches it; partial slots per
// (segment, KV head) = that target * 128 (chunk_split_slots).
// Multi-row segments whose (query row, head) pairs fit one verify
// wavefront (verify_col_tiles 16-wide MFMA column tiles) go to the streaming
// verify kernel (short speculative drafts); longer ones to the chunk kernel.
// The choice depends only on the segment's own (n, G) and the head dim.
// PKV_VERIFY_MAX_PAIRS, when set, lowers the limit (0 turns the path off).
// A verify wavefront's tiles are read once per launch (the launch's column
// tiles hold every segment's pairs, so no two wavefronts share a tile):
// nontemporal loads (PKV_VERIFY_STREAM_LOADS 1) keep them from displacing
// reused lines, and cold-cache steps stay as fast as warm ones.
#ifndef PKV_VERIFY_STREAM_LOADS
#define PKV_VERIFY_STREAM_LOADS 1
#endif
#if PKV_VERIFY_STREAM_LOADS
#define PKV_VERIFY_DMA_HINT "nt"
#else
#define PKV_VERIFY_DMA_HINT ""
#endif
// Verify prefetch depth (tiles in flight per wavefront) for launches with
// many wavefronts; launches with fewer than PKV_DECODE_FEW_WAVES take 3.
#ifndef PKV_VERIFY_SHALLOW_STAGES
#define PKV_VERIFY_SHALLOW_STAGES 1
#endif
#ifndef PKV_VERIFY_RESCALE_SLACK
#define PKV_VERIFY_RESCALE_SLACK 8.0f
#endif
#ifndef PKV_VERIFY_MAX_PAIRS
#define PKV_VERIFY_MAX_PAIRS 1024
#endif
constexpr int kVerifyPartitionTokens = PKV_DECODE_PARTITION_TOKENS;
// Column groups (wavefronts streaming the same partition) a verify segment
// may take.
#ifndef PKV_VERIFY_GROUPS
#define PKV_VERIFY_GROUPS 1
#endif
// 16-wide (row, head) pair tiles per verify wavefront (register budget).
__host__ __device__ constexpr int verify_col_tiles(int head_dim) { return head_dim == 64 ? 3 : 2; }
__host__ __device__ constexpr int verify_max_pairs(int head_dim) {
  return verify_col_tiles(head_dim) * 16 * PKV_VERIFY_GROUPS < PKV_VERIFY_MAX_PAIRS
             ? verify_col_tiles(head_dim) * 16 * PKV_VERIFY_GROUPS
             : PKV_VERIFY_MAX_PAIRS;
}
__host__ __device__ constexpr bool verify_segment(int n, int G, int head_dim) {
  return n > 1 && n * G <= verify_max_pairs(head_dim);
}
__host__ __device__ constexpr int verify_rows_cap(int G, int head_dim) {
  return G > 0 ? verify_max_pairs(head_dim) / G : 0;
}

// Fewest 64-token K/V tiles per key range of a split segment (1,024 keys):
// long enough to amortize a workgroup's prologue and its partial's merge.
#ifndef PKV_CHUNK_MIN_TILES_PER_SPLIT
#define PKV_CHUNK_MIN_TILES_PER_SPLIT 16
#endif
#ifndef PKV_CHUNK_SPLIT_ROW_TILES_D64
#define PKV_CHUNK_SPLIT_ROW_TILES_D64 64
#endif
#ifndef PKV_CHUNK_SPLIT_ROW_TILES_D128
#define PKV_CHUNK_SPLIT_ROW_TILES_D128 32
#endif
__host__ __device__ constexpr int chunk_split_row_tiles(int head_dim) {
  return head_dim == 64 ? PKV_CHUNK_SPLIT_ROW_TILES_D64 : PKV_CHUNK_SPLIT_ROW_TILES_D128;
}
__host__ __device__ constexpr int chunk_split_slots(int head_dim) { return chunk_split_row_tiles(head_dim) * 128; }

// Chunk kernel LDS ring: tokens per stage and stages, per head_dim.
#ifndef PKV_CHUNK_RING_TOK_D64
#define PKV_CHUNK_RING_TOK_D64 64
#endif
#ifndef PKV_CHUNK_RING_STAGES_D64
#define PKV_CHUNK_RING_STAGES_D64 4
#endif
// Chunk kernel occupancy hint: wavefronts per SIMD the register budget must
// allow (the second launch-bounds argument).
#ifndef PKV_CHUNK_MIN_WAVES_D64
#define PKV_CHUNK_MIN_WAVES_D64 2
#endif
#ifndef PKV_CHUNK_MIN_WAVES_D128
#define PKV_CHUNK_MIN_WAVES_D128 2
#endif
// Read the V operands midway through phase A (1) or at the start of phase B.
#ifndef PKV_CHUNK_EARLY_V_D64
#define PKV_CHUNK_EARLY_V_D64 1
#endif
#ifndef PKV_CHUNK_EARLY_V_D128
#define PKV_CHUNK_EARLY_V_D128 0
#endif
// Run a step's decode rows on an auxiliary stream beside its chunk kernels
// when the host knows both are present.
#ifndef PKV_CONCURRENT_DECODE
#define PKV_CONCURRENT_DECODE 1
#endif
#ifndef PKV_CHUNK_TABLE_WINDOW
#define PKV_CHUNK_TABLE_WINDOW 512
#endif
#ifndef PKV_CHUNK_RING_TOK_D128
#define PKV_CHUNK_RING_TOK_D128 32
#endif
#ifndef PKV_CHUNK_RING_STAGES_D128
#define PKV_CHUNK_RING_STAGES_D128 4
#endif
// floats per partial slot: D accumulators, running max, running sum, padding
// to a 16-byte multiple
template <int D>
constexpr int kChunkSlotFloats = D + 4;
constexpr int kDecodeWavesPerCU = PKV_DECODE_WAVES_PER_CU;

struct AttendArgs {
  const void *q;
  void *out;
  const void *k;
  const void *v;
  const int32_t *row_to_slot;
  const int32_t *query_start;
  const int32_t *query_len;
  const int32_t *context_lens;
  const int32_t *block_tables;
  float *part_acc;   // [part_rows][Hq][part_max][D]
  float *part_ml;    // [part_rows][Hq][part_max][2]  (running max in log2 units, sum)
  // Key-range partials of split multi-row segments: [Hkv][chunk_slots][D + 4].
  // Segment b's slots start after those of the split segments before it
  // (chunk_slot_base); M-row m, range s of it is slot base + m * splits + s.
  float *chunk_part;
  // Partition partials of verify rows: [verify_rows][Hq][part_max][D] and
  // [verify_rows][Hq][part_max][2]; segment b's rows start after those of the
  // verify segments before it (verify_row_base).
  float *verify_acc;
  float *verify_ml;
  int64_t chunk_slots;  // capacity of chunk_part per KV head, in slots
  int32_t verify_rows;  // capacity of the verify partials, in rows
  int32_t max_query;    // host bounds: a segment longer than max_query is skipped,
  int32_t max_context;  // a context longer than max_context is cut to it
  int32_t num_segments;
  int32_t num_slots;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t total_q;
  int32_t part_max;     // partitions per row the workspace holds
  int32_t multirow;     // 0: decode path takes query_len == 1 segments only; 1: every row
  int32_t out_bf16;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
  const float *scales;  // 8-bit pools: [num_blocks][Hkv][2][16] per-row scales, K then V (else null)
};

// KV append; optionally also copies stage_len int32 of step metadata from
// device-readable pinned host memory to a device buffer in the same launch.
int launch_kv_append(const int32_t *slot_mapping, const void *k_new, const void *v_new,
                     int32_t num_tokens, const pkv_pool &pool, hipStream_t stream,
                     const int32_t *stage_src = nullptr, int32_t *stage_dst = nullptr, int32_t stage_len = 0);

// Contiguous rebuild of each segment's visible window (the gather ablation).
int launch_gather_window(const int32_t *row_to_slot, int32_t num_segments, const int32_t *context_lens,
                         const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq,
                         int32_t max_context_len, const int32_t *dst_block_start, const pkv_pool &src,
                         const pkv_pool &dst, hipStream_t stream);

// 16-byte units per (token, head) row of a pool (head_dim x element bytes / 16).
int pool_row16(const pkv_pool &pool);

// Whole-block copies src[c] -> dst[c] (K and V, every head, with an 8-bit
// pool's scales); the ids may sit in device-readable pinned host memory.
int launch_copy_blocks(const int32_t *src, const int32_t *dst, int32_t num_copies, const pkv_pool &pool,
                       hipStream_t stream);

// Short multi-row segments (verify_segment) on the streaming verify kernel,
// plus the merge of their partitions when `need_merge`.
// `max_pairs` is the launch's largest segment's n * G and `work_waves` its
// exact count of (segment, KV head, partition) items when the host knows
// them, else -1: they pick the column tiles and prefetch depth per wavefront.
int launch_verify(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, bool need_merge,
                  int32_t max_pairs, int64_t work_waves, hipStream_t stream);

// Decode path (one query row per work item; split-context partitions) and,
// when `need_reduce` (some row has more than one partition), the partition
// reduce.  `max_context_len` sizes the grid only.
// `work_waves` is the launch's exact count of (row, KV head, partition)
// items when the host knows it, else -1.
// `decode_rows`: the count of query_len == 1 segments when the host knows
// it, else -1.
int launch_decode(const AttendArgs &a, int32_t dtype, int32_t head_dim, int32_t max_context_len, bool need_reduce,
                  int64_t work_waves, int32_t decode_rows, hipStream_t stream);

// Decode rows over an 8-bit pool (codes + per-row scales); in multi-row
// mode also the multi-row segments that the chunk kernel does not take.  `decode_rows`: the launch's count of
// query_len == 1 segments when the host knows it, else -1.
int launch_decode_q8(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, int stages,
                     int32_t decode_rows, hipStream_t stream);
int launch_decode_mfma(const AttendArgs &a, int32_t head_dim, int32_t max_context_len, int stages,
                       hipStream_t stream);

// Multi-row segments (query_len > 1) on MFMA tiles (bf16 pools, and 8-bit
// pools through fp16 tiles converted in LDS).  chunk_supported()
// tells whether this shape is built; otherwise multi-row segments take the
// decode path row by row.
bool chunk_supported(int32_t dtype, int32_t head_dim, int32_t group);
// Whether a multi-row segment of n rows and context L is cut into key
// ranges (whose partials the merge launch combines).  need_merge false
// skips that launch: the caller knows that no segment of the step is cut.
bool chunk_segment_splits(int32_t n, int32_t L, int32_t G, int32_t head_dim);
int launch_chunk(const AttendArgs &a, int32_t dtype, int32_t head_dim, int32_t max_query_len, int32_t max_context_len,
                 bool need_merge, hipStream_t stream);

int device_cu_count();

}  // namespace pkv
