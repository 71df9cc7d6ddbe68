/*
 * pagedkv.h - C ABI for the paged-KV mixed step on AMD MI355X (gfx950).
 *
 * The problem these calls solve is stated in "Continuous batching: Qwen3.8-27B
 * at 301 tok/s across five clients, up to 1.97x llama.cpp" (lucebox blog):
 *   - §Paged KV and paged attention: attention KV lives in fixed-size
 *     physical blocks of one shared pool; each sequence owns a block table
 *     mapping its logical token positions to physical blocks; attention walks
 *     that table in logical order with no gather or relocation of the cache;
 *     a finished sequence's blocks return to the pool without moving others;
 *     an explicit pool size is rounded to whole blocks.
 *   - §Keeping track of each request: every admitted request owns a stable
 *     sequence slot (block table + state); the compact batch names slots
 *     through an explicit row-to-slot map.
 *   - §Chunked prefill is a slot phase: each selected prompt chunk appends
 *     directly to its slot's paged KV.
 *   - §Packing unequal prompt chunks together: prompt chunks and decode rows
 *     share one packed token axis; per-query causal positions and block-table
 *     metadata let both attend in one pass.
 *   - §Admission and step planning are different decisions: KV capacity is
 *     reserved atomically.
 * mlxcel user guide "연속 배칭" (continuous batching), §Paged KV 캐시와
 * 프리픽스 공유: decode reserves its blocks before the forward pass.
 *
 * Conventions
 *   - All integers are int32 unless stated.  Pointers marked "device" are HIP
 *     device pointers; "host" pointers are ordinary process memory.
 *   - The caller owns every buffer (pool, inputs, outputs, workspace), and
 *     every stream and event the library uses.  The library never allocates
 *     or frees device memory and creates no streams or events.  Its only
 *     global state is the scratch of pkv_paged_attend_noalloc (a device array
 *     in the library's code object, one per GPU, and its device address,
 *     looked up once per GPU).
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  Argument errors are returned before
 *     anything is launched; launch failures return PKV_ERR_HIP; faults show
 *     up at the caller's next synchronisation.
 *   - Kernels do not validate metadata values.  They never access memory
 *     outside the buffers described below, whatever the metadata holds, but
 *     the result of invalid metadata is unspecified.  pkv_validate_step checks
 *     host copies of the metadata against every rule stated here.
 *
 * Pool layout (the pages leave the layout to the backend): K and V are two
 * separate device arrays, each [num_blocks][num_kv_heads][block_size][head_dim],
 * row-major, element type `dtype`.  One (block, KV head) tile of K or V is one
 * contiguous span of block_size * head_dim elements.  A flat pool token slot
 * s = block * block_size + offset names position `offset` of block `block`.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* a pointer, size or metadata value is invalid      */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not built: see "Supported shapes"        */
  PKV_ERR_NO_SPACE = -3,    /* allocator: not enough free blocks; state unchanged */
  PKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required         */
  PKV_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed         */
  PKV_ERR_STATE = -6        /* allocator: slot not in the required state          */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_I8 = 2 } pkv_dtype;

/* The shared KV pool.  Supported shapes: block_size 16; head_dim 64 or 128;
 * dtype PKV_F32, PKV_BF16 or PKV_I8.
 *
 * PKV_I8 is an 8-bit KV cache (the lucebox blog's R9700 DFlash2 section runs
 * its KV in an 8-bit format; the pages do not define one, so this is the
 * library's own).  k and v hold int8 codes in the layout above; scales holds
 * one float32 per (block, KV head, K or V, position):
 * [num_blocks][num_kv_heads][2][block_size], the block's 16 K scales of a KV
 * head followed by its 16 V scales, so one 128-byte run carries both halves
 * of a tile's scales.  A stored row (the head_dim values of one token and KV
 * head) stands for code * scale.  Rows are written by
 * pkv_kv_append from bf16 input:
 *   amax = max |x| over the row;  amax == 0 gives codes 0 and scale 0;
 *   otherwise inv = 127 / amax and scale = amax / 127 (float32, correctly
 *   rounded), code = round-half-to-even(float32(x * inv)) clamped to +-127.
 * Queries (q_packed) on an 8-bit pool are bf16 and are used as fp16 (exact
 * for |q| below 65504; magnitudes under 2^-14 keep fp16's subnormal
 * precision); output is float32 or bf16.
 * On an 8-bit pool, multi-row segments (prompt chunks, drafts) run on the
 * prompt-chunk kernel's 8-bit form: each staged tile's codes are converted
 * once per workgroup into fp16 tiles holding the codes exactly, so every
 * (row, head) pair of a 128-pair row tile shares one read of the window. */
typedef struct {
  void *k;              /* device [num_blocks][num_kv_heads][block_size][head_dim] */
  void *v;              /* device, same shape and dtype as k                        */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;        /* pkv_dtype */
  float *scales;        /* PKV_I8 only: device [num_blocks][num_kv_heads][2][block_size]
                           (index 0 = K, 1 = V); NULL for other dtypes              */
} pkv_pool;

/* ------------------------------------------------------------------ device */

/* KV append (lucebox blog §Chunked prefill is a slot phase: a chunk appends
 * directly to its slot's paged KV).  For every token t < num_tokens and every
 * KV head h, copies k_new[t][h][:] to K[s / bs][h][s % bs][:] and v_new[t][h][:]
 * to V[...] where s = slot_mapping[t].  A bit-exact copy: no conversion
 * (an 8-bit pool stores the row's codes and scale instead).
 *   slot_mapping  device int32 [num_tokens]; flat pool token slots.  Entries
 *                 must be distinct (a repeat is a write race); an entry outside
 *                 [0, num_blocks * block_size) is skipped (nothing written).
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_dim], pool dtype
 *                 (bf16 for a PKV_I8 pool: each row is quantized as stated
 *                 at pkv_pool, codes and scale stored together).
 * num_tokens == 0 is a no-op.  Returns PKV_OK, PKV_ERR_INVALID_ARG,
 * PKV_ERR_UNSUPPORTED or PKV_ERR_HIP. */
int pkv_kv_append(const int32_t *slot_mapping, const void *k_new, const void *v_new,
                  int32_t num_tokens, const pkv_pool *pool, void *stream);

/* Whole-block copies for copy-on-write (mlxcel user guide "연속 배칭" §Paged
 * KV 캐시와 프리픽스 공유: a shared block is copied only when a sequence
 * diverges in it).  For c < num_copies copies physical block src_blocks[c]
 * into dst_blocks[c]: K and V, every KV head, all block_size positions
 * (with their scales for an 8-bit pool); a bit-exact copy.  dst blocks must be distinct and differ from every src
 * block; a block id outside [0, num_blocks) skips that pair.
 *   src_blocks, dst_blocks   int32 [num_copies] in memory the device can read
 *                 (device memory, or pinned host memory from hipHostMalloc).
 * num_copies == 0 is a no-op.  Returns PKV_OK, PKV_ERR_INVALID_ARG,
 * PKV_ERR_UNSUPPORTED or PKV_ERR_HIP. */
int pkv_copy_blocks(const int32_t *src_blocks, const int32_t *dst_blocks, int32_t num_copies,
                    const pkv_pool *pool, void *stream);

/* Gather ablation (mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스
 * 공유: the native block-table decode is compared with a gather path that
 * rebuilds each sequence's visible window on every step).  Not needed by the
 * block-table path; it exists to measure what that path avoids.  For every
 * segment b with slot s = row_to_slot[b] and L = context_lens[s], copies the
 * slot's logical blocks j = 0 .. ceil(L / block_size) - 1, whole (K and V,
 * every head, scales of an 8-bit pool included), from src block
 * block_tables[s][j] to dst block
 * dst_block_start[b] + j.  Afterwards the window reads through the identity
 * table (dst_block_start[b], dst_block_start[b] + 1, ...) of the dst pool.
 *   row_to_slot, context_lens, block_tables, num_slots, max_blocks_per_seq
 *                 device, as for pkv_paged_attend.
 *   max_context_len   host upper bound of L over the segments (grid sizing).
 *   dst_block_start   device int32 [num_segments]; the ranges
 *                 [start, start + ceil(L / block_size)) must not overlap.
 *   src, dst      pools with equal heads, head_dim, dtype and block size;
 *                 blocks outside either pool are skipped.
 * Returns PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED or PKV_ERR_HIP. */
int pkv_gather_kv(const int32_t *row_to_slot, int32_t num_segments, const int32_t *context_lens,
                  const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq,
                  int32_t max_context_len, const int32_t *dst_block_start, const pkv_pool *src,
                  const pkv_pool *dst, void *stream);

/* Mixed-step paged attention (lucebox blog §Paged KV and paged attention and
 * §Packing unequal prompt chunks together).  The packed batch has
 * num_segments segments; segment b owns rows [query_start[b],
 * query_start[b] + query_len[b]) of q_packed and out, and the stable sequence
 * slot s = row_to_slot[b].  That slot holds L = context_lens[s] tokens in the
 * pool (this step's appended tokens included) listed by block_tables[s][0 ..
 * ceil(L / block_size)).  Row i of the segment sits at position
 * L - query_len[b] + i and attends to the slot's tokens 0 .. L - query_len[b] + i
 * (causal inside the chunk; a decode row, query_len 1, sees all L).  Query head
 * h reads KV head h / (num_q_heads / num_kv_heads).  For each row and head:
 *     out = sum_j softmax_j(scale * q . K_j) V_j
 * accumulated in fp32.
 *   q_packed      device [total_q][num_q_heads][head_dim], pool dtype (bf16
 *                 for a PKV_I8 pool, which attends over code * scale).
 *   row_to_slot, query_start, query_len   device int32 [num_segments].
 *                 query_len >= 1; segments cover disjoint rows; a slot appears
 *                 in at most one segment; query_len <= L.
 *   context_lens  device int32 [num_slots], indexed by slot.
 *   block_tables  device int32 [num_slots][max_blocks_per_seq], by slot.
 *   max_query_len, max_context_len   host upper bounds over the segments
 *                 (they size the grid and the workspace).  A bound below the
 *                 truth gives wrong but deterministic results and no access
 *                 outside the buffers: a segment with query_len >
 *                 max_query_len is skipped (its rows are not written), a
 *                 context longer than max_context_len is cut to it.
 *                 pkv_mixed_step rejects such bounds (PKV_ERR_INVALID_ARG).
 *   scale         softmax scale (1/sqrt(head_dim) for standard attention);
 *                 finite and > 0, else PKV_ERR_INVALID_ARG.
 *   out           device [total_q][num_q_heads][head_dim]; out_dtype PKV_F32,
 *                 or PKV_BF16 when the pool is bf16 or 8-bit (rounded to
 *                 nearest even).
 *   workspace     device scratch of at least pkv_paged_attend_workspace_bytes
 *                 bytes (may be NULL when that is 0); contents on entry ignored.
 * Rows not covered by any segment are not written.  Multi-row segments on
 * an fp32 pool run row by row on the decode path (any length; each row reads
 * its own window).  Returns PKV_OK, PKV_ERR_INVALID_ARG,
 * PKV_ERR_UNSUPPORTED (shape not built: num_q_heads / num_kv_heads > 8,
 * head_dim not 64/128, block_size not 16), PKV_ERR_WORKSPACE or
 * PKV_ERR_HIP. */
int pkv_paged_attend(const void *q_packed, int32_t total_q, int32_t num_q_heads,
                     const int32_t *row_to_slot, const int32_t *query_start,
                     const int32_t *query_len, int32_t num_segments,
                     const int32_t *context_lens, const int32_t *block_tables,
                     int32_t num_slots, int32_t max_blocks_per_seq,
                     int32_t max_query_len, int32_t max_context_len,
                     const pkv_pool *pool, float scale,
                     void *out, int32_t out_dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/* pkv_paged_attend without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The partials that pkv_paged_attend keeps
 * in the caller's workspace (split-context, key-range and draft partitions)
 * go instead to a scratch array inside the library: PKV_NOALLOC_SCRATCH_BYTES
 * of device memory on every GPU the library is loaded on, held until the
 * process ends.  A step whose pkv_paged_attend_workspace_bytes exceeds that
 * returns PKV_ERR_WORKSPACE before anything is launched.  The call allocates
 * nothing (no hipMalloc or hipFree).  Every call on one GPU shares that GPU's
 * scratch, and its contents on entry are ignored: calls that overlap on one
 * GPU (several streams or host threads) race, and the caller must order
 * them.  Other arguments, results and status codes as for pkv_paged_attend;
 * the results are bit-identical to pkv_paged_attend's. */
#define PKV_NOALLOC_SCRATCH_BYTES (128ull << 20)
int pkv_paged_attend_noalloc(const void *q_packed, int32_t total_q, int32_t num_q_heads,
                             const int32_t *row_to_slot, const int32_t *query_start,
                             const int32_t *query_len, int32_t num_segments,
                             const int32_t *context_lens, const int32_t *block_tables,
                             int32_t num_slots, int32_t max_blocks_per_seq,
                             int32_t max_query_len, int32_t max_context_len,
                             const pkv_pool *pool, float scale,
                             void *out, int32_t out_dtype, void *stream);

/* One step's device half in two kernel launches (lucebox blog §Chunked prefill
 * is a slot phase: the chunk appends to the slot's paged KV, then every packed
 * row attends over it).  The step's metadata, already lowered into pinned host
 * memory that the device can read (hipHostMalloc), is copied to device memory
 * by the append kernel itself - no separate copy call - and the attention
 * kernels read the device copy.  Equivalent to copying host_meta to dev_meta,
 * then pkv_copy_blocks (only when num_copies > 0: the copy-on-write pairs from
 * pkv_lower_step_cow, a third launch), then pkv_kv_append, then
 * pkv_paged_attend, on `stream`.
 *   host_meta     pinned host int32 [meta_len]; must stay unchanged until the
 *                 step's kernels have run (record an event after the call).
 *   dev_meta      device int32 [meta_len], overwritten.
 *   *_off         offsets (in int32) of each array inside host_meta/dev_meta:
 *                 slot_mapping [num_tokens], query_start / query_len /
 *                 row_to_slot [num_segments], context_lens [num_slots];
 *                 copy_off: copy_src [num_copies] then copy_dst [num_copies]
 *                 (read from host_meta; ignored when num_copies == 0).
 *   block_tables  device, as for pkv_paged_attend (kept on the device across
 *                 steps; only changed tables need re-sending).
 *   max_query_len, max_context_len   must hold for every segment (checked on
 *                 the host copy; PKV_ERR_INVALID_ARG otherwise).
 *   aux_stream, aux_fork_event, aux_join_event   optional, caller-owned
 *                 (hipStream_t, hipEvent_t as void*; default priority).  When
 *                 aux_stream is set (both events then required) and a step
 *                 holds both prompt-chunk segments and decode or draft rows,
 *                 the HBM-bound decode/draft kernels run on aux_stream beside
 *                 the chunk kernels on `stream`: the call records
 *                 aux_fork_event on `stream`, makes aux_stream wait on it,
 *                 records aux_join_event on aux_stream after its kernels and
 *                 makes `stream` wait on that, so all of the step's work is
 *                 still ordered before later work on `stream`.  The choice
 *                 changes no result bit.  Calls that share these objects must
 *                 not run concurrently from several host threads.  The events
 *                 only order the two streams; they may be created with
 *                 hipEventDisableSystemFence, which spares each record a
 *                 system-scope cache writeback.  NULL: one stream.
 * Other arguments as for pkv_kv_append and pkv_paged_attend; same status codes.
 * Argument errors (a bad scale included) are returned before anything is
 * appended. */
typedef struct {
  const int32_t *host_meta;
  int32_t *dev_meta;
  int32_t meta_len;
  int32_t slot_mapping_off, query_start_off, query_len_off, row_to_slot_off, context_lens_off;
  int32_t num_tokens, num_segments, num_slots, total_q, num_q_heads;
  int32_t max_blocks_per_seq, max_query_len, max_context_len;
  const void *k_new, *v_new, *q_packed;
  const int32_t *block_tables;
  float scale;
  void *out;
  int32_t out_dtype;
  void *workspace;
  size_t workspace_bytes;
  int32_t copy_off, num_copies;
  void *aux_stream;
  void *aux_fork_event, *aux_join_event;
} pkv_step_desc;

int pkv_mixed_step(const pkv_step_desc *step, const pkv_pool *pool, void *stream);

/* Bytes of workspace pkv_paged_attend needs for these bounds and this pool
 * (split-context partial results).  Pure host arithmetic; returns 0 when no
 * workspace is needed and (size_t)-1 for invalid arguments. */
size_t pkv_paged_attend_workspace_bytes(int32_t num_segments, int32_t total_q,
                                        int32_t num_q_heads, int32_t max_query_len,
                                        int32_t max_context_len, const pkv_pool *pool);

/* Tokens per split-context partition used by the decode path (a constant of
 * the build, so a row's reduction order depends on its own length only). */
int32_t pkv_decode_partition_tokens(void);

/* Static text for a status code. */
const char *pkv_status_str(int status);

/* -------------------------------------------------------- host allocator */

/* A host-only block-pool allocator with stable sequence slots (lucebox blog
 * §Keeping track of each request, §Paged KV and paged attention, §Admission
 * and step planning are different decisions).  It touches no device memory.
 * Blocks are handed out in the order of `free_order` (a permutation of
 * [0, num_blocks); NULL = ascending); blocks released by a slot go back on
 * top of the free list in table order, so they are reused first.  Not
 * thread-safe: one allocator per scheduler. */
typedef struct pkv_alloc pkv_alloc;

int pkv_alloc_create(int32_t num_blocks, int32_t block_size, int32_t max_slots,
                     int32_t max_blocks_per_seq, const int32_t *free_order /* host or NULL */,
                     pkv_alloc **out /* host */);
void pkv_alloc_destroy(pkv_alloc *alloc);

/* Mark `slot` in use with an empty table (PKV_ERR_STATE if already in use). */
int pkv_slot_acquire(pkv_alloc *alloc, int32_t slot);
/* Return all of the slot's blocks to the pool and free the slot. */
int pkv_slot_release(pkv_alloc *alloc, int32_t slot);
/* Shrink the slot to new_len tokens (rejected speculative drafts); blocks no
 * longer needed return to the pool. */
int pkv_slot_truncate(pkv_alloc *alloc, int32_t slot, int32_t new_len);
/* Grow the slot's table so it can hold total_tokens; all or nothing
 * (PKV_ERR_NO_SPACE leaves every table and the free list unchanged). */
int pkv_reserve(pkv_alloc *alloc, int32_t slot, int32_t total_tokens);

/* Lower one step.  entry_slots / entry_new_tokens (host, [num_entries]) name,
 * in packed order, the slots that advance and how many new tokens each
 * appends (1 for a decode row, the chunk length for a prompt chunk, the draft
 * count for speculative verification).  Reserves the blocks the step needs
 * (all or nothing over the whole step), advances each slot's length, and
 * writes these host arrays:
 *   slot_mapping  [sum of entry_new_tokens] (capacity slot_mapping_cap):
 *                 position p of slot s maps to
 *                 block_tables[s][p / block_size] * block_size + p % block_size;
 *   query_start, query_len, row_to_slot   [num_entries];
 *   context_lens  [max_slots]   tokens per slot after this step (0 if unused);
 *   block_tables  [max_slots][max_blocks_per_seq]   (unused entries 0).
 * Any output pointer may be NULL to skip it.  Returns PKV_OK,
 * PKV_ERR_INVALID_ARG (bad slot, repeated slot, n < 1, table overflow, small
 * capacity), PKV_ERR_STATE (slot not acquired) or PKV_ERR_NO_SPACE. */
int pkv_lower_step(pkv_alloc *alloc, int32_t num_entries, const int32_t *entry_slots,
                   const int32_t *entry_new_tokens, int32_t *slot_mapping,
                   int32_t slot_mapping_cap, int32_t *query_start, int32_t *query_len,
                   int32_t *row_to_slot, int32_t *context_lens, int32_t *block_tables);

/* Shared prefixes (mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스
 * 공유: requests with a common prompt prefix keep one copy of its KV blocks;
 * a later request adopts them by reference instead of prefilling again, and a
 * shared block is duplicated only when one sequence writes into it).
 * Every block held by a table has a reference count (the number of tables
 * holding it); release and truncate drop references, and a block goes back on
 * top of the free list when its count reaches 0.
 *
 * pkv_slot_adopt: `slot` (acquired, empty) takes the first
 * ceil(num_tokens / block_size) blocks of src_slot's table by reference and
 * holds num_tokens tokens (0 <= num_tokens <= src_slot's length).  No device
 * work: the adopted tokens are read in place.  Returns PKV_OK,
 * PKV_ERR_INVALID_ARG (bad slots, slot == src_slot, bad num_tokens) or
 * PKV_ERR_STATE (a slot not acquired, or `slot` not empty).
 * pkv_block_refs: reference count of a block (0 = free), -1 if out of range. */
int pkv_slot_adopt(pkv_alloc *alloc, int32_t slot, int32_t src_slot, int32_t num_tokens);
int32_t pkv_block_refs(const pkv_alloc *alloc, int32_t block);

/* pkv_lower_step with copy-on-write.  A slot's next write lands in the block
 * holding position `length`; when another table also holds that block, the
 * slot's table gets a fresh block in its place (taken before the step's
 * other new blocks) and the pair is listed:
 *   copy_src, copy_dst   host int32 [copy_cap]: entry c asks for block
 *                 copy_src[c] to be copied whole into block copy_dst[c]
 *                 (K and V, every head) BEFORE this step's append - see
 *                 pkv_copy_blocks and pkv_step_desc.copy_off;
 *   *num_copies   host, number of pairs written (at most one per entry, so
 *                 copy_cap = num_entries always suffices).
 * The fresh blocks count against the free list like any new block (all or
 * nothing).  pkv_lower_step is this call without copy buffers: it returns
 * PKV_ERR_STATE, changing nothing, when the step would need a copy. */
int pkv_lower_step_cow(pkv_alloc *alloc, int32_t num_entries, const int32_t *entry_slots,
                       const int32_t *entry_new_tokens, int32_t *slot_mapping,
                       int32_t slot_mapping_cap, int32_t *query_start, int32_t *query_len,
                       int32_t *row_to_slot, int32_t *context_lens, int32_t *block_tables,
                       int32_t *copy_src, int32_t *copy_dst, int32_t copy_cap,
                       int32_t *num_copies);

/* Current state: free block count; a slot's token count and block count
 * (-1 / PKV_ERR_STATE if not in use); copy of a slot's table (host out). */
int32_t pkv_free_blocks(const pkv_alloc *alloc);
int pkv_slot_info(const pkv_alloc *alloc, int32_t slot, int32_t *num_tokens, int32_t *num_blocks);
int pkv_slot_table(const pkv_alloc *alloc, int32_t slot, int32_t *table, int32_t capacity);

/* An explicit pool size in tokens rounded up to whole blocks (lucebox blog
 * §Paged KV and paged attention).  Returns -1 for negative tokens or
 * block_size <= 0. */
int64_t pkv_pool_blocks_for_tokens(int64_t tokens, int32_t block_size);

/* Check host copies of one step's metadata against every rule stated for
 * pkv_kv_append and pkv_paged_attend (tiling of the packed rows, slot ranges
 * and uniqueness, query_len <= L, table capacity, block ids in the pool,
 * slot_mapping range and uniqueness).  slot_mapping may be NULL.  Returns
 * PKV_OK or PKV_ERR_INVALID_ARG; *bad_index (host, may be NULL) receives the
 * index of the first offending entry. */
int pkv_validate_step(int32_t total_q, int32_t num_segments, const int32_t *row_to_slot,
                      const int32_t *query_start, const int32_t *query_len,
                      int32_t num_slots, const int32_t *context_lens,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      int32_t num_blocks, int32_t block_size,
                      const int32_t *slot_mapping, int32_t num_tokens, int32_t *bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
