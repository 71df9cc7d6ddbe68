// C-ABI entry points for the device side: argument checks, workspace sizing
// and kernel dispatch on the caller's stream.
#include <atomic>
#include <cmath>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

namespace {

bool pool_ok(const pkv_pool *p) {
  if (!p || !p->k || !p->v) return false;
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0 || p->block_size <= 0 || p->head_dim <= 0) return false;
  if (p->dtype == PKV_I8) return p->scales != nullptr;
  return p->dtype == PKV_F32 || p->dtype == PKV_BF16;
}

bool pool_supported(const pkv_pool *p) {
  return p->block_size == kBlockTokens && (p->head_dim == 64 || p->head_dim == 128);
}

// Multi-row segments go to the chunk kernels (bf16 pools, and 8-bit pools
// through fp16 tiles) when that shape is built; otherwise (fp32 pools) they
// take the decode path row by row.
bool multirow_on_decode_path(int32_t dtype, int32_t head_dim, int32_t group, int32_t max_query_len) {
  return max_query_len > 1 && !chunk_supported(dtype, head_dim, group);
}

struct WorkspaceLayout {
  int64_t rows = 0, part_max = 0, verify_rows = 0, chunk_slots = 0;
  size_t acc_bytes = 0, ml_bytes = 0, chunk_bytes = 0, vacc_bytes = 0, vml_bytes = 0;
  size_t decode_bytes() const { return acc_bytes + ml_bytes; }
  size_t total() const { return acc_bytes + ml_bytes + chunk_bytes + vacc_bytes + vml_bytes; }
};

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

WorkspaceLayout workspace_layout(int32_t num_segments, int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_query_len, int32_t max_context_len, int32_t dtype, int32_t group) {
  WorkspaceLayout w;
  const bool multirow = multirow_on_decode_path(dtype, head_dim, group, max_query_len);
  w.part_max = (static_cast<int64_t>(max_context_len) + kDecodePartitionTokens - 1) / kDecodePartitionTokens;
  if (w.part_max <= 1) {
    w.part_max = 1;
  } else {
    w.rows = multirow ? total_q : num_segments;
    const int64_t n = w.rows * num_q_heads * w.part_max;
    w.acc_bytes = static_cast<size_t>(n) * head_dim * sizeof(float);
    w.acc_bytes = (w.acc_bytes + 255) & ~static_cast<size_t>(255);
    w.ml_bytes = static_cast<size_t>(n) * 2 * sizeof(float);
    w.ml_bytes = (w.ml_bytes + 255) & ~static_cast<size_t>(255);
  }
  if (max_query_len > 1 && !multirow && group > 0) {
    // Multi-row segments cover disjoint rows of at least two each.
    const int64_t multi_segs = std::min<int64_t>(num_segments, total_q / 2);
    // Key-range partials of split multi-row segments (see chunk.hip): per KV
    // head, a split segment holds (M-rows x ranges) slots, at most one
    // split target's worth (chunk_split_slots), and each M-row has at most
    // as many ranges as the longest context allows.
    const int64_t kv_heads = num_q_heads / group;
    const int64_t kv_tiles = (static_cast<int64_t>(max_context_len) + 63) / 64;
    int64_t max_splits = (kv_tiles + PKV_CHUNK_MIN_TILES_PER_SPLIT - 1) / PKV_CHUNK_MIN_TILES_PER_SPLIT;
    max_splits = std::min<int64_t>(max_splits, chunk_split_row_tiles(head_dim));
    if (max_splits > 1) {
      w.chunk_slots = std::min<int64_t>(multi_segs * chunk_split_slots(head_dim),
                                        static_cast<int64_t>(total_q) * group * max_splits);
      w.chunk_bytes = align256(static_cast<size_t>(kv_heads * w.chunk_slots) * (head_dim + 4) * sizeof(float));
    }
    // Partition partials of the rows of verify segments (see verify.hip;
    // bf16 pools only).
    if (w.part_max > 1 && dtype == PKV_BF16) {
      w.verify_rows = std::min<int64_t>(total_q, multi_segs * verify_rows_cap(group, head_dim));
      const int64_t n = w.verify_rows * num_q_heads * w.part_max;
      w.vacc_bytes = align256(static_cast<size_t>(n) * head_dim * sizeof(float));
      w.vml_bytes = align256(static_cast<size_t>(n) * 2 * sizeof(float));
    }
  }
  return w;
}

// What the host knows about a step's segments: pkv_mixed_step reads it from
// the pinned host copy of the metadata; pkv_paged_attend (metadata on the
// device only) leaves `known` false and every kernel is launched.
struct StepFacts {
  bool known = false;
  int32_t decode_rows = 0;         // segments with query_len == 1
  int32_t chunk_segments = 0;      // segments with query_len > 1 on the chunk kernel
  int32_t chunk_split = 0;         // of those, segments cut into key ranges
  int32_t max_decode_context = 0;  // longest context among the decode rows
  int64_t decode_parts = 0;        // split-context partitions over the decode rows
  int32_t verify_segments = 0;     // multi-row segments on the verify kernel
  int32_t max_verify_context = 0;  // longest context among them
  int32_t max_verify_pairs = 0;    // largest n * G among them
  int64_t verify_parts = 0;        // their partitions
};

// A caller-owned second stream and fork/join events that let a step's
// HBM-bound kernels (decode rows, verify drafts) run beside its chunk
// kernels (pkv_step_desc.aux_*); absent, everything runs on one stream.
struct AuxStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

int attend(const void *q_packed, int32_t total_q, int32_t num_q_heads, const int32_t *row_to_slot,
           const int32_t *query_start, const int32_t *query_len, int32_t num_segments, const int32_t *context_lens,
           const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq, int32_t max_query_len,
           int32_t max_context_len, const pkv_pool *pool, float scale, void *out, int32_t out_dtype, void *workspace,
           size_t workspace_bytes, hipStream_t s, const StepFacts &facts, bool check_only = false,
           const AuxStream *aux = nullptr);

// Scratch of pkv_paged_attend_noalloc: the partials that pkv_paged_attend
// keeps in the caller's workspace, in a file-scope device array instead (one
// copy on every GPU the library is loaded on, held until the process ends).
// Host code never uses the array's name as an address: its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in noalloc_scratch_ptr.
constexpr size_t kNoallocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> noalloc_scratch_ptr[kMaxScratchDevices];

int noalloc_scratch_for_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return PKV_ERR_UNSUPPORTED;
  void *p = noalloc_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the same address on every lookup: a concurrent first call stores it too
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    noalloc_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

int pkv_kv_append(const int32_t *slot_mapping, const void *k_new, const void *v_new, int32_t num_tokens,
                  const pkv_pool *pool, void *stream) {
  if (!pool_ok(pool) || num_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (!pool_supported(pool)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping || !k_new || !v_new) return PKV_ERR_INVALID_ARG;
  return launch_kv_append(slot_mapping, k_new, v_new, num_tokens, *pool, static_cast<hipStream_t>(stream));
}

int pkv_copy_blocks(const int32_t *src_blocks, const int32_t *dst_blocks, int32_t num_copies, const pkv_pool *pool,
                    void *stream) {
  if (!pool_ok(pool) || num_copies < 0 || num_copies > 65535) return PKV_ERR_INVALID_ARG;
  if (!pool_supported(pool)) return PKV_ERR_UNSUPPORTED;
  if (num_copies == 0) return PKV_OK;
  if (!src_blocks || !dst_blocks) return PKV_ERR_INVALID_ARG;
  return launch_copy_blocks(src_blocks, dst_blocks, num_copies, *pool, static_cast<hipStream_t>(stream));
}

int pkv_gather_kv(const int32_t *row_to_slot, int32_t num_segments, const int32_t *context_lens,
                  const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq,
                  int32_t max_context_len, const int32_t *dst_block_start, const pkv_pool *src,
                  const pkv_pool *dst, void *stream) {
  if (!pool_ok(src) || !pool_ok(dst) || num_segments < 0 || num_segments > INT32_MAX / 2 || num_slots <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim || src->dtype != dst->dtype ||
      src->block_size != dst->block_size)
    return PKV_ERR_INVALID_ARG;
  if (!pool_supported(src)) return PKV_ERR_UNSUPPORTED;
  if (num_segments == 0 || max_context_len == 0) return PKV_OK;
  if (!row_to_slot || !context_lens || !block_tables || !dst_block_start) return PKV_ERR_INVALID_ARG;
  return launch_gather_window(row_to_slot, num_segments, context_lens, block_tables, num_slots, max_blocks_per_seq,
                              max_context_len, dst_block_start, *src, *dst, static_cast<hipStream_t>(stream));
}

size_t pkv_paged_attend_workspace_bytes(int32_t num_segments, int32_t total_q, int32_t num_q_heads,
                                        int32_t max_query_len, int32_t max_context_len, const pkv_pool *pool) {
  if (!pool || num_segments < 0 || total_q < 0 || num_q_heads <= 0 || max_query_len < 0 || max_context_len < 0 ||
      pool->head_dim <= 0)
    return static_cast<size_t>(-1);
  if (pool->num_kv_heads <= 0 || num_q_heads % pool->num_kv_heads != 0) return static_cast<size_t>(-1);
  return workspace_layout(num_segments, total_q, num_q_heads, pool->head_dim, max_query_len, max_context_len,
                          pool->dtype, num_q_heads / pool->num_kv_heads)
      .total();
}

// The causal mask and the running max assume a positive, finite scale.
static bool scale_ok(float scale) { return std::isfinite(scale) && scale > 0.f; }

int32_t pkv_decode_partition_tokens(void) { return kDecodePartitionTokens; }

int pkv_paged_attend(const void *q_packed, int32_t total_q, int32_t num_q_heads, const int32_t *row_to_slot,
                     const int32_t *query_start, const int32_t *query_len, int32_t num_segments,
                     const int32_t *context_lens, const int32_t *block_tables, int32_t num_slots,
                     int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_context_len,
                     const pkv_pool *pool, float scale, void *out, int32_t out_dtype, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return attend(q_packed, total_q, num_q_heads, row_to_slot, query_start, query_len, num_segments, context_lens,
                block_tables, num_slots, max_blocks_per_seq, max_query_len, max_context_len, pool, scale, out,
                out_dtype, workspace, workspace_bytes, static_cast<hipStream_t>(stream), StepFacts{});
}

int pkv_paged_attend_noalloc(const void *q_packed, int32_t total_q, int32_t num_q_heads, const int32_t *row_to_slot,
                             const int32_t *query_start, const int32_t *query_len, int32_t num_segments,
                             const int32_t *context_lens, const int32_t *block_tables, int32_t num_slots,
                             int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_context_len,
                             const pkv_pool *pool, float scale, void *out, int32_t out_dtype, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Argument errors first, then whether the step needs partials at all, then
  // whether they fit the scratch (the placeholder address is only compared,
  // never used), all before any HIP call.
  int st = attend(q_packed, total_q, num_q_heads, row_to_slot, query_start, query_len, num_segments, context_lens,
                  block_tables, num_slots, max_blocks_per_seq, max_query_len, max_context_len, pool, scale, out,
                  out_dtype, nullptr, 0, s, StepFacts{}, true);
  if (st == PKV_OK)      // no partials: nothing of the scratch is needed
    return attend(q_packed, total_q, num_q_heads, row_to_slot, query_start, query_len, num_segments, context_lens,
                  block_tables, num_slots, max_blocks_per_seq, max_query_len, max_context_len, pool, scale, out,
                  out_dtype, nullptr, 0, s, StepFacts{});
  if (st != PKV_ERR_WORKSPACE) return st;
  void *const placeholder = reinterpret_cast<void *>(static_cast<uintptr_t>(256));
  st = attend(q_packed, total_q, num_q_heads, row_to_slot, query_start, query_len, num_segments, context_lens,
              block_tables, num_slots, max_blocks_per_seq, max_query_len, max_context_len, pool, scale, out,
              out_dtype, placeholder, kNoallocScratchBytes, s, StepFacts{}, true);
  if (st != PKV_OK) return st;   // PKV_ERR_WORKSPACE: the step's partials exceed the scratch
  void *ws = nullptr;
  st = noalloc_scratch_for_current_device(&ws);
  if (st != PKV_OK) return st;
  return attend(q_packed, total_q, num_q_heads, row_to_slot, query_start, query_len, num_segments, context_lens,
                block_tables, num_slots, max_blocks_per_seq, max_query_len, max_context_len, pool, scale, out,
                out_dtype, ws, kNoallocScratchBytes, s, StepFacts{});
}

int pkv_mixed_step(const pkv_step_desc *d, const pkv_pool *pool, void *stream) {
  if (!d || !pool_ok(pool) || !d->host_meta || !d->dev_meta || d->meta_len < 0 || d->num_tokens < 0 ||
      d->num_segments < 0 || d->num_slots <= 0 || !scale_ok(d->scale))
    return PKV_ERR_INVALID_ARG;
  auto in_meta = [&](int32_t off, int64_t n) { return off >= 0 && off + n <= d->meta_len; };
  if (!in_meta(d->slot_mapping_off, d->num_tokens) || !in_meta(d->query_start_off, d->num_segments) ||
      !in_meta(d->query_len_off, d->num_segments) || !in_meta(d->row_to_slot_off, d->num_segments) ||
      !in_meta(d->context_lens_off, d->num_slots))
    return PKV_ERR_INVALID_ARG;
  if (d->num_copies < 0 || d->num_copies > 65535 ||
      (d->num_copies > 0 && !in_meta(d->copy_off, 2 * static_cast<int64_t>(d->num_copies))))
    return PKV_ERR_INVALID_ARG;
  if (!pool_supported(pool)) return PKV_ERR_UNSUPPORTED;
  if (d->num_tokens > 0 && (!d->k_new || !d->v_new)) return PKV_ERR_INVALID_ARG;
  // the second stream needs both events
  const bool has_aux = d->aux_stream != nullptr;
  if (has_aux && (!d->aux_fork_event || !d->aux_join_event)) return PKV_ERR_INVALID_ARG;
  // The host bounds must hold for every segment (the host copy of the
  // metadata is at hand here; pkv_paged_attend cannot check them).
  {
    const int32_t *hq = d->host_meta + d->query_len_off;
    const int32_t *hs = d->host_meta + d->row_to_slot_off;
    const int32_t *hl = d->host_meta + d->context_lens_off;
    for (int32_t b = 0; b < d->num_segments; ++b) {
      if (hq[b] > d->max_query_len) return PKV_ERR_INVALID_ARG;
      if (hs[b] >= 0 && hs[b] < d->num_slots && hl[hs[b]] > d->max_context_len) return PKV_ERR_INVALID_ARG;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t *m = d->dev_meta;
  // Every argument error is reported before the first launch.
  const int chk = attend(d->q_packed, d->total_q, d->num_q_heads, m + d->row_to_slot_off, m + d->query_start_off,
                         m + d->query_len_off, d->num_segments, m + d->context_lens_off, d->block_tables,
                         d->num_slots, d->max_blocks_per_seq, d->max_query_len, d->max_context_len, pool, d->scale,
                         d->out, d->out_dtype, d->workspace, d->workspace_bytes, s, StepFacts{}, true);
  if (chk != PKV_OK) return chk;
  if (d->num_copies > 0) {
    const int32_t *cp = d->host_meta + d->copy_off;
    const int sc = launch_copy_blocks(cp, cp + d->num_copies, d->num_copies, *pool, s);
    if (sc != PKV_OK) return sc;
  }
  const int st = launch_kv_append(d->host_meta + d->slot_mapping_off, d->k_new, d->v_new, d->num_tokens, *pool, s,
                                  d->host_meta, d->dev_meta, d->meta_len);
  if (st != PKV_OK) return st;
  StepFacts f;
  f.known = true;
  const int32_t *hq = d->host_meta + d->query_len_off;
  const int32_t *hs = d->host_meta + d->row_to_slot_off;
  const int32_t *hl = d->host_meta + d->context_lens_off;
  for (int32_t b = 0; b < d->num_segments; ++b) {
    if (hq[b] == 1) {
      ++f.decode_rows;
      if (hs[b] >= 0 && hs[b] < d->num_slots) {
        const int32_t L = hl[hs[b]];
        if (L > f.max_decode_context) f.max_decode_context = L;
        f.decode_parts += L > 0 ? (L + kDecodePartitionTokens - 1) / kDecodePartitionTokens : 1;
      }
    } else if (hq[b] > 1) {
      const int32_t G = d->num_q_heads / pool->num_kv_heads;
      if (pool->dtype == PKV_BF16 && verify_segment(hq[b], G, pool->head_dim)) {
        ++f.verify_segments;
        if (hq[b] * G > f.max_verify_pairs) f.max_verify_pairs = hq[b] * G;
        if (hs[b] >= 0 && hs[b] < d->num_slots) {
          const int32_t L = hl[hs[b]];
          if (L > f.max_verify_context) f.max_verify_context = L;
          f.verify_parts += L > 0 ? (L + kVerifyPartitionTokens - 1) / kVerifyPartitionTokens : 1;
        }
      } else {
        ++f.chunk_segments;
        // the unclamped context: at least the kernel's count of ranges
        if (hs[b] < 0 || hs[b] >= d->num_slots || chunk_segment_splits(hq[b], hl[hs[b]], G, pool->head_dim))
          ++f.chunk_split;
      }
    }
  }
  if (f.max_decode_context > d->max_context_len) f.max_decode_context = d->max_context_len;
  if (f.max_verify_context > d->max_context_len) f.max_verify_context = d->max_context_len;
  AuxStream aux;
  aux.stream = static_cast<hipStream_t>(d->aux_stream);
  aux.fork = static_cast<hipEvent_t>(d->aux_fork_event);
  aux.join = static_cast<hipEvent_t>(d->aux_join_event);
  return attend(d->q_packed, d->total_q, d->num_q_heads, m + d->row_to_slot_off, m + d->query_start_off,
                m + d->query_len_off, d->num_segments, m + d->context_lens_off, d->block_tables, d->num_slots,
                d->max_blocks_per_seq, d->max_query_len, d->max_context_len, pool, d->scale, d->out, d->out_dtype,
                d->workspace, d->workspace_bytes, s, f, false, has_aux ? &aux : nullptr);
}

}  // extern "C"

namespace pkv {
namespace {

int attend(const void *q_packed, int32_t total_q, int32_t num_q_heads, const int32_t *row_to_slot,
           const int32_t *query_start, const int32_t *query_len, int32_t num_segments, const int32_t *context_lens,
           const int32_t *block_tables, int32_t num_slots, int32_t max_blocks_per_seq, int32_t max_query_len,
           int32_t max_context_len, const pkv_pool *pool, float scale, void *out, int32_t out_dtype, void *workspace,
           size_t workspace_bytes, hipStream_t s, const StepFacts &facts, bool check_only, const AuxStream *aux) {
  if (!pool_ok(pool) || total_q < 0 || num_segments < 0 || num_q_heads <= 0 || num_slots <= 0 ||
      max_blocks_per_seq <= 0 || max_query_len < 0 || max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads != 0 || !scale_ok(scale)) return PKV_ERR_INVALID_ARG;
  if (out_dtype != PKV_F32 && !(out_dtype == PKV_BF16 && pool->dtype != PKV_F32)) return PKV_ERR_INVALID_ARG;
  if (!pool_supported(pool) || num_q_heads / pool->num_kv_heads > 8) return PKV_ERR_UNSUPPORTED;
  if (num_segments == 0 || total_q == 0) return PKV_OK;  // nothing to attend (nor to check further)
  if (!q_packed || !row_to_slot || !query_start || !query_len || !context_lens || !block_tables || !out)
    return PKV_ERR_INVALID_ARG;
  if (max_query_len > total_q) max_query_len = total_q;
  if (max_query_len < 1) max_query_len = 1;

  const int32_t group = num_q_heads / pool->num_kv_heads;
  const bool multirow = multirow_on_decode_path(pool->dtype, pool->head_dim, group, max_query_len);
  const WorkspaceLayout ws = workspace_layout(num_segments, total_q, num_q_heads, pool->head_dim, max_query_len,
                                              max_context_len, pool->dtype, group);
  if (ws.total() > 0 && (!workspace || workspace_bytes < ws.total())) return PKV_ERR_WORKSPACE;
  if (check_only) return PKV_OK;

  AttendArgs a{};
  a.q = q_packed;
  a.out = out;
  a.k = pool->k;
  a.v = pool->v;
  a.row_to_slot = row_to_slot;
  a.query_start = query_start;
  a.query_len = query_len;
  a.context_lens = context_lens;
  a.block_tables = block_tables;
  a.part_acc = ws.decode_bytes() ? static_cast<float *>(workspace) : nullptr;
  a.part_ml = ws.decode_bytes() ? reinterpret_cast<float *>(static_cast<char *>(workspace) + ws.acc_bytes) : nullptr;
  char *wsb = static_cast<char *>(workspace);
  a.chunk_part = ws.chunk_bytes ? reinterpret_cast<float *>(wsb + ws.decode_bytes()) : nullptr;
  a.verify_acc =
      ws.vacc_bytes ? reinterpret_cast<float *>(wsb + ws.decode_bytes() + ws.chunk_bytes) : nullptr;
  a.verify_ml =
      ws.vml_bytes ? reinterpret_cast<float *>(wsb + ws.decode_bytes() + ws.chunk_bytes + ws.vacc_bytes) : nullptr;
  a.verify_rows = static_cast<int32_t>(ws.verify_rows);
  a.chunk_slots = ws.chunk_slots;
  a.max_query = max_query_len;
  a.max_context = max_context_len;
  a.num_segments = num_segments;
  a.num_slots = num_slots;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.total_q = total_q;
  a.part_max = static_cast<int32_t>(ws.part_max);
  a.multirow = multirow ? 1 : 0;
  a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.scales = pool->dtype == PKV_I8 ? pool->scales : nullptr;

  // Multi-row segments on the chunk kernels, or on the verify kernel when
  // short (unless every multi-row segment goes row by row on the decode
  // path); decode rows on the decode kernels, whose grid and partition
  // reduce follow the decode rows' own longest context when the host knows
  // it.  Chunk work is matrix-bound, decode and verify work HBM-bound: when
  // the host knows a step has both kinds and the caller lent a second
  // stream, the HBM-bound kernels run on it beside the chunk kernels.
  const bool multi = max_query_len > 1 && !multirow;
  const bool run_chunk = multi && (!facts.known || facts.chunk_segments > 0);
  // (the verify kernel reads bf16 pools; other pools' short segments take the chunk kernel)
  const bool run_verify = multi && pool->dtype == PKV_BF16 && (!facts.known || facts.verify_segments > 0);
  const bool run_decode = !facts.known || multirow || facts.decode_rows > 0;
  const int32_t decode_ctx = facts.known && !multirow ? facts.max_decode_context : max_context_len;
  const bool need_reduce = decode_ctx > kDecodePartitionTokens;
  const int32_t verify_ctx = facts.known ? facts.max_verify_context : max_context_len;
  const bool need_merge = verify_ctx > kVerifyPartitionTokens;
  const int64_t work_waves = facts.known && !multirow ? facts.decode_parts * pool->num_kv_heads : -1;
  auto launch_streaming = [&](hipStream_t st) {
    int r = PKV_OK;
    if (run_verify)
      r = launch_verify(a, pool->head_dim, verify_ctx, need_merge, facts.known ? facts.max_verify_pairs : -1,
                        facts.known ? facts.verify_parts * pool->num_kv_heads : -1, st);
    if (r == PKV_OK && run_decode)
      r = launch_decode(a, pool->dtype, pool->head_dim, decode_ctx, need_reduce, work_waves,
                        facts.known ? facts.decode_rows : -1, st);
    return r;
  };
  if (run_chunk && (run_decode || run_verify) && facts.known && aux && PKV_CONCURRENT_DECODE) {
    if (hipEventRecord(aux->fork, s) != hipSuccess || hipStreamWaitEvent(aux->stream, aux->fork, 0) != hipSuccess)
      return PKV_ERR_HIP;
    const int sd = launch_streaming(aux->stream);
    // the join is recorded even after a failed launch, so `s` never waits
    // on a stale event
    if (hipEventRecord(aux->join, aux->stream) != hipSuccess) return PKV_ERR_HIP;
    const int sc =
        launch_chunk(a, pool->dtype, pool->head_dim, max_query_len, max_context_len, facts.chunk_split > 0, s);
    if (hipStreamWaitEvent(s, aux->join, 0) != hipSuccess) return PKV_ERR_HIP;
    return sd != PKV_OK ? sd : sc;
  }
  if (run_chunk) {
    const int st = launch_chunk(a, pool->dtype, pool->head_dim, max_query_len, max_context_len,
                                !facts.known || facts.chunk_split > 0, s);
    if (st != PKV_OK) return st;
  }
  return launch_streaming(s);
}

}  // namespace
}  // namespace pkv
