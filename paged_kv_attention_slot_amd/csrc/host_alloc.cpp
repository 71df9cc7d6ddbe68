// Host-side block-pool allocator, step lowering and metadata validator.
//
// "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog):
//   §Keeping track of each request - stable sequence slots, explicit
//     row-to-slot maps; retiring one slot moves no other.
//   §Paged KV and paged attention - fixed-size blocks in one shared pool,
//     per-sequence block tables, freed blocks reassigned to new requests,
//     explicit pool sizes rounded to whole blocks.
//   §Admission and step planning are different decisions - atomic
//     reservation of KV capacity.
// mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유 - decode
//   reserves blocks before the forward pass; requests that share a prompt
//   prefix store its blocks once (reference counts), a request adopts
//   another's blocks instead of prefilling them again, and a shared block is
//   copied (copy-on-write) only when one sequence's contents diverge in it.
//
// Every block in some table carries a reference count = the number of tables
// that hold it; a block returns to the free list when its count reaches 0.
// A slot may write only into blocks whose count is 1.  Appends land at
// positions >= the slot's length, and adoption shares only blocks below the
// adopted length, so the one block a step can find shared is the one that
// holds position `length` (the partial last block): lowering replaces it in
// that slot's table by a fresh block and lists the pair (old, new), whose
// contents the device copies before the append.
//
// The free list is a stack: the next block handed out is at the back of
// `free_`.  The constructor lays out `free_order` so that its first entry is
// handed out first; a released table is pushed in reverse so that its first
// block is on top (reused first).
#include <cstring>
#include <new>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t max_slots = 0;
  int32_t max_blocks = 0;
  std::vector<int32_t> free_;                 // stack; back = next out
  std::vector<std::vector<int32_t>> tables;   // per slot, logical order
  std::vector<int32_t> lengths;               // tokens per slot
  std::vector<char> in_use;
  std::vector<int32_t> refs;                  // per block: tables holding it
};

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool slot_ok(const pkv_alloc *a, int32_t s) { return a && s >= 0 && s < a->max_slots; }

int32_t extra_blocks(const pkv_alloc *a, int32_t slot, int64_t total_tokens) {
  int64_t need = ceil_div(total_tokens, a->block_size);
  int64_t have = static_cast<int64_t>(a->tables[slot].size());
  return need > have ? static_cast<int32_t>(need - have) : 0;
}

int32_t take_free(pkv_alloc *a) {
  int32_t b = a->free_.back();
  a->free_.pop_back();
  a->refs[b] = 1;
  return b;
}

void grow(pkv_alloc *a, int32_t slot, int32_t extra) {
  for (int32_t i = 0; i < extra; ++i) a->tables[slot].push_back(take_free(a));
}

// Drop the table's references past `keep`, last block first; blocks no other
// table holds go back on top of the free list.
void give_back(pkv_alloc *a, std::vector<int32_t> &table, size_t keep) {
  for (size_t i = table.size(); i > keep; --i) {
    int32_t b = table[i - 1];
    if (--a->refs[b] == 0) a->free_.push_back(b);
  }
  table.resize(keep);
}

// Index in the slot's table of a shared block that its next write would
// land in, or -1.
int64_t shared_write_block(const pkv_alloc *a, int32_t slot) {
  const std::vector<int32_t> &t = a->tables[slot];
  int64_t idx = a->lengths[slot] / a->block_size;
  if (idx < static_cast<int64_t>(t.size()) && a->refs[t[idx]] > 1) return idx;
  return -1;
}

}  // namespace

extern "C" {

int pkv_alloc_create(int32_t num_blocks, int32_t block_size, int32_t max_slots,
                     int32_t max_blocks_per_seq, const int32_t *free_order, pkv_alloc **out) {
  if (!out || num_blocks < 0 || block_size <= 0 || max_slots <= 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  std::vector<int32_t> order(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PKV_ERR_INVALID_ARG;
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pkv_alloc *a = new (std::nothrow) pkv_alloc;
  if (!a) return PKV_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->max_slots = max_slots;
  a->max_blocks = max_blocks_per_seq;
  a->free_.assign(order.rbegin(), order.rend());
  a->tables.resize(max_slots);
  a->lengths.assign(max_slots, 0);
  a->in_use.assign(max_slots, 0);
  a->refs.assign(num_blocks, 0);
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_alloc *alloc) { delete alloc; }

int pkv_slot_acquire(pkv_alloc *a, int32_t slot) {
  if (!slot_ok(a, slot)) return PKV_ERR_INVALID_ARG;
  if (a->in_use[slot]) return PKV_ERR_STATE;
  a->in_use[slot] = 1;
  a->tables[slot].clear();
  a->lengths[slot] = 0;
  return PKV_OK;
}

int pkv_slot_release(pkv_alloc *a, int32_t slot) {
  if (!slot_ok(a, slot)) return PKV_ERR_INVALID_ARG;
  if (!a->in_use[slot]) return PKV_ERR_STATE;
  give_back(a, a->tables[slot], 0);
  a->lengths[slot] = 0;
  a->in_use[slot] = 0;
  return PKV_OK;
}

int pkv_slot_truncate(pkv_alloc *a, int32_t slot, int32_t new_len) {
  if (!slot_ok(a, slot)) return PKV_ERR_INVALID_ARG;
  if (!a->in_use[slot]) return PKV_ERR_STATE;
  if (new_len < 0 || new_len > a->lengths[slot]) return PKV_ERR_INVALID_ARG;
  give_back(a, a->tables[slot], static_cast<size_t>(ceil_div(new_len, a->block_size)));
  a->lengths[slot] = new_len;
  return PKV_OK;
}

int pkv_reserve(pkv_alloc *a, int32_t slot, int32_t total_tokens) {
  if (!slot_ok(a, slot) || total_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (!a->in_use[slot]) return PKV_ERR_STATE;
  if (ceil_div(total_tokens, a->block_size) > a->max_blocks) return PKV_ERR_INVALID_ARG;
  int32_t extra = extra_blocks(a, slot, total_tokens);
  if (extra > static_cast<int32_t>(a->free_.size())) return PKV_ERR_NO_SPACE;
  grow(a, slot, extra);
  return PKV_OK;
}

int pkv_slot_adopt(pkv_alloc *a, int32_t slot, int32_t src_slot, int32_t num_tokens) {
  if (!slot_ok(a, slot) || !slot_ok(a, src_slot) || slot == src_slot || num_tokens < 0)
    return PKV_ERR_INVALID_ARG;
  if (!a->in_use[slot] || !a->in_use[src_slot]) return PKV_ERR_STATE;
  if (a->lengths[slot] != 0 || !a->tables[slot].empty()) return PKV_ERR_STATE;
  if (num_tokens > a->lengths[src_slot]) return PKV_ERR_INVALID_ARG;
  const size_t nb = static_cast<size_t>(ceil_div(num_tokens, a->block_size));
  const std::vector<int32_t> &src = a->tables[src_slot];
  for (size_t i = 0; i < nb; ++i) {
    a->tables[slot].push_back(src[i]);
    ++a->refs[src[i]];
  }
  a->lengths[slot] = num_tokens;
  return PKV_OK;
}

int32_t pkv_block_refs(const pkv_alloc *a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refs[block];
}

int pkv_lower_step_cow(pkv_alloc *a, int32_t num_entries, const int32_t *entry_slots,
                       const int32_t *entry_new_tokens, int32_t *slot_mapping, int32_t slot_mapping_cap,
                       int32_t *query_start, int32_t *query_len, int32_t *row_to_slot,
                       int32_t *context_lens, int32_t *block_tables, int32_t *copy_src,
                       int32_t *copy_dst, int32_t copy_cap, int32_t *num_copies) {
  if (!a || num_entries < 0 || (num_entries > 0 && (!entry_slots || !entry_new_tokens)))
    return PKV_ERR_INVALID_ARG;
  if (num_copies) *num_copies = 0;
  // Validate the whole step before changing anything.
  std::vector<char> seen(a->max_slots, 0);
  int64_t total_new = 0, total_extra = 0, copies = 0;
  for (int32_t e = 0; e < num_entries; ++e) {
    int32_t s = entry_slots[e], n = entry_new_tokens[e];
    if (!slot_ok(a, s) || n < 1 || seen[s]) return PKV_ERR_INVALID_ARG;
    if (!a->in_use[s]) return PKV_ERR_STATE;
    seen[s] = 1;
    int64_t total = static_cast<int64_t>(a->lengths[s]) + n;
    if (total > INT32_MAX || ceil_div(total, a->block_size) > a->max_blocks) return PKV_ERR_INVALID_ARG;
    total_new += n;
    total_extra += extra_blocks(a, s, total);
    if (shared_write_block(a, s) >= 0) ++copies;
  }
  if (slot_mapping && total_new > slot_mapping_cap) return PKV_ERR_INVALID_ARG;
  if (copies > 0 && (!copy_src || !copy_dst)) return PKV_ERR_STATE;
  if (copies > copy_cap && copies > 0) return PKV_ERR_INVALID_ARG;
  // An upper bound: a block shared by two writers of this step is copied by
  // the first only (the second then holds it alone).
  if (total_extra + copies > static_cast<int64_t>(a->free_.size())) return PKV_ERR_NO_SPACE;

  int32_t row = 0, ncopy = 0;
  for (int32_t e = 0; e < num_entries; ++e) {
    int32_t s = entry_slots[e], n = entry_new_tokens[e];
    int32_t first = a->lengths[s];
    const int64_t idx = shared_write_block(a, s);
    if (idx >= 0) {
      int32_t old = a->tables[s][idx];
      int32_t fresh = take_free(a);
      --a->refs[old];
      a->tables[s][idx] = fresh;
      copy_src[ncopy] = old;
      copy_dst[ncopy] = fresh;
      ++ncopy;
    }
    grow(a, s, extra_blocks(a, s, static_cast<int64_t>(first) + n));
    const std::vector<int32_t> &t = a->tables[s];
    if (slot_mapping) {
      for (int32_t p = first; p < first + n; ++p)
        slot_mapping[row + (p - first)] = t[p / a->block_size] * a->block_size + p % a->block_size;
    }
    if (query_start) query_start[e] = row;
    if (query_len) query_len[e] = n;
    if (row_to_slot) row_to_slot[e] = s;
    a->lengths[s] = first + n;
    row += n;
  }
  if (context_lens) {
    for (int32_t s = 0; s < a->max_slots; ++s) context_lens[s] = a->in_use[s] ? a->lengths[s] : 0;
  }
  if (block_tables) {
    std::memset(block_tables, 0, sizeof(int32_t) * static_cast<size_t>(a->max_slots) * a->max_blocks);
    for (int32_t s = 0; s < a->max_slots; ++s) {
      if (!a->in_use[s]) continue;
      const std::vector<int32_t> &t = a->tables[s];
      if (!t.empty())
        std::memcpy(block_tables + static_cast<size_t>(s) * a->max_blocks, t.data(), t.size() * sizeof(int32_t));
    }
  }
  if (num_copies) *num_copies = ncopy;
  return PKV_OK;
}

int pkv_lower_step(pkv_alloc *a, int32_t num_entries, const int32_t *entry_slots,
                   const int32_t *entry_new_tokens, int32_t *slot_mapping, int32_t slot_mapping_cap,
                   int32_t *query_start, int32_t *query_len, int32_t *row_to_slot,
                   int32_t *context_lens, int32_t *block_tables) {
  return pkv_lower_step_cow(a, num_entries, entry_slots, entry_new_tokens, slot_mapping, slot_mapping_cap,
                            query_start, query_len, row_to_slot, context_lens, block_tables, nullptr, nullptr, 0,
                            nullptr);
}

int32_t pkv_free_blocks(const pkv_alloc *a) { return a ? static_cast<int32_t>(a->free_.size()) : -1; }

int pkv_slot_info(const pkv_alloc *a, int32_t slot, int32_t *num_tokens, int32_t *num_blocks) {
  if (!slot_ok(a, slot)) return PKV_ERR_INVALID_ARG;
  bool used = a->in_use[slot];
  if (num_tokens) *num_tokens = used ? a->lengths[slot] : -1;
  if (num_blocks) *num_blocks = used ? static_cast<int32_t>(a->tables[slot].size()) : -1;
  return used ? PKV_OK : PKV_ERR_STATE;
}

int pkv_slot_table(const pkv_alloc *a, int32_t slot, int32_t *table, int32_t capacity) {
  if (!slot_ok(a, slot) || !table) return PKV_ERR_INVALID_ARG;
  if (!a->in_use[slot]) return PKV_ERR_STATE;
  const std::vector<int32_t> &t = a->tables[slot];
  if (static_cast<int64_t>(t.size()) > capacity) return PKV_ERR_INVALID_ARG;
  if (!t.empty()) std::memcpy(table, t.data(), t.size() * sizeof(int32_t));   // an empty table's data() may be null
  return PKV_OK;
}

int64_t pkv_pool_blocks_for_tokens(int64_t tokens, int32_t block_size) {
  if (tokens < 0 || block_size <= 0) return -1;
  return ceil_div(tokens, block_size);
}

int pkv_validate_step(int32_t total_q, int32_t num_segments, const int32_t *row_to_slot,
                      const int32_t *query_start, const int32_t *query_len, int32_t num_slots,
                      const int32_t *context_lens, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t block_size,
                      const int32_t *slot_mapping, int32_t num_tokens, int32_t *bad_index) {
  auto fail = [&](int32_t i) {
    if (bad_index) *bad_index = i;
    return PKV_ERR_INVALID_ARG;
  };
  if (bad_index) *bad_index = -1;
  if (total_q < 0 || num_segments < 0 || num_slots <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || block_size <= 0 || num_tokens < 0)
    return fail(-1);
  if (num_segments > 0 && (!row_to_slot || !query_start || !query_len || !context_lens || !block_tables))
    return fail(-1);
  // Segments tile disjoint row ranges inside [0, total_q); a slot appears once.
  std::vector<char> rows(total_q, 0), slots(num_slots, 0);
  for (int32_t b = 0; b < num_segments; ++b) {
    int32_t s = row_to_slot[b], r0 = query_start[b], n = query_len[b];
    if (s < 0 || s >= num_slots || slots[s]) return fail(b);
    slots[s] = 1;
    if (n < 1 || r0 < 0 || static_cast<int64_t>(r0) + n > total_q) return fail(b);
    for (int32_t r = r0; r < r0 + n; ++r) {
      if (rows[r]) return fail(b);
      rows[r] = 1;
    }
    int32_t L = context_lens[s];
    if (L < n || ceil_div(L, block_size) > max_blocks_per_seq) return fail(b);
    const int32_t *t = block_tables + static_cast<size_t>(s) * max_blocks_per_seq;
    for (int64_t j = 0; j < ceil_div(L, block_size); ++j)
      if (t[j] < 0 || t[j] >= num_blocks) return fail(b);
  }
  if (slot_mapping) {
    std::unordered_set<int32_t> seen;
    seen.reserve(static_cast<size_t>(num_tokens) * 2);
    int64_t limit = static_cast<int64_t>(num_blocks) * block_size;
    for (int32_t t = 0; t < num_tokens; ++t) {
      int32_t s = slot_mapping[t];
      if (s < 0 || s >= limit || !seen.insert(s).second) return fail(t);
    }
  }
  return PKV_OK;
}

const char *pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_NO_SPACE: return "not enough free KV blocks";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_STATE: return "slot in the wrong state";
    default: return "unknown status";
  }
}

}  // extern "C"
