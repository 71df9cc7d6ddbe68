// Randomized driver for the host allocator, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py (host code
// only).  Every entry point is called with valid and invalid arguments
// (bad slots, lengths past the table, repeated slots, small capacities,
// corrupted step metadata); after every call the reference counts must equal
// a recount over the live tables, and the free count must equal the number
// of unreferenced blocks.  Exit status 0 means no invariant broke; the
// sanitizers abort on any memory or undefined-behaviour error.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kBlocks = 96, kBS = 16, kSlots = 8, kMaxB = 12;

bool check(const pkv_alloc *a) {
  std::vector<int> count(kBlocks, 0);
  std::vector<int32_t> table(kMaxB);
  for (int s = 0; s < kSlots; ++s) {
    int32_t n = 0, nb = 0;
    if (pkv_slot_info(a, s, &n, &nb) != PKV_OK) continue;
    if (nb < 0 || nb > kMaxB || n < 0 || n > nb * kBS) return false;
    if (pkv_slot_table(a, s, table.data(), kMaxB) != PKV_OK) return false;
    for (int j = 0; j < nb; ++j) {
      if (table[j] < 0 || table[j] >= kBlocks) return false;
      ++count[table[j]];
    }
  }
  int unreferenced = 0;
  for (int b = 0; b < kBlocks; ++b) {
    if (pkv_block_refs(a, b) != count[b]) return false;
    unreferenced += count[b] == 0;
  }
  return pkv_free_blocks(a) == unreferenced && pkv_block_refs(a, -1) == -1 && pkv_block_refs(a, kBlocks) == -1;
}

}  // namespace

int main(int argc, char **argv) {
  const unsigned seed = argc > 1 ? static_cast<unsigned>(std::atoi(argv[1])) : 1u;
  std::mt19937 rng(seed);
  auto pick = [&](int lo, int hi) { return lo + static_cast<int>(rng() % static_cast<unsigned>(hi - lo + 1)); };
  std::vector<int32_t> order(kBlocks);
  for (int i = 0; i < kBlocks; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_alloc *bad = nullptr;
  if (pkv_alloc_create(-1, kBS, kSlots, kMaxB, nullptr, &bad) == PKV_OK || bad != nullptr) return 3;
  std::vector<int32_t> dup(order);
  dup[1] = dup[0];                                        // not a permutation
  if (pkv_alloc_create(kBlocks, kBS, kSlots, kMaxB, dup.data(), &bad) == PKV_OK) return 3;
  pkv_alloc *a = nullptr;
  if (pkv_alloc_create(kBlocks, kBS, kSlots, kMaxB, order.data(), &a) != PKV_OK) return 2;

  std::vector<int32_t> sm, qs, ql, rs, cl(kSlots), bt(kSlots * kMaxB), cs, cd;
  for (int it = 0; it < 20000; ++it) {
    const int s = pick(-1, kSlots);                       // -1 and kSlots are out of range
    switch (pick(0, 8)) {
      case 0: pkv_slot_acquire(a, s); break;
      case 1: pkv_slot_release(a, s); break;
      case 2: pkv_slot_truncate(a, s, pick(-5, 200)); break;
      case 3: pkv_reserve(a, s, pick(-5, kMaxB * kBS + 20)); break;
      case 4: pkv_slot_adopt(a, s, pick(-1, kSlots), pick(-5, 200)); break;
      case 5:
      case 6: {
        const int ne = pick(0, 5);
        std::vector<int32_t> es(ne), en(ne);
        int total = 0;
        for (int e = 0; e < ne; ++e) {
          es[e] = pick(-1, kSlots);
          en[e] = pick(-1, 40);
          total += en[e] > 0 ? en[e] : 0;
        }
        const int cap = pick(0, 2) == 0 ? pick(0, total) : total;   // sometimes too small
        sm.assign(total + 1, -7);
        qs.assign(ne + 1, -7);
        ql.assign(ne + 1, -7);
        rs.assign(ne + 1, -7);
        cs.assign(ne + 1, -7);
        cd.assign(ne + 1, -7);
        int32_t nc = -1;
        const bool cow = pick(0, 3) != 0;
        const int st = cow ? pkv_lower_step_cow(a, ne, es.data(), en.data(), sm.data(), cap, qs.data(), ql.data(),
                                                rs.data(), cl.data(), bt.data(), cs.data(), cd.data(), ne, &nc)
                           : pkv_lower_step(a, ne, es.data(), en.data(), sm.data(), cap, qs.data(), ql.data(),
                                            rs.data(), cl.data(), bt.data());
        if (st == PKV_OK) {
          int32_t bad = -2;
          const int v = pkv_validate_step(total, ne, rs.data(), qs.data(), ql.data(), kSlots, cl.data(), bt.data(),
                                          kMaxB, kBlocks, kBS, sm.data(), total, &bad);
          if (v != PKV_OK) {
            std::fprintf(stderr, "seed %u it %d: a successful lowering failed validation at %d\n", seed, it, bad);
            return 4;
          }
          if (total > 0) {                                 // corrupt one entry: must be rejected
            sm[pick(0, total - 1)] = kBlocks * kBS + pick(0, 5);
            if (pkv_validate_step(total, ne, rs.data(), qs.data(), ql.data(), kSlots, cl.data(), bt.data(), kMaxB,
                                  kBlocks, kBS, sm.data(), total, &bad) == PKV_OK)
              return 5;
          }
        }
        break;
      }
      case 7: {
        int32_t n = 0, nb = 0;
        pkv_slot_info(a, s, &n, &nb);
        std::vector<int32_t> small(2);
        pkv_slot_table(a, s, small.data(), 2);             // may be too small: an error, no overflow
        break;
      }
      default:
        pkv_validate_step(pick(-1, 10), pick(-1, 3), nullptr, nullptr, nullptr, kSlots, nullptr, nullptr, kMaxB,
                          kBlocks, kBS, nullptr, 0, nullptr);
        break;
    }
    if (!check(a)) {
      std::fprintf(stderr, "seed %u it %d: allocator invariants broken\n", seed, it);
      return 6;
    }
  }
  pkv_alloc_destroy(a);
  std::printf("ok\n");
  return 0;
}
