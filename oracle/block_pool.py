"""Plain block-pool allocator and step lowering (oracle side, test infrastructure).

Follows "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog):
  * §Keeping track of each request: every admitted request owns a stable
    sequence slot holding its block table; the compact batch names slots
    through an explicit row-to-slot map, and retiring one slot moves no other.
  * §Paged KV and paged attention: fixed-size physical blocks in one shared
    pool; a block table maps a sequence's logical token positions to physical
    blocks; a finished sequence's blocks return to the pool and can be handed
    to a new request without moving the others; an explicit pool size is
    rounded to whole blocks.
  * §Admission and step planning are different decisions: KV capacity is
    reserved atomically (all or nothing).
mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유: decode reserves
its blocks before the forward pass.

Readings where the pages are silent (each listed in the design notes):
  * hand-out order: blocks are handed out in the order of a given free list
    (a seeded permutation for fragmentation); released blocks go back on top
    of the list (LIFO) in table order, so they are reused first, first block
    first;
  * slot_mapping entry of token position p of slot s is
    block_table[s][p // block_size] * block_size + p % block_size;
  * context_lens[s] counts the tokens in the cache after this step's append;
  * unused block-table entries and unused context_lens are 0.
"""
from __future__ import annotations

import numpy as np


class NoSpace(Exception):
    """Not enough free blocks; the allocator state is unchanged."""


def pool_blocks_for_tokens(tokens: int, block_size: int) -> int:
    """An explicit pool size in tokens, rounded up to whole blocks."""
    if tokens < 0 or block_size <= 0:
        raise ValueError("bad pool size")
    return -(-tokens // block_size)


class BlockPool:
    def __init__(self, num_blocks, block_size, max_slots, max_blocks_per_seq, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_slots = int(max_slots)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        # Top of the stack is the end of the list: the next block handed out.
        self.free = list(reversed(order))
        self.tables = {}     # slot -> list of physical blocks, in logical order
        self.lengths = {}    # slot -> tokens held

    # -- slot lifecycle -------------------------------------------------
    def acquire(self, slot):
        if not (0 <= slot < self.max_slots) or slot in self.tables:
            raise ValueError(f"slot {slot} not available")
        self.tables[slot] = []
        self.lengths[slot] = 0

    def release(self, slot):
        table = self.tables.pop(slot)
        del self.lengths[slot]
        for b in reversed(table):         # first block of the table ends on top
            self.free.append(b)

    def truncate(self, slot, new_len):
        """Drop tokens past new_len (rejected drafts); blocks no longer needed
        go back on top of the free list."""
        if not (0 <= new_len <= self.lengths[slot]):
            raise ValueError("bad truncate length")
        keep = -(-new_len // self.block_size)
        table = self.tables[slot]
        for b in reversed(table[keep:]):
            self.free.append(b)
        del table[keep:]
        self.lengths[slot] = new_len

    # -- reservation ----------------------------------------------------
    def _extra_blocks(self, slot, total_tokens):
        need = -(-total_tokens // self.block_size)
        return max(0, need - len(self.tables[slot]))

    def reserve(self, slot, total_tokens):
        """Grow the slot's table so it can hold total_tokens; all or nothing."""
        if -(-total_tokens // self.block_size) > self.max_blocks_per_seq:
            raise ValueError("sequence longer than the block table")
        extra = self._extra_blocks(slot, total_tokens)
        if extra > len(self.free):
            raise NoSpace(f"need {extra} blocks, {len(self.free)} free")
        for _ in range(extra):
            self.tables[slot].append(self.free.pop())

    # -- lowering one step ----------------------------------------------
    def lower_step(self, entries):
        """entries: [(slot, n_new)] in packed order.  Reserves (atomically for
        the whole step), assigns positions, advances lengths, and returns the
        kernel metadata as int32 numpy arrays."""
        seen = set()
        total_extra = 0
        for slot, n in entries:
            if slot not in self.tables or slot in seen or n < 1:
                raise ValueError(f"bad step entry ({slot}, {n})")
            seen.add(slot)
            total = self.lengths[slot] + n
            if -(-total // self.block_size) > self.max_blocks_per_seq:
                raise ValueError("sequence longer than the block table")
            total_extra += self._extra_blocks(slot, total)
        if total_extra > len(self.free):
            raise NoSpace(f"step needs {total_extra} blocks, {len(self.free)} free")
        for slot, n in entries:
            self.reserve(slot, self.lengths[slot] + n)

        slot_mapping, query_start, query_len, row_to_slot = [], [], [], []
        row = 0
        for slot, n in entries:
            table = self.tables[slot]
            first = self.lengths[slot]
            for p in range(first, first + n):
                slot_mapping.append(table[p // self.block_size] * self.block_size + p % self.block_size)
            query_start.append(row)
            query_len.append(n)
            row_to_slot.append(slot)
            row += n
            self.lengths[slot] = first + n
        context_lens, block_tables = self.snapshot()
        i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
        return dict(slot_mapping=i32(slot_mapping), query_start=i32(query_start),
                    query_len=i32(query_len), row_to_slot=i32(row_to_slot),
                    context_lens=context_lens, block_tables=block_tables)

    def snapshot(self):
        context_lens = np.zeros(self.max_slots, dtype=np.int32)
        block_tables = np.zeros((self.max_slots, self.max_blocks_per_seq), dtype=np.int32)
        for slot, table in self.tables.items():
            context_lens[slot] = self.lengths[slot]
            block_tables[slot, :len(table)] = table
        return context_lens, block_tables

    def free_count(self):
        return len(self.free)
