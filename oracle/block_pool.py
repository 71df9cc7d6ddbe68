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
its blocks before the forward pass; requests sharing a prompt prefix keep one
copy of its blocks, counted by reference; a request adopts another's blocks
instead of prefilling them, and a shared block is duplicated (copy-on-write)
only when one sequence's contents diverge inside it.

Readings where the pages are silent (each listed in the design notes):
  * hand-out order: blocks are handed out in the order of a given free list
    (a seeded permutation for fragmentation); released blocks go back on top
    of the list (LIFO) in table order, so they are reused first, first block
    first;
  * slot_mapping entry of token position p of slot s is
    block_table[s][p // block_size] * block_size + p % block_size;
  * context_lens[s] counts the tokens in the cache after this step's append;
  * unused block-table entries and unused context_lens are 0;
  * a block's reference count is the number of tables holding it; it goes
    back on the free list when the count drops to 0;
  * adopting n tokens shares the first ceil(n / block_size) blocks;
  * a slot may write only into a block no other table holds.  Before a step
    writes into a shared block, the writer takes a fresh block off the free
    list (before the step's other new blocks for that slot), its table points
    there, and the pair (old, fresh) is listed for a whole-block copy that
    runs before the append.  Slots are handled in packed order, so when two
    writers of one step share a block, the first copies it and the second
    then holds the original alone.
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
        self.refs = [0] * self.num_blocks   # block -> number of tables holding it

    def _take(self):
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def _drop(self, blocks):
        """Drop one reference to each block, last block first."""
        for b in reversed(blocks):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)

    # -- slot lifecycle -------------------------------------------------
    def acquire(self, slot):
        if not (0 <= slot < self.max_slots) or slot in self.tables:
            raise ValueError(f"slot {slot} not available")
        self.tables[slot] = []
        self.lengths[slot] = 0

    def release(self, slot):
        table = self.tables.pop(slot)
        del self.lengths[slot]
        self._drop(table)                 # first block of the table ends on top

    def truncate(self, slot, new_len):
        """Drop tokens past new_len (rejected drafts); blocks no longer needed
        go back on top of the free list."""
        if not (0 <= new_len <= self.lengths[slot]):
            raise ValueError("bad truncate length")
        keep = -(-new_len // self.block_size)
        table = self.tables[slot]
        self._drop(table[keep:])
        del table[keep:]
        self.lengths[slot] = new_len

    def adopt(self, slot, src_slot, num_tokens):
        """`slot` (acquired, empty) takes src_slot's first num_tokens tokens by
        reference: no copy, the blocks are shared."""
        if slot == src_slot or self.tables[slot] or self.lengths[slot]:
            raise ValueError("adopt needs an empty slot distinct from the source")
        if not (0 <= num_tokens <= self.lengths[src_slot]):
            raise ValueError("bad adopt length")
        shared = self.tables[src_slot][: -(-num_tokens // self.block_size)]
        for b in shared:
            self.refs[b] += 1
        self.tables[slot] = list(shared)
        self.lengths[slot] = num_tokens

    def _shared_write_index(self, slot):
        """Index in the slot's table of the block its next token lands in, if
        another table also holds that block; else None."""
        i = self.lengths[slot] // self.block_size
        table = self.tables[slot]
        if i < len(table) and self.refs[table[i]] > 1:
            return i
        return None

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
            self.tables[slot].append(self._take())

    # -- lowering one step ----------------------------------------------
    def lower_step(self, entries):
        """entries: [(slot, n_new)] in packed order.  Reserves (atomically for
        the whole step), assigns positions, advances lengths, and returns the
        kernel metadata as int32 numpy arrays, with the copy-on-write pairs
        as copy_src / copy_dst."""
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
            if self._shared_write_index(slot) is not None:
                total_extra += 1          # an upper bound (see the module notes)
        if total_extra > len(self.free):
            raise NoSpace(f"step needs {total_extra} blocks, {len(self.free)} free")
        copies = []
        for slot, n in entries:
            i = self._shared_write_index(slot)
            if i is not None:
                old = self.tables[slot][i]
                fresh = self._take()
                self.refs[old] -= 1
                self.tables[slot][i] = fresh
                copies.append((old, fresh))
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
                    context_lens=context_lens, block_tables=block_tables,
                    copy_src=i32([c[0] for c in copies]), copy_dst=i32([c[1] for c in copies]))

    def snapshot(self):
        context_lens = np.zeros(self.max_slots, dtype=np.int32)
        block_tables = np.zeros((self.max_slots, self.max_blocks_per_seq), dtype=np.int32)
        for slot, table in self.tables.items():
            context_lens[slot] = self.lengths[slot]
            block_tables[slot, :len(table)] = table
        return context_lens, block_tables

    def free_count(self):
        return len(self.free)
