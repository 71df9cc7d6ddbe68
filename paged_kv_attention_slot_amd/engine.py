"""A small step executor over the library: one KV pool, one block-pool
allocator, device copies of the slot metadata, and the per-step sequence

    lower the step plan (host C++)  ->  one async copy of the metadata
    ->  kv_append (HIP)  ->  paged_attend (HIP)

all on the caller's current stream.  It plays the role the lucebox blog
(§One scheduler, model-specific execution) gives the engine below the
scheduler: it owns the slots' block tables and lowers the selected prompt
chunks and decode rows into the packed layout the kernels read.

Metadata travels in one pinned host buffer per step (two buffers used in
turn, each reused only after its previous copy has finished).  The device
block tables are re-sent only when a table changed (a block was reserved,
released or truncated); slots that reserved decode headroom ahead of time
(§Admission and step planning: capacity for the prompt and rolling decode
headroom) send no table bytes on their decode steps.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import binding as B


@dataclass
class StepMeta:
    host: dict                # host int32 arrays from the lowering
    slot_mapping: object      # device int32 [T]
    query_start: object       # device int32 [B]
    query_len: object
    row_to_slot: object
    context_lens: object      # device int32 [max_slots]
    total_q: int
    max_query_len: int
    max_context_len: int


class _Staging:
    """A pinned host int32 buffer, its device twin and the event of its last copy."""

    def __init__(self, torch, device, n):
        self.host = torch.empty(n, dtype=torch.int32, pin_memory=True)
        self.dev = torch.empty(n, dtype=torch.int32, device=device)
        self.np = self.host.numpy()
        self.event = None


class PagedKVEngine:
    def __init__(self, *, num_blocks, num_kv_heads, num_q_heads, head_dim, dtype, max_slots,
                 max_blocks_per_seq, free_order=None, device="cuda", poison=True):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.num_q_heads = int(num_q_heads)
        self.pool = B.KVPool(num_blocks, num_kv_heads, head_dim, dtype, device=self.device, poison=poison)
        self.alloc = B.BlockAllocator(num_blocks, 16, max_slots, max_blocks_per_seq, free_order)
        self.max_slots, self.max_blocks_per_seq = int(max_slots), int(max_blocks_per_seq)
        self.d_block_tables = torch.zeros((self.max_slots, self.max_blocks_per_seq), dtype=torch.int32,
                                          device=self.device)
        self.h_block_tables = np.zeros((self.max_slots, self.max_blocks_per_seq), dtype=np.int32)
        self._tables_dirty = True
        self._staging = []
        self._turn = 0
        self._workspace = None

    # -- slot lifecycle (host allocator) --------------------------------
    def acquire(self, slot):
        self.alloc.acquire(slot)
        self._tables_dirty = True

    def release(self, slot):
        self.alloc.release(slot)
        self._tables_dirty = True

    def truncate(self, slot, new_len):
        self.alloc.truncate(slot, new_len)
        self._tables_dirty = True

    def reserve(self, slot, total_tokens):
        self.alloc.reserve(slot, total_tokens)
        self._tables_dirty = True

    # -- one step ---------------------------------------------------------
    def _stage(self, n):
        torch = self.torch
        if len(self._staging) < 2 or self._staging[0].np.size < n:
            cap = max(n, 4096)
            self._staging = [_Staging(torch, self.device, cap), _Staging(torch, self.device, cap)]
        st = self._staging[self._turn]
        self._turn ^= 1
        if st.event is not None:
            st.event.synchronize()          # the copy that last used this buffer is done
        return st

    def _refresh_tables(self):
        """Rebuild the host mirror of every table and send it to the device."""
        self.h_block_tables.fill(0)
        for slot in range(self.max_slots):
            t = self.alloc.slot_table(slot)
            if t:
                self.h_block_tables[slot, :len(t)] = t
        self.d_block_tables.copy_(self.torch.from_numpy(self.h_block_tables))
        self._tables_dirty = False

    def lower(self, entries) -> StepMeta:
        torch = self.torch
        nseg = len(entries)
        t = int(sum(e[1] for e in entries))
        # packed metadata: slot_mapping | query_start | query_len | row_to_slot | context_lens
        offs = [int(x) for x in np.cumsum([0, t, nseg, nseg, nseg, self.max_slots])]
        st = self._stage(offs[-1])
        h = st.np
        host = dict(slot_mapping=h[offs[0]:offs[1]], query_start=h[offs[1]:offs[2]],
                    query_len=h[offs[2]:offs[3]], row_to_slot=h[offs[3]:offs[4]],
                    context_lens=h[offs[4]:offs[5]])
        free_before = self.alloc.free_blocks()
        self.alloc.lower_step(entries, out=host)
        if self.alloc.free_blocks() != free_before:
            self._tables_dirty = True
        st.dev[:offs[-1]].copy_(st.host[:offs[-1]], non_blocking=True)
        if self._tables_dirty:
            self._refresh_tables()
        st.event = torch.cuda.Event()
        st.event.record()
        d = st.dev
        ql = host["query_len"]
        ctx = host["context_lens"][host["row_to_slot"]] if nseg else np.zeros(0, np.int32)
        snapshot = {k: np.array(v) for k, v in host.items()}
        snapshot["block_tables"] = self.h_block_tables
        return StepMeta(host=snapshot, slot_mapping=d[offs[0]:offs[1]], query_start=d[offs[1]:offs[2]],
                        query_len=d[offs[2]:offs[3]], row_to_slot=d[offs[3]:offs[4]],
                        context_lens=d[offs[4]:offs[5]], total_q=t,
                        max_query_len=int(ql.max()) if nseg else 0,
                        max_context_len=int(ctx.max()) if nseg else 0)

    def append(self, meta: StepMeta, k_new, v_new):
        B.kv_append(meta.slot_mapping, k_new, v_new, self.pool)

    def workspace_for(self, meta: StepMeta):
        n = B.workspace_bytes(len(meta.host["row_to_slot"]), meta.total_q, self.num_q_heads, meta.max_query_len,
                              meta.max_context_len, self.pool)
        if n == 0:
            return None
        if self._workspace is None or self._workspace.numel() < n:
            self._workspace = self.torch.empty(n, dtype=self.torch.uint8, device=self.device)
        return self._workspace

    def attend(self, meta: StepMeta, q, scale, out=None, out_dtype=None):
        torch = self.torch
        if out is None:
            out = torch.empty((meta.total_q, self.num_q_heads, self.pool.head_dim),
                              dtype=out_dtype or torch.float32, device=self.device)
        return B.paged_attend(q, meta.row_to_slot, meta.query_start, meta.query_len, meta.context_lens,
                              self.d_block_tables, self.pool, scale, max_query_len=meta.max_query_len,
                              max_context_len=meta.max_context_len, out=out, workspace=self.workspace_for(meta))

    def step(self, entries, k_new, v_new, q, scale, out=None, out_dtype=None):
        meta = self.lower(entries)
        self.append(meta, k_new, v_new)
        return self.attend(meta, q, scale, out=out, out_dtype=out_dtype), meta
