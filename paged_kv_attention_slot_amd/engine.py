"""A small step executor over the library: one KV pool, one block-pool
allocator, device copies of the slot metadata, and the per-step sequence

    lower the step plan (host C++)  ->  copy metadata to the device
    ->  kv_append (HIP)  ->  paged_attend (HIP)

all on the caller's current stream.  It plays the role the lucebox blog
(§One scheduler, model-specific execution) gives the engine below the
scheduler: it owns the slots' block tables and lowers the selected prompt
chunks and decode rows into the packed layout the kernels read.
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
    total_q: int
    max_query_len: int
    max_context_len: int


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
        self.d_context_lens = torch.zeros(self.max_slots, dtype=torch.int32, device=self.device)
        self.d_block_tables = torch.zeros((self.max_slots, self.max_blocks_per_seq), dtype=torch.int32,
                                          device=self.device)
        self._workspace = None

    # -- slot lifecycle (host allocator) --------------------------------
    def acquire(self, slot):
        self.alloc.acquire(slot)

    def release(self, slot):
        self.alloc.release(slot)

    def truncate(self, slot, new_len):
        self.alloc.truncate(slot, new_len)

    def reserve(self, slot, total_tokens):
        self.alloc.reserve(slot, total_tokens)

    # -- one step ---------------------------------------------------------
    def lower(self, entries) -> StepMeta:
        torch = self.torch
        host = self.alloc.lower_step(entries)
        dev = self.device

        def h2d(a):
            return torch.from_numpy(a).to(dev)

        self.d_context_lens.copy_(torch.from_numpy(host["context_lens"]))
        self.d_block_tables.copy_(torch.from_numpy(host["block_tables"]))
        ql = host["query_len"]
        ctx = host["context_lens"][host["row_to_slot"]] if len(ql) else np.zeros(0, np.int32)
        return StepMeta(host=host, slot_mapping=h2d(host["slot_mapping"]), query_start=h2d(host["query_start"]),
                        query_len=h2d(ql), row_to_slot=h2d(host["row_to_slot"]), total_q=int(ql.sum()),
                        max_query_len=int(ql.max()) if len(ql) else 0,
                        max_context_len=int(ctx.max()) if len(ctx) else 0)

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
        return B.paged_attend(q, meta.row_to_slot, meta.query_start, meta.query_len, self.d_context_lens,
                              self.d_block_tables, self.pool, scale, max_query_len=meta.max_query_len,
                              max_context_len=meta.max_context_len, out=out, workspace=self.workspace_for(meta))

    def step(self, entries, k_new, v_new, q, scale, out=None, out_dtype=None):
        meta = self.lower(entries)
        self.append(meta, k_new, v_new)
        return self.attend(meta, q, scale, out=out, out_dtype=out_dtype), meta
