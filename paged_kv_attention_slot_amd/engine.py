"""A small step executor over the library: one KV pool, one block-pool
allocator, device copies of the slot metadata, and the per-step sequence

    lower the step plan (host C++)  ->  one async copy of the metadata
    ->  [copy-on-write block copies (HIP)]  ->  kv_append (HIP)
    ->  paged_attend (HIP)

all on the caller's current stream.  It plays the role the lucebox blog
(§One scheduler, model-specific execution) gives the engine below the
scheduler: it owns the slots' block tables and lowers the selected prompt
chunks and decode rows into the packed layout the kernels read.

Metadata travels in one pinned host buffer per step, copied on the step's
own stream (so stream order protects the device copy).  A ring of buffers
is used in turn; a host buffer is rewritten only after the copy that last
read it has finished, which with a ring this deep has always happened
already - the host never sleeps on the GPU inside the step loop.  One-call
steps share one completion event per group of STEP_GROUP steps (an event
record costs the GPU a few microseconds per step); a buffer whose group is
still open when its turn comes records the group's event first.  The device
block tables are re-sent only when a table changed (a block was reserved,
released or truncated); slots that reserved decode headroom ahead of time
(§Admission and step planning: capacity for the prompt and rolling decode
headroom) send no table bytes on their decode steps.

Shared prompt prefixes (mlxcel user guide "연속 배칭" §Paged KV 캐시와
프리픽스 공유): `adopt` lets an empty slot take another slot's first tokens
by reference; when a step writes into a block that another table still
holds, the lowering hands the writer a fresh block and lists the pair, and
the block is copied on the device before the append.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import binding as B


_DEV_FIELDS = ("slot_mapping", "query_start", "query_len", "row_to_slot", "context_lens", "copy_src", "copy_dst")


@dataclass
class StepMeta:
    """A lowered step.  The device arrays - slot_mapping [T], query_start /
    query_len / row_to_slot [B], context_lens [max_slots], copy_src /
    copy_dst [num_copies] (copy-on-write pairs), all int32 - are views of the
    staged device copy, made on first use (the one-call path never needs
    them)."""
    host: dict                # host int32 arrays from the lowering
    dev: object               # device int32 staging buffer holding the arrays
    offs: tuple               # start of each array in `dev`, in _DEV_FIELDS order, then the end
    stream: object            # handle of the stream the step was lowered on
    total_q: int
    max_query_len: int
    max_context_len: int
    num_copies: int = 0
    copy_off: int = 0         # offset of copy_src in the staged metadata

    def __getattr__(self, name):
        if name in _DEV_FIELDS:
            i = _DEV_FIELDS.index(name)
            view = self.dev[self.offs[i]:self.offs[i + 1]]
            setattr(self, name, view)
            return view
        raise AttributeError(name)


@dataclass
class PreparedStep:
    """A lowered step and its pkv_mixed_step descriptor (see prepare_fused)."""
    desc: object
    staging: object
    stream: object
    meta: StepMeta
    out: object
    keep: tuple


class _Staging:
    """A pinned host int32 buffer, its device twin, and the event recorded
    after the copy that last read the host buffer."""

    def __init__(self, torch, device, n):
        self.host = torch.empty(n, dtype=torch.int32, pin_memory=True)
        self.dev = torch.empty(n, dtype=torch.int32, device=device)
        self.np = self.host.numpy()
        self.addr = self.host.data_ptr()
        self.own = torch.cuda.Event()   # this buffer's event (split-call steps)
        self.copied = self.own          # the event that marks the buffer's last reader done
        self.used = False


class PagedKVEngine:
    STAGING_RING = 16
    STEP_GROUP = 8          # one-call steps per completion event (<= STAGING_RING / 2)
    use_aux_stream = True   # lend pkv_mixed_step a second stream (decode beside chunks)

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
        self._group_event = None        # event shared by the open group of one-call steps
        self._group_n = 0
        self._group_stream = None
        self._workspace = None
        self._ws_key = None
        self._ws_bytes = 0
        self._aux = None        # second stream and fork/join events lent to pkv_mixed_step
        self._entries = None    # the last step plan, its int32 arrays and their addresses

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

    def adopt(self, slot, src_slot, num_tokens):
        """`slot` (acquired, empty) shares src_slot's first num_tokens tokens."""
        self.alloc.adopt(slot, src_slot, num_tokens)
        self._tables_dirty = True

    # -- one step ---------------------------------------------------------
    def _stage(self, n):
        torch = self.torch
        if not self._staging or self._staging[0].np.size < n:
            cap = max(n, 4096)
            self._staging = [_Staging(torch, self.device, cap) for _ in range(self.STAGING_RING)]
        st = self._staging[self._turn]
        self._turn = (self._turn + 1) % self.STAGING_RING
        if st.used:
            if st.copied is self._group_event:
                self._close_group()         # its group is still open: record the event now
            if not st.copied.query():
                st.copied.synchronize()     # the kernels that last read this host buffer are done
        return st

    def _close_group(self):
        if self._group_event is not None and self._group_n > 0:
            self._group_event.record(self._group_stream)
        self._group_event = None
        self._group_n = 0

    def _refresh_tables(self):
        """Rebuild the host mirror of every table and send it to the device.
        The mirror is a new array each time: earlier steps' snapshots keep the
        tables they were lowered with."""
        tables = np.zeros_like(self.h_block_tables)
        for slot in range(self.max_slots):
            t = self.alloc.slot_table(slot)
            if t:
                tables[slot, :len(t)] = t
        self.h_block_tables = tables
        self.d_block_tables.copy_(self.torch.from_numpy(tables))
        self._tables_dirty = False

    def _aux_handles(self):
        """Handles of the second stream (default priority) and the two events
        that pkv_mixed_step uses to run a step's decode and draft kernels
        beside its chunk kernels.  Created once per engine.  The events only
        order the two streams on this GPU, so they are made without the
        system-scope fence a default event record pays (a cache writeback
        of the whole device between the append and the attention kernels)."""
        if self._aux is None:
            torch = self.torch
            with torch.cuda.device(self.device):
                s = torch.cuda.Stream(device=self.device)
                fork, join = B.StreamEvent(), B.StreamEvent()
            self._aux = (s, fork, join)
        s, fork, join = self._aux
        return s.cuda_stream, fork.handle.value, join.handle.value

    def _plan_arrays(self, entries):
        """The plan's slots and new-token counts as int32 arrays (reused while
        the plan is unchanged, as on a run of decode steps) and their total."""
        c = self._entries
        if c is None or not isinstance(entries, list) or c[0] != entries:
            slots = np.ascontiguousarray([e[0] for e in entries], dtype=np.int32)
            news = np.ascontiguousarray([e[1] for e in entries], dtype=np.int32)
            c = ([tuple(e) for e in entries], slots, news, int(news.sum()) if len(news) else 0,
                 slots.ctypes.data, news.ctypes.data)
            self._entries = c
        return c[1], c[2], c[3], c[4], c[5]

    def _lower_host(self, entries):
        """Lower the step into the next pinned staging buffer (host only)."""
        stream = self.torch.cuda.current_stream(self.device)
        nseg = len(entries)
        slots, news, t, slots_addr, news_addr = self._plan_arrays(entries)
        # packed metadata: slot_mapping | query_start | query_len | row_to_slot | context_lens
        #                  | copy-on-write room (up to one pair per entry)
        o1 = t
        o2 = o1 + nseg
        o3 = o2 + nseg
        o4 = o3 + nseg
        o5 = o4 + self.max_slots
        st = self._stage(o5 + 2 * nseg)
        h = st.np
        free_before = self.alloc.free_blocks()
        a = st.addr
        nc = self.alloc.lower_step_raw(nseg, slots_addr, news_addr, a, t, a + 4 * o1, a + 4 * o2,
                                       a + 4 * o3, a + 4 * o4, a + 4 * o5, a + 4 * (o5 + nseg), nseg)
        if self.alloc.free_blocks() != free_before:
            self._tables_dirty = True     # new blocks, copy-on-write blocks included
        # copy_src [nc] then copy_dst [nc]
        cs, cd = o5, o5 + nc
        if nc:
            h[cd:cd + nc] = h[o5 + nseg:o5 + nseg + nc].copy()
        if self._tables_dirty:
            self._refresh_tables()
        row_to_slot = h[o3:o4]
        context_lens = h[o4:o5]
        snapshot = dict(slot_mapping=h[:o1].copy(), query_start=h[o1:o2].copy(), query_len=h[o2:o3].copy(),
                        row_to_slot=row_to_slot.copy(), context_lens=context_lens.copy(),
                        copy_src=h[cs:cd].copy(), copy_dst=h[cd:cd + nc].copy())
        snapshot["block_tables"] = self.h_block_tables
        max_q = int(news.max()) if nseg else 0
        max_ctx = int(context_lens[row_to_slot].max()) if nseg else 0
        offs = (0, o1, o2, o3, o4, cs, cd, cd + nc)
        meta = StepMeta(host=snapshot, dev=st.dev, offs=offs, stream=B.ctypes.c_void_p(stream.cuda_stream),
                        total_q=t, max_query_len=max_q, max_context_len=max_ctx, num_copies=nc, copy_off=cs)
        return meta, st, offs[:6] + (cd + nc,), stream

    def lower(self, entries) -> StepMeta:
        """Lower the step and copy its metadata to the device (stream order)."""
        meta, st, offs, stream = self._lower_host(entries)
        st.dev[:offs[-1]].copy_(st.host[:offs[-1]], non_blocking=True)
        st.copied = st.own
        st.copied.record(stream)
        st.used = True
        return meta

    def prepare_fused(self, entries, k_new, v_new, q, scale, out=None, out_dtype=None):
        """Lower on the host and build the one-call step descriptor for
        pkv_mixed_step (run it with run_prepared; running it again replays the
        same append and attention)."""
        torch = self.torch
        meta, st, offs, stream = self._lower_host(entries)
        if out is None:
            out = torch.empty((meta.total_q, self.num_q_heads, self.pool.head_dim),
                              dtype=out_dtype or torch.float32, device=self.device)
        ws = self.workspace_for(meta)
        nseg = len(entries)
        aux = self._aux_handles() if self.use_aux_stream else (None, None, None)
        desc = B.StepDesc(st.host.data_ptr(), st.dev.data_ptr(), offs[-1], offs[0], offs[1], offs[2], offs[3], offs[4],
                          meta.total_q, nseg, self.max_slots, meta.total_q, self.num_q_heads, self.max_blocks_per_seq,
                          meta.max_query_len, meta.max_context_len, k_new.data_ptr(), v_new.data_ptr(),
                          q.data_ptr(), self.d_block_tables.data_ptr(), float(scale), out.data_ptr(),
                          B.pkv_dtype_of(out.dtype), ws.data_ptr() if ws is not None else None,
                          ws.numel() if ws is not None else 0, meta.copy_off, meta.num_copies, *aux)
        # the tensors are held so their memory outlives every replay
        return PreparedStep(desc=desc, staging=st, stream=stream, meta=meta, out=out,
                            keep=(k_new, v_new, q, ws))

    def run_prepared(self, prep):
        """One library call (pkv_mixed_step): the append kernel stages the
        metadata to the device and appends; attention follows."""
        B.mixed_step(prep.desc, self.pool, prep.meta.stream)
        # the step's kernels have read the host buffer once the group's event,
        # recorded after this step or a later one on the same stream, completes
        if self._group_event is None or self._group_stream != prep.stream:
            self._close_group()
            self._group_event = B.StreamEvent()     # no system fence: the step's kernels only read the buffer
            self._group_stream = prep.stream
        prep.staging.copied = self._group_event
        prep.staging.used = True
        self._group_n += 1
        if self._group_n >= self.STEP_GROUP:
            self._close_group()
        return prep.out

    def fused_step(self, entries, k_new, v_new, q, scale, out=None, out_dtype=None):
        """Lower on the host, then one library call (pkv_mixed_step)."""
        prep = self.prepare_fused(entries, k_new, v_new, q, scale, out=out, out_dtype=out_dtype)
        return self.run_prepared(prep), prep.meta

    def append(self, meta: StepMeta, k_new, v_new):
        """Copy-on-write block copies (if any), then the KV append."""
        if meta.num_copies:
            B.copy_blocks(meta.copy_src, meta.copy_dst, self.pool, stream=meta.stream)
        B.kv_append(meta.slot_mapping, k_new, v_new, self.pool, stream=meta.stream)

    def workspace_for(self, meta: StepMeta):
        key = (len(meta.host["row_to_slot"]), meta.total_q, meta.max_query_len, meta.max_context_len)
        if key != self._ws_key:
            self._ws_bytes = B.workspace_bytes(key[0], key[1], self.num_q_heads, key[2], key[3], self.pool)
            self._ws_key = key
        n = self._ws_bytes
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
        res = B.paged_attend(q, meta.row_to_slot, meta.query_start, meta.query_len, meta.context_lens,
                             self.d_block_tables, self.pool, scale, max_query_len=meta.max_query_len,
                             max_context_len=meta.max_context_len, out=out, workspace=self.workspace_for(meta),
                             stream=meta.stream)
        return res

    def step(self, entries, k_new, v_new, q, scale, out=None, out_dtype=None):
        meta = self.lower(entries)
        self.append(meta, k_new, v_new)
        return self.attend(meta, q, scale, out=out, out_dtype=out_dtype), meta
