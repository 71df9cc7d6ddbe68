"""Run a whole workload through the oracle (test infrastructure).

The step order follows "Continuous batching: Qwen3.8-27B at 301 tok/s ..."
(lucebox blog) §Chunked prefill is a slot phase: the step's tokens are
appended to each slot's paged KV, then every packed row attends over its
slot's history.  Copy-on-write block copies (mlxcel user guide "연속 배칭"
§Paged KV 캐시와 프리픽스 공유) run before the append.  Workloads with an
8-bit KV cache quantize on append and attend over the dequantized values
(oracle/quant.py).  The pool starts filled with NaN so that any read of an
unwritten position shows up in the result.
"""
from __future__ import annotations

import numpy as np

from .block_pool import BlockPool
from .attention import append_reference, copy_blocks_reference, paged_attention
from .quant import append_reference_q8, paged_attention_q8

Q8_CODE_POISON = -128     # outside the code range [-127, 127]

NAN_BITS = {"f32": (np.uint32, 0x7FC00000, np.float32), "bf16": (np.uint16, 0x7FC0, np.uint16)}


def poisoned_pool(w):
    """One K or V pool; for 8-bit workloads a (codes, scales) pair with codes
    -128 (never a valid code) and NaN scales."""
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    if getattr(w, "kv_quant", "") == "q8":
        return (np.full(shape, Q8_CODE_POISON, dtype=np.int8),
                np.full(shape[:3], np.nan, dtype=np.float32))
    utype, bits, store = NAN_BITS[w.dtype]
    return np.full(shape, bits, dtype=utype).view(store)


def append_kv(w, pk, pv, slot_mapping, k_new, v_new):
    if getattr(w, "kv_quant", "") == "q8":
        ck, sk, cv, sv = append_reference_q8(pk[0], pk[1], pv[0], pv[1], slot_mapping, k_new, v_new,
                                             w.block_size)
        return (ck, sk), (cv, sv)
    return append_reference(pk, pv, slot_mapping, k_new, v_new, w.block_size)


def copy_kv(w, pk, pv, copy_src, copy_dst):
    if getattr(w, "kv_quant", "") == "q8":
        ck, cv = copy_blocks_reference(pk[0], pv[0], copy_src, copy_dst)
        sk, sv = copy_blocks_reference(pk[1], pv[1], copy_src, copy_dst)
        return (ck, sk), (cv, sv)
    return copy_blocks_reference(pk, pv, copy_src, copy_dst)


def attend_step(w, st, pk, pv, meta):
    args = (w.block_size, meta["block_tables"], meta["context_lens"], meta["row_to_slot"],
            meta["query_start"], meta["query_len"], w.scale)
    if getattr(w, "kv_quant", "") == "q8":
        return paged_attention_q8(st.q, pk, pv, *args)
    return paged_attention(st.q, pk, pv, w.dtype, *args)


def apply_ops(pool: BlockPool, ops):
    for op in ops:
        if op[0] == "acquire":
            pool.acquire(op[1])
        elif op[0] == "release":
            pool.release(op[1])
        elif op[0] == "truncate":
            pool.truncate(op[1], op[2])
        elif op[0] == "adopt":
            pool.adopt(op[1], op[2], op[3])
        else:
            raise ValueError(op)


def place_history(w, alloc: BlockPool, pk, pv):
    """Acquire every history slot and append its prior tokens (not attended)."""
    for slot, _, _ in w.history:
        alloc.acquire(slot)
    entries = [(slot, len(k)) for slot, k, _ in w.history if len(k) > 0]
    if entries:
        meta = alloc.lower_step(entries)
        hk = np.concatenate([k for _, k, _ in w.history if len(k) > 0])
        hv = np.concatenate([v for _, _, v in w.history if len(v) > 0])
        pk, pv = append_kv(w, pk, pv, meta["slot_mapping"], hk, hv)
    return pk, pv


def run_workload(w, steps=None):
    """Returns a list with, per step: dict(meta=..., out=fp64 [T][Hq][D])."""
    alloc = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
    pk, pv = poisoned_pool(w), poisoned_pool(w)
    pk, pv = place_history(w, alloc, pk, pv)
    results = []
    for i, st in enumerate(w.steps):
        if steps is not None and i not in steps:
            break
        apply_ops(alloc, st.ops)
        meta = alloc.lower_step([(s.slot, s.n) for s in st.segments])
        pk, pv = copy_kv(w, pk, pv, meta["copy_src"], meta["copy_dst"])
        pk, pv = append_kv(w, pk, pv, meta["slot_mapping"], st.k_new, st.v_new)
        out = attend_step(w, st, pk, pv, meta)
        results.append(dict(meta=meta, out=out))
    return results, (pk, pv)
