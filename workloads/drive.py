"""Feed a Workload to a step engine on the GPU (harness glue, no arithmetic).

`engine` is any object with acquire/release/truncate/lower/append/attend/step
methods and a `pool` (see paged_kv_attention_slot_amd.engine.PagedKVEngine).
"""
from __future__ import annotations

import numpy as np


def to_device(raw: np.ndarray, dtype: str, device):
    """Raw workload values -> torch tensor on `device` with the same bits."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(raw, dtype=np.uint16).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def pool_torch_dtype(w):
    """The pool's element type: the workload dtype, or int8 codes for an
    8-bit KV workload (whose inputs stay bf16)."""
    import torch
    return torch.int8 if getattr(w, "kv_quant", "") == "q8" else torch_dtype(w.dtype)


def make_engine(engine_cls, w, device="cuda", free_order=None, poison=True):
    return engine_cls(num_blocks=w.num_blocks, num_kv_heads=w.num_kv_heads, num_q_heads=w.num_q_heads,
                      head_dim=w.head_dim, dtype=pool_torch_dtype(w), max_slots=w.max_slots,
                      max_blocks_per_seq=w.max_blocks_per_seq,
                      free_order=w.free_order if free_order is None else free_order, device=device, poison=poison)


def place_history(engine, w, device="cuda"):
    """Acquire every history slot and append its prior tokens (no attention)."""
    for slot, _, _ in w.history:
        engine.acquire(slot)
    entries = [(slot, len(k)) for slot, k, _ in w.history if len(k) > 0]
    if not entries:
        return
    meta = engine.lower(entries)
    hk = np.concatenate([k for _, k, _ in w.history if len(k) > 0])
    hv = np.concatenate([v for _, _, v in w.history if len(v) > 0])
    engine.append(meta, to_device(hk, w.dtype, device), to_device(hv, w.dtype, device))


def apply_ops(engine, ops):
    for op in ops:
        if op[0] == "acquire":
            engine.acquire(op[1])
        elif op[0] == "release":
            engine.release(op[1])
        elif op[0] == "truncate":
            engine.truncate(op[1], op[2])
        elif op[0] == "adopt":
            engine.adopt(op[1], op[2], op[3])
        else:
            raise ValueError(op)


def step_tensors(w, step_index, device="cuda"):
    st = w.steps[step_index]
    return (to_device(st.k_new, w.dtype, device), to_device(st.v_new, w.dtype, device),
            to_device(st.q, w.dtype, device))


def run_step(engine, w, step_index, device="cuda", out_dtype=None, fused=False):
    """Apply the step's slot ops, then lower + append + attend (separate
    calls, or the one-call fused step).  Returns (out tensor, StepMeta)."""
    st = w.steps[step_index]
    apply_ops(engine, st.ops)
    k, v, q = step_tensors(w, step_index, device)
    entries = [(s.slot, s.n) for s in st.segments]
    if fused:
        return engine.fused_step(entries, k, v, q, w.scale, out_dtype=out_dtype)
    return engine.step(entries, k, v, q, w.scale, out_dtype=out_dtype)
