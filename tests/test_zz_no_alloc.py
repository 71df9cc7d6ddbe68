"""pkv_paged_attend_noalloc (the entry point for callers that cannot
allocate) against pkv_paged_attend with a caller workspace: bit-identical
outputs on two calls in a row, the second with a smaller step, through the
C ABI.  The steps need every kind of partial the workspace holds: decode
rows past one split-context partition (reduce), short drafts whose rows span
partitions (verify merge), and prompt chunks cut into key ranges (merge)."""
import numpy as np
import pytest

import paged_kv_attention_slot_amd as pk
from workloads import make_custom
from workloads.drive import make_engine, place_history, step_tensors

pytestmark = pytest.mark.gpu

STEPS = [
    # slot, history, rows
    [(0, 3000, 1), (1, 700, 1), (2, 1500, 4), (3, 2000, 40), (4, 0, 512), (5, 5000, 1)],
    [(0, 900, 1), (1, 40, 3), (2, 1100, 24)],           # smaller: fewer rows, shorter contexts
]


def _one(seqs, seed):
    import torch
    w = make_custom(seqs, dtype="bf16", hq=32, hkv=8, d=128, seed=seed)
    eng = make_engine(pk.PagedKVEngine, w)
    place_history(eng, w)
    st = w.steps[0]
    k, v, q = step_tensors(w, 0)
    meta = eng.lower([(s.slot, s.n) for s in st.segments])
    eng.append(meta, k, v)
    want = eng.attend(meta, q, w.scale)                        # pkv_paged_attend + workspace
    got = torch.full_like(want, float("nan"))
    pk.paged_attend_noalloc(q, meta.row_to_slot, meta.query_start, meta.query_len, meta.context_lens,
                            eng.d_block_tables, eng.pool, w.scale, max_query_len=meta.max_query_len,
                            max_context_len=meta.max_context_len, out=got)
    torch.cuda.synchronize()
    need = pk.workspace_bytes(len(st.segments), meta.total_q, w.num_q_heads, meta.max_query_len,
                              meta.max_context_len, eng.pool)
    return want.cpu().numpy(), got.cpu().numpy(), need


def test_noalloc_equals_workspace_entry_point_on_two_calls(gpu_available):
    sizes = []
    for i, seqs in enumerate(STEPS):
        print(f"no-alloc call {i}: {seqs}", flush=True)
        want, got, need = _one(seqs, seed=50 + i)
        assert 0 < need <= pk.binding.NOALLOC_SCRATCH_BYTES
        assert np.array_equal(want.view(np.int32), got.view(np.int32)), f"call {i}"
        sizes.append(want.shape[0])
    assert sizes[1] < sizes[0]
