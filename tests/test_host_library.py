"""CPU tests of libpagedkv.so: it loads without a GPU, exports every symbol
the header declares, and its C++ allocator / step lowering / validator agree
bit-exactly with the oracle's plain allocator (no device calls here)."""
import ctypes

import numpy as np
import pytest

import paged_kv_attention_slot_amd as pk
from oracle.block_pool import BlockPool, NoSpace as OracleNoSpace
from workloads import make_workload


def test_library_loads_and_exports_header_symbols():
    lib = pk.lib()
    names = pk.header_symbols()
    assert "pkv_kv_append" in names and "pkv_paged_attend" in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert pk.decode_partition_tokens() % 16 == 0


def test_status_strings():
    lib = pk.lib()
    for st in range(0, -7, -1):
        assert lib.pkv_status_str(st)
    assert lib.pkv_status_str(-3).decode() == "not enough free KV blocks"


def test_device_entry_points_reject_bad_arguments_without_gpu():
    """Argument errors are returned before anything touches a device."""
    lib = pk.lib()
    d = pk.binding.PoolDesc(0, 0, 10, 16, 2, 64, 1)            # NULL k/v
    assert lib.pkv_kv_append(None, None, None, 4, ctypes.byref(d), None) == pk.binding.PKV_ERR_INVALID_ARG
    d2 = pk.binding.PoolDesc(16, 16, 10, 8, 2, 64, 1)          # block size 8 not built
    assert lib.pkv_kv_append(None, None, None, 4, ctypes.byref(d2), None) == pk.binding.PKV_ERR_UNSUPPORTED
    d3 = pk.binding.PoolDesc(16, 16, 10, 16, 2, 96, 1)         # head_dim 96 not built
    assert lib.pkv_paged_attend(16, 1, 4, 16, 16, 16, 1, 16, 16, 1, 1, 1, 1, ctypes.byref(d3), 1.0, 16, 0,
                                None, 0, None) == pk.binding.PKV_ERR_UNSUPPORTED
    d4 = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, 1)
    # 3 query heads over 2 KV heads
    assert lib.pkv_paged_attend(16, 1, 3, 16, 16, 16, 1, 16, 16, 1, 1, 1, 1, ctypes.byref(d4), 1.0, 16, 0,
                                None, 0, None) == pk.binding.PKV_ERR_INVALID_ARG
    # 18 query heads over 2 KV heads: G = 9 > 8
    assert lib.pkv_paged_attend(16, 1, 18, 16, 16, 16, 1, 16, 16, 1, 1, 1, 1, ctypes.byref(d4), 1.0, 16, 0,
                                None, 0, None) == pk.binding.PKV_ERR_UNSUPPORTED
    # bf16 output from an fp32 pool
    d5 = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, 0)
    assert lib.pkv_paged_attend(16, 1, 4, 16, 16, 16, 1, 16, 16, 1, 1, 1, 1, ctypes.byref(d5), 1.0, 16, 1,
                                None, 0, None) == pk.binding.PKV_ERR_INVALID_ARG
    # the softmax scale must be finite and positive
    for bad in (0.0, -0.125, float("inf"), float("nan")):
        assert lib.pkv_paged_attend(16, 1, 4, 16, 16, 16, 1, 16, 16, 1, 1, 1, 1, ctypes.byref(d4), bad, 16, 0,
                                    None, 0, None) == pk.binding.PKV_ERR_INVALID_ARG
        step = pk.binding.StepDesc()
        meta = (ctypes.c_int32 * 8)()
        step.host_meta = ctypes.cast(meta, ctypes.c_void_p)
        step.dev_meta = 16
        step.meta_len = 8
        step.num_slots = 1
        step.scale = bad
        assert lib.pkv_mixed_step(ctypes.byref(step), ctypes.byref(d4), None) == pk.binding.PKV_ERR_INVALID_ARG
    # 8-bit pools: scales required; a long multi-row segment's key-range
    # partials need workspace
    d8 = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, pk.PKV_I8, 16)
    d8_noscale = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, pk.PKV_I8)
    assert lib.pkv_paged_attend(16, 4, 4, 16, 16, 16, 1, 16, 16, 1, 1000, 4, 5000, ctypes.byref(d8), 1.0, 16, 0,
                                None, 0, None) == pk.binding.PKV_ERR_WORKSPACE
    assert lib.pkv_paged_attend_workspace_bytes(1, 4, 4, 4, 5000, ctypes.byref(d8)) > 0
    assert lib.pkv_paged_attend(16, 1, 4, 16, 16, 16, 1, 16, 16, 1, 1, 1, 16, ctypes.byref(d8_noscale), 1.0, 16,
                                0, None, 0, None) == pk.binding.PKV_ERR_INVALID_ARG
    assert lib.pkv_kv_append(None, None, None, 4, ctypes.byref(d8_noscale), None) == pk.binding.PKV_ERR_INVALID_ARG
    # block copies: a negative count, or a NULL pool
    assert lib.pkv_copy_blocks(None, None, -1, ctypes.byref(d4), None) == pk.binding.PKV_ERR_INVALID_ARG
    assert lib.pkv_copy_blocks(None, None, 1, ctypes.byref(d), None) == pk.binding.PKV_ERR_INVALID_ARG
    assert lib.pkv_copy_blocks(None, None, 0, ctypes.byref(d4), None) == pk.binding.PKV_OK
    # copy-on-write pairs that do not fit in the staged metadata
    step = pk.binding.StepDesc()
    meta = (ctypes.c_int32 * 8)()
    step.host_meta = ctypes.cast(meta, ctypes.c_void_p)
    step.dev_meta = 16
    step.meta_len = 8
    step.num_slots = 1
    step.scale = 1.0
    step.copy_off, step.num_copies = 4, 3
    assert lib.pkv_mixed_step(ctypes.byref(step), ctypes.byref(d4), None) == pk.binding.PKV_ERR_INVALID_ARG
    # decode rows with a long context need workspace; none given
    assert lib.pkv_paged_attend(16, 1, 4, 16, 16, 16, 1, 16, 16, 1, 1000, 1, 5000, ctypes.byref(d4), 1.0, 16, 0,
                                None, 0, None) == pk.binding.PKV_ERR_WORKSPACE


def test_empty_calls_return_ok_without_touching_the_device():
    """An append of no tokens and an attention over no segments or no rows
    succeed before any launch, with NULL pointers for the empty arrays."""
    lib = pk.lib()
    d = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, 1)
    assert lib.pkv_kv_append(None, None, None, 0, ctypes.byref(d), None) == pk.binding.PKV_OK
    # no segments
    assert lib.pkv_paged_attend(None, 0, 4, None, None, None, 0, None, None, 1, 1, 0, 0, ctypes.byref(d), 0.125,
                                None, 0, None, 0, None) == pk.binding.PKV_OK
    # segments but no rows
    assert lib.pkv_paged_attend(None, 0, 4, None, None, None, 3, None, None, 1, 1, 0, 0, ctypes.byref(d), 0.125,
                                None, 0, None, 0, None) == pk.binding.PKV_OK
    assert lib.pkv_paged_attend_noalloc(None, 0, 4, None, None, None, 0, None, None, 1, 1, 0, 0, ctypes.byref(d),
                                        0.125, None, 0, None) == pk.binding.PKV_OK


def test_workspace_sizing():
    d = pk.binding.PoolDesc(16, 16, 10, 16, 8, 128, 1)
    lib = pk.lib()
    pt = pk.decode_partition_tokens()
    assert lib.pkv_paged_attend_workspace_bytes(64, 64, 32, 1, pt, ctypes.byref(d)) == 0
    n = lib.pkv_paged_attend_workspace_bytes(64, 64, 32, 1, 4 * pt, ctypes.byref(d))
    acc = 64 * 32 * 4 * 128 * 4
    assert n == ((acc + 255) // 256) * 256 + 64 * 32 * 4 * 2 * 4


def test_workspace_sizing_mixed_step_follows_rows_not_segments():
    """Config 2's bounds (9 segments, 520 packed rows, 32/8 heads, head_dim
    128, a 512-row chunk, contexts up to 4000): decode partials per segment
    and partition; chunk key-range partials per (M-row, range) of the packed
    rows, at most ceil(ceil(4000 / 64) / 16) = 4 ranges each; verify partials
    for at most 9 segments x 8 rows (32 pairs / G 4) of the packed rows."""
    d = pk.binding.PoolDesc(16, 16, 10, 16, 8, 128, 1)
    lib = pk.lib()
    n = lib.pkv_paged_attend_workspace_bytes(9, 520, 32, 512, 4000, ctypes.byref(d))
    parts = -(-4000 // pk.decode_partition_tokens())
    decode = 9 * 32 * parts * 128 * 4 + 9 * 32 * parts * 2 * 4
    chunk_slots = min(9 * 32 * 128, 520 * 4 * 4)
    chunk = 8 * chunk_slots * (128 + 4) * 4
    vrows = min(520, 9 * 8)
    verify = vrows * 32 * parts * 128 * 4 + vrows * 32 * parts * 2 * 4
    assert n == decode + chunk + verify          # every part is a multiple of 256 here
    # a decode-only step of the same size needs no chunk or verify partials
    assert lib.pkv_paged_attend_workspace_bytes(9, 9, 32, 1, 4000, ctypes.byref(d)) == decode


def test_mixed_step_rejects_understated_bounds_and_half_a_stream_pair():
    """pkv_mixed_step checks the host copy of the metadata against the host
    bounds, and a lent second stream without its events, before any launch."""
    lib = pk.lib()
    d4 = pk.binding.PoolDesc(16, 16, 10, 16, 2, 64, 1)
    # one 5-row segment for slot 0 with 40 tokens: query_start | query_len |
    # row_to_slot | context_lens
    meta = (ctypes.c_int32 * 8)(0, 5, 0, 40)

    def step(max_q, max_ctx):
        st = pk.binding.StepDesc()
        st.host_meta = ctypes.cast(meta, ctypes.c_void_p)
        st.dev_meta = 16
        st.meta_len = 8
        st.query_start_off, st.query_len_off, st.row_to_slot_off, st.context_lens_off = 0, 1, 2, 3
        st.num_segments, st.num_slots, st.total_q, st.num_q_heads = 1, 1, 5, 4
        st.max_blocks_per_seq, st.max_query_len, st.max_context_len = 4, max_q, max_ctx
        st.scale = 0.125
        return st
    for max_q, max_ctx in ((4, 40), (5, 39), (1, 1)):
        st = step(max_q, max_ctx)
        assert lib.pkv_mixed_step(ctypes.byref(st), ctypes.byref(d4), None) == pk.binding.PKV_ERR_INVALID_ARG
    st = step(5, 40)
    st.aux_stream = 16                    # a stream without its fork / join events
    assert lib.pkv_mixed_step(ctypes.byref(st), ctypes.byref(d4), None) == pk.binding.PKV_ERR_INVALID_ARG


def _lower_raw(al, entries, max_slots):
    """The engine's packed lowering (BlockAllocator.lower_step_raw into one
    int32 buffer at plain addresses: slot_mapping | query_start | query_len |
    row_to_slot | context_lens | copy_src room | copy_dst room), unpacked."""
    n = len(entries)
    slots = np.ascontiguousarray([e[0] for e in entries], dtype=np.int32)
    news = np.ascontiguousarray([e[1] for e in entries], dtype=np.int32)
    t = int(news.sum())
    o = np.cumsum([0, t, n, n, n, max_slots, n, n])
    buf = np.full(int(o[-1]) + 8, -7, dtype=np.int32)   # poisoned, with a tail that must stay untouched
    a = buf.ctypes.data
    nc = al.lower_step_raw(n, slots.ctypes.data, news.ctypes.data, a, t, *(a + 4 * int(x) for x in o[1:7]), n)
    assert (buf[int(o[-1]):] == -7).all()
    keys = ("slot_mapping", "query_start", "query_len", "row_to_slot", "context_lens")
    got = {k: buf[o[i]:o[i + 1]].copy() for i, k in enumerate(keys)}
    got["copy_src"] = buf[o[5]:o[5] + nc].copy()
    got["copy_dst"] = buf[o[6]:o[6] + nc].copy()
    return got


def _random_ops(seed, n_ops=300, adopt=False, raw=False):
    rng = np.random.default_rng(seed)
    nb, bs, slots, maxb = 64, 16, 8, 12
    order = rng.permutation(nb).astype(np.int32)
    ours = pk.BlockAllocator(nb, bs, slots, maxb, order)
    ref = BlockPool(nb, bs, slots, maxb, order)
    live = set()
    for _ in range(n_ops):
        kind = rng.integers(0, 5)
        if kind == 0 and len(live) < slots:
            s = int(rng.choice([x for x in range(slots) if x not in live]))
            ours.acquire(s)
            ref.acquire(s)
            donors = [x for x in sorted(live) if ref.lengths[x] > 0]
            live.add(s)
            if adopt and donors and rng.random() < 0.7:
                src = int(rng.choice(donors))
                n = int(rng.integers(0, ref.lengths[src] + 1))
                ours.adopt(s, src, n)
                ref.adopt(s, src, n)
        elif kind == 1 and live:
            s = int(rng.choice(sorted(live)))
            ours.release(s)
            ref.release(s)
            live.discard(s)
        elif kind == 2 and live:
            s = int(rng.choice(sorted(live)))
            L = ref.lengths[s]
            nl = int(rng.integers(0, L + 1))
            ours.truncate(s, nl)
            ref.truncate(s, nl)
        elif kind == 3 and live:
            s = int(rng.choice(sorted(live)))
            tot = int(rng.integers(0, maxb * bs + 1))
            try:
                ref.reserve(s, tot)
                ok = True
            except OracleNoSpace:
                ok = False
            if ok:
                ours.reserve(s, tot)
            else:
                with pytest.raises(pk.NoSpace):
                    ours.reserve(s, tot)
        elif kind == 4 and live:
            chosen = [int(x) for x in rng.permutation(sorted(live))[: rng.integers(1, len(live) + 1)]]
            entries = []
            for s in chosen:
                room = maxb * bs - ref.lengths[s]
                if room >= 1:
                    entries.append((s, int(rng.integers(1, min(room, 40) + 1))))
            if not entries:
                continue
            try:
                want = ref.lower_step(entries)
                ok = True
            except OracleNoSpace:
                ok = False
            lower = (lambda e: _lower_raw(ours, e, slots)) if raw else ours.lower_step
            if ok:
                got = lower(entries)
                for k in want:
                    if k in got or not raw:
                        assert np.array_equal(got[k], want[k]), k
            else:
                with pytest.raises(pk.NoSpace):
                    lower(entries)
        # full state comparison after every op
        assert ours.free_blocks() == ref.free_count()
        assert [ours.block_refs(b) for b in range(nb)] == ref.refs
        for s in range(slots):
            if s in live:
                assert ours.slot_table(s) == ref.tables[s]
                assert ours.slot_info(s)[0] == ref.lengths[s]
            else:
                assert ours.slot_info(s) is None


@pytest.mark.parametrize("seed", range(6))
def test_allocator_and_lowering_match_oracle(seed):
    _random_ops(seed)


@pytest.mark.parametrize("seed", range(6))
def test_adoption_and_copy_on_write_match_oracle(seed):
    """Shared prefixes: adopt, reference counts, and the copy-on-write pairs
    of each lowering (compared key by key with the oracle's)."""
    _random_ops(100 + seed, adopt=True)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("adopt", [False, True], ids=["plain", "shared_prefixes"])
def test_raw_address_lowering_matches_oracle(seed, adopt):
    """The engine's lowering path (plain addresses into one packed buffer)
    gives the oracle's arrays and copy-on-write pairs, and writes nothing
    past its arrays."""
    _random_ops(200 + seed, adopt=adopt, raw=True)


def test_adoption_errors_and_plain_lowering_refuses_copies():
    al = pk.BlockAllocator(16, 16, 4, 8)
    al.acquire(0)
    al.lower_step([(0, 20)])                         # 2 blocks, the second partial
    al.acquire(1)
    with pytest.raises(pk.PagedKVError):
        al.adopt(1, 0, 21)                           # more than the source holds
    with pytest.raises(pk.PagedKVError):
        al.adopt(1, 1, 0)                            # itself
    with pytest.raises(pk.PagedKVError):
        al.adopt(2, 0, 4)                            # slot 2 not acquired
    al.adopt(1, 0, 20)
    t0 = al.slot_table(0)
    assert al.slot_table(1) == t0 and [al.block_refs(b) for b in t0] == [2, 2]
    with pytest.raises(pk.PagedKVError):
        al.adopt(1, 0, 4)                            # slot 1 no longer empty
    # the C entry point without copy buffers refuses a step that needs a copy
    lib = pk.lib()
    slots, news = np.array([1], np.int32), np.array([1], np.int32)
    st = lib.pkv_lower_step(al._h, 1, slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            news.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, 0, None, None, None,
                            None, None)
    assert st == pk.binding.PKV_ERR_STATE
    assert al.slot_info(1) == (20, 2)                # nothing changed
    meta = al.lower_step([(1, 1)])
    assert meta["copy_src"].tolist() == [t0[1]] and al.slot_table(1)[0] == t0[0]
    assert al.slot_table(1)[1] == meta["copy_dst"][0] != t0[1]
    assert [al.block_refs(b) for b in t0] == [2, 1]
    al.release(0)
    assert al.block_refs(t0[0]) == 1 and al.block_refs(t0[1]) == 0
    al.release(1)
    assert al.free_blocks() == 16


def test_allocator_matches_oracle_on_config_workloads():
    for name in ["1", "2", "4b", "5"]:
        w = make_workload(name)
        ours = pk.BlockAllocator(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
        ref = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
        for slot, _, _ in w.history:
            ours.acquire(slot)
            ref.acquire(slot)
        ent = [(s, len(k)) for s, k, _ in w.history if len(k)]
        a, b = ours.lower_step(ent), ref.lower_step(ent)
        assert all(np.array_equal(a[k], b[k]) for k in b)
        for st in w.steps:
            for op in st.ops:
                getattr(ours, op[0])(*op[1:])
                {"acquire": ref.acquire, "release": ref.release, "truncate": ref.truncate}[op[0]](*op[1:])
            ent = [(s.slot, s.n) for s in st.segments]
            a, b = ours.lower_step(ent), ref.lower_step(ent)
            assert all(np.array_equal(a[k], b[k]) for k in b)
            ok, bad = pk.validate_step(a, int(a["query_len"].sum()), w.num_blocks, w.block_size,
                                       w.max_blocks_per_seq)
            assert ok, bad


def test_worked_example_through_cpp_allocator():
    order = [7, 2, 9, 4, 1, 8, 0, 3, 5, 6]
    al = pk.BlockAllocator(10, 16, 4, 8, order)
    al.acquire(0)
    al.reserve(0, 64)
    al.acquire(1)
    al.reserve(1, 32)
    assert al.slot_table(0) == [7, 2, 9, 4] and al.slot_table(1) == [1, 8]
    al.release(1)
    al.acquire(2)
    al.reserve(2, 32)
    assert al.slot_table(2) == [1, 8] and al.slot_table(0) == [7, 2, 9, 4]


def test_state_errors():
    al = pk.BlockAllocator(4, 16, 2, 4)
    with pytest.raises(pk.PagedKVError):
        al.release(0)                       # not acquired
    al.acquire(0)
    with pytest.raises(pk.PagedKVError):
        al.acquire(0)                       # twice
    with pytest.raises(pk.PagedKVError):
        al.lower_step([(0, 1), (0, 1)])     # same slot twice in one step
    with pytest.raises(pk.PagedKVError):
        al.lower_step([(1, 1)])             # slot 1 not acquired
    with pytest.raises(pk.PagedKVError):
        al.reserve(0, 5 * 16)               # beyond the table capacity
    with pytest.raises(pk.NoSpace):
        al.acquire(1) or al.lower_step([(0, 40), (1, 40)])   # 3 + 3 blocks > 4


def test_pool_rounding():
    assert pk.pool_blocks_for_tokens(98304, 16) == 6144
    assert pk.pool_blocks_for_tokens(24576, 16) == 1536
    assert pk.pool_blocks_for_tokens(1, 16) == 1
    assert pk.pool_blocks_for_tokens(-1, 16) == -1


def _meta():
    return dict(row_to_slot=np.array([2, 0], np.int32), query_start=np.array([0, 3], np.int32),
                query_len=np.array([3, 1], np.int32), context_lens=np.array([20, 0, 5, 0], np.int32),
                block_tables=np.array([[1, 2], [0, 0], [3, 0], [0, 0]], np.int32),
                slot_mapping=np.array([50, 51, 52, 36], np.int32))


def test_validator_accepts_good_and_names_each_rule():
    ok, _ = pk.validate_step(_meta(), 4, 4, 16, 2)
    assert ok
    cases = [
        ("row_to_slot", np.array([2, 2], np.int32), 1),          # slot twice
        ("row_to_slot", np.array([2, 9], np.int32), 1),          # slot out of range
        ("query_start", np.array([0, 2], np.int32), 1),          # overlapping rows
        ("query_len", np.array([3, 2], np.int32), 1),            # beyond total_q
        ("query_len", np.array([6, 1], np.int32), 0),            # query_len > L (L = 5)
        ("context_lens", np.array([40, 0, 5, 0], np.int32), 1),  # table capacity 2 blocks
        ("block_tables", np.array([[1, 7], [0, 0], [3, 0], [0, 0]], np.int32), 1),   # block not in pool
        ("slot_mapping", np.array([50, 51, 50, 36], np.int32), 2),   # duplicate
        ("slot_mapping", np.array([50, 51, 52, 64], np.int32), 3),   # outside the pool
    ]
    for key, val, bad_idx in cases:
        m = _meta()
        m[key] = val
        ok, bad = pk.validate_step(m, 4, 4, 16, 2)
        assert not ok and bad == bad_idx, (key, val, bad)


def test_noalloc_rejects_steps_beyond_its_scratch_without_gpu():
    """pkv_paged_attend_noalloc checks arguments, then whether the step's
    partials fit its fixed scratch, before any HIP call: 1000 decode rows
    over contexts up to 32768 need ~1 GiB of split-context partials."""
    lib = pk.lib()
    d = pk.binding.PoolDesc(16, 16, 10, 16, 8, 128, 1)
    need = lib.pkv_paged_attend_workspace_bytes(1000, 1000, 32, 1, 32768, ctypes.byref(d))
    assert need > pk.binding.NOALLOC_SCRATCH_BYTES
    assert lib.pkv_paged_attend_noalloc(16, 1000, 32, 16, 16, 16, 1000, 16, 16, 1000, 2048, 1, 32768,
                                        ctypes.byref(d), 0.088, 16, 0, None) == pk.binding.PKV_ERR_WORKSPACE
    # argument errors come first (a bad scale), as for pkv_paged_attend
    assert lib.pkv_paged_attend_noalloc(16, 1000, 32, 16, 16, 16, 1000, 16, 16, 1000, 2048, 1, 32768,
                                        ctypes.byref(d), -1.0, 16, 0, None) == pk.binding.PKV_ERR_INVALID_ARG


def test_step_meta_device_views_follow_offsets():
    """StepMeta's device arrays are views of the staged buffer at the offsets
    the lowering recorded (made on first use)."""
    import torch
    from paged_kv_attention_slot_amd.engine import StepMeta
    dev = torch.arange(40, dtype=torch.int32)
    offs = (0, 3, 5, 7, 9, 17, 19, 21)      # T = 3, B = 2, 8 slots, 2 copy pairs
    meta = StepMeta(host={}, dev=dev, offs=offs, stream=None, total_q=3, max_query_len=2, max_context_len=9,
                    num_copies=2, copy_off=17)
    names = ("slot_mapping", "query_start", "query_len", "row_to_slot", "context_lens", "copy_src", "copy_dst")
    for i, name in enumerate(names):
        view = getattr(meta, name)
        assert view.tolist() == list(range(offs[i], offs[i + 1])), name
        assert view.data_ptr() == dev.data_ptr() + 4 * offs[i]
        assert getattr(meta, name) is view          # made once
    with pytest.raises(AttributeError):
        meta.not_a_field
