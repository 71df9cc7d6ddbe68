"""Pins for the CPU oracle: checks against things other than the oracle itself.

* brute force: a scalar loop with math.exp over hand-placed tiny pools;
* a library routine: torch CPU scaled_dot_product_attention in fp64 with its
  own lower-right causal mask and its own GQA grouping;
* closed forms (one key, constant V, q = 0, a dominant key, GQA twins);
* invariants from the pages (physical placement, chunking, slot reuse);
* the pages' worked block-table example (tests/golden/).
A last group plants plausible mistakes in the oracle and checks that the pins
above catch each one.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import attention as pa
from oracle.block_pool import BlockPool, NoSpace, pool_blocks_for_tokens
from oracle.step import run_workload
from workloads import bf16_bits_from_f32, make_custom, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- helpers
def logical_kv(w):
    """Per slot: the logical [L][Hkv][D] K and V after step 0 (history + new)."""
    out = {}
    st = w.steps[0]
    row = 0
    news = {}
    for seg in st.segments:
        news[seg.slot] = (st.k_new[row:row + seg.n], st.v_new[row:row + seg.n])
        row += seg.n
    for slot, hk, hv in w.history:
        nk, nv = news.get(slot, (hk[:0], hv[:0]))
        out[slot] = (np.concatenate([hk, nk]), np.concatenate([hv, nv]))
    return out


def sdpa_reference(w):
    """torch CPU fp64 SDPA over each sequence's logical K/V (no paging)."""
    kv = logical_kv(w)
    st = w.steps[0]
    q = pa.decode_values(st.q, w.dtype)
    out = np.empty_like(q)
    row = 0
    for seg in st.segments:
        k, v = kv[seg.slot]
        L = len(k)
        qt = torch.from_numpy(q[row:row + seg.n]).permute(1, 0, 2)[None]              # [1][Hq][n][D]
        kt = torch.from_numpy(pa.decode_values(k, w.dtype)).permute(1, 0, 2)[None]     # [1][Hkv][L][D]
        vt = torch.from_numpy(pa.decode_values(v, w.dtype)).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal_lower_right(seg.n, L),
                                           scale=w.scale, enable_gqa=True)
        out[row:row + seg.n] = o[0].permute(1, 0, 2).numpy()
        row += seg.n
    return out


def brute_force(q, k, v, scale, n_rows, L):
    """Scalar loops: row i of n sits at position L-n+i; head h reads KV head
    h*Hkv//Hq... written as the group index of h among Hq/Hkv equal groups."""
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    per = hq // hkv
    out = np.zeros((n_rows, hq, d))
    for i in range(n_rows):
        last = L - n_rows + i
        for h in range(hq):
            g = 0
            while (g + 1) * per <= h:
                g += 1
            scores = []
            for j in range(last + 1):
                acc = 0.0
                for e in range(d):
                    acc += float(q[i, h, e]) * float(k[j, g, e])
                scores.append(acc * scale)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            for e in range(d):
                out[i, h, e] = sum(ws[j] * float(v[j, g, e]) for j in range(last + 1)) / tot
    return out


def run_step0(w):
    res, pools = run_workload(w, steps={0})
    return res[0], pools


# --------------------------------------------------------------- decoding
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x4049, 0x0000, 0x8000], dtype=np.uint16)
    vals = pa.decode_values(bits, "bf16")
    assert list(vals) == [1.0, -2.0, 0.25, 3.140625, 0.0, -0.0]


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7 -> even mantissa (1.0).
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6).
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    got = pa.decode_values(bf16_bits_from_f32(x), "bf16")
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7]


# --------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    """Two sequences in a 6-block pool (block size 2) placed by hand at
    shuffled blocks; one decode row and one 3-row causal segment."""
    rng = np.random.default_rng(seed)
    bs, hq, hkv, d = 2, 2, 1, 4
    lens = {0: 5, 1: 4}
    nrows = {0: 1, 1: 3}
    pool_k = np.full((6, hkv, bs, d), np.nan, dtype=np.float32)
    pool_v = np.full((6, hkv, bs, d), np.nan, dtype=np.float32)
    tables = np.zeros((2, 3), dtype=np.int32)
    phys = rng.permutation(6)
    logical = {}
    used = 0
    for s in (0, 1):
        L = lens[s]
        k = rng.standard_normal((L, hkv, d)).astype(np.float32)
        v = rng.standard_normal((L, hkv, d)).astype(np.float32)
        logical[s] = (k, v)
        for j in range(-(-L // bs)):
            tables[s, j] = phys[used]
            used += 1
        for p in range(L):
            pool_k[tables[s, p // bs], :, p % bs, :] = k[p]
            pool_v[tables[s, p // bs], :, p % bs, :] = v[p]
    q = rng.standard_normal((4, hq, d)).astype(np.float32)
    scale = 0.37
    out = pa.paged_attention(q, pool_k, pool_v, "f32", bs, tables, np.array([5, 4]),
                             np.array([0, 1]), np.array([0, 1]), np.array([1, 3]), scale)
    ref0 = brute_force(q[0:1], *logical[0], scale, 1, 5)
    ref1 = brute_force(q[1:4], *logical[1], scale, 3, 4)
    np.testing.assert_allclose(out[0:1], ref0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[1:4], ref1, rtol=0, atol=1e-12)


# --------------------------------------------------------------- library routine
MIXED = [(3, 40, 1), (0, 16, 1), (5, 0, 37), (1, 33, 20), (2, 15, 1), (4, 63, 2)]


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 8, 2, 64), ("bf16", 6, 2, 32), ("bf16", 5, 1, 16),
                                            ("f32", 4, 4, 8)])
def test_paged_equals_contiguous_sdpa(dtype, hq, hkv, d):
    w = make_custom(MIXED, dtype=dtype, hq=hq, hkv=hkv, d=d, seed=11)
    r, _ = run_step0(w)
    np.testing.assert_allclose(r["out"], sdpa_reference(w), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["1", "1+1", "2"])
def test_configs_equal_contiguous_sdpa(name):
    w = make_workload(name)
    r, _ = run_step0(w)
    np.testing.assert_allclose(r["out"], sdpa_reference(w), rtol=0, atol=1e-12)


# --------------------------------------------------------------- closed forms
def _single(seq_len, n, q, k, v, scale=0.5, bs=4):
    """Place one sequence contiguously (identity table) and attend."""
    hkv, d = k.shape[1], k.shape[2]
    nb = -(-seq_len // bs)
    pk = np.full((nb + 1, hkv, bs, d), np.nan)
    pv = np.full((nb + 1, hkv, bs, d), np.nan)
    for p in range(seq_len):
        pk[p // bs, :, p % bs] = k[p]
        pv[p // bs, :, p % bs] = v[p]
    table = np.arange(nb + 1, dtype=np.int32)[None]
    return pa.paged_attention(q.astype(np.float32), pk.astype(np.float32), pv.astype(np.float32), "f32", bs,
                              table, np.array([seq_len]), np.array([0]), np.array([0]), np.array([n]), scale)


def test_closed_form_single_key_is_v0():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 2, 8)).astype(np.float32)
    v = rng.standard_normal((1, 2, 8)).astype(np.float32)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out = _single(1, 1, q, k, v)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2].astype(np.float64))


def test_closed_form_constant_v_and_zero_q():
    rng = np.random.default_rng(4)
    L = 23
    k = rng.standard_normal((L, 1, 8)).astype(np.float32)
    c = rng.standard_normal(8).astype(np.float32)
    v_const = np.broadcast_to(c, (L, 1, 8)).copy()
    q = rng.standard_normal((3, 2, 8)).astype(np.float32)
    out = _single(L, 3, q, k, v_const)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), rtol=0, atol=1e-14)
    # q = 0: every visible key weighs the same, so the output is the mean of visible V.
    v = rng.standard_normal((L, 1, 8)).astype(np.float32)
    out0 = _single(L, 3, np.zeros((3, 2, 8), np.float32), k, v)
    for i in range(3):
        vis = L - 3 + i + 1
        np.testing.assert_allclose(out0[i, 0], v[:vis, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_closed_form_dominant_key():
    rng = np.random.default_rng(5)
    L = 30
    k = (0.01 * rng.standard_normal((L, 1, 8))).astype(np.float32)
    v = rng.standard_normal((L, 1, 8)).astype(np.float32)
    q = np.zeros((1, 1, 8), np.float32)
    q[0, 0, 0] = 10.0
    k[17, 0, 0] = 40.0            # score 400 * scale above the others
    out = _single(L, 1, q, k, v, scale=1.0)
    np.testing.assert_allclose(out[0, 0], v[17, 0], rtol=0, atol=1e-12)


def test_closed_form_gqa_twins_identical():
    w = make_custom([(0, 50, 1), (1, 20, 5)], dtype="bf16", hq=8, hkv=2, d=16, seed=9)
    st = w.steps[0]
    st.q[:, 1] = st.q[:, 0]          # heads 0 and 1 share KV head 0
    st.q[:, 5] = st.q[:, 4]          # heads 4 and 5 share KV head 1
    r, _ = run_step0(w)
    assert np.array_equal(r["out"][:, 1], r["out"][:, 0])
    assert np.array_equal(r["out"][:, 5], r["out"][:, 4])


# --------------------------------------------------------------- invariants
def test_block_permutation_invariance_bitwise():
    w1 = make_custom(MIXED, dtype="bf16", hq=4, hkv=2, d=32, seed=21)
    w2 = make_custom(MIXED, dtype="bf16", hq=4, hkv=2, d=32, seed=21)
    w2.free_order = np.random.default_rng(99).permutation(w2.num_blocks).astype(np.int32)
    r1, _ = run_step0(w1)
    r2, _ = run_step0(w2)
    assert not np.array_equal(r1["meta"]["block_tables"], r2["meta"]["block_tables"])
    assert np.array_equal(r1["out"], r2["out"])


def _prompt_in_chunks(chunks, total, seed=31, bs=16, hq=4, hkv=2, d=16):
    """One prompt of `total` tokens attended in the given chunk sizes; returns
    the concatenated rows."""
    rng = np.random.default_rng(seed)
    k = bf16_bits_from_f32(rng.standard_normal((total, hkv, d), dtype=np.float32))
    v = bf16_bits_from_f32(rng.standard_normal((total, hkv, d), dtype=np.float32))
    q = bf16_bits_from_f32(rng.standard_normal((total, hq, d), dtype=np.float32))
    nb = -(-total // bs) + 3
    alloc = BlockPool(nb, bs, 1, nb, rng.permutation(nb))
    pk = np.full((nb, hkv, bs, d), 0x7FC0, np.uint16)
    pv = pk.copy()
    alloc.acquire(0)
    outs, pos = [], 0
    for c in chunks:
        meta = alloc.lower_step([(0, c)])
        pk, pv = pa.append_reference(pk, pv, meta["slot_mapping"], k[pos:pos + c], v[pos:pos + c], bs)
        outs.append(pa.paged_attention(q[pos:pos + c], pk, pv, "bf16", bs, meta["block_tables"],
                                       meta["context_lens"], meta["row_to_slot"], meta["query_start"],
                                       meta["query_len"], 0.25))
        pos += c
    return np.concatenate(outs)


def test_chunking_invariance():
    """One 96-row prompt segment equals the same prompt in three 32-row steps
    (lucebox blog §Chunked prefill: C[0:512], C[512:1024], ...), and a row
    split as 95 rows + one decode row."""
    whole = _prompt_in_chunks([96], 96)
    np.testing.assert_allclose(_prompt_in_chunks([32, 32, 32], 96), whole, rtol=0, atol=1e-13)
    np.testing.assert_allclose(_prompt_in_chunks([50, 45, 1], 96), whole, rtol=0, atol=1e-13)


def test_segment_order_and_slot_relabel_invariance():
    base = [(0, 40, 1), (3, 25, 7), (7, 10, 1)]
    w1 = make_custom(base, seed=41, d=16)
    r1, _ = run_step0(w1)
    # Same data, slots relabelled (0,3,7) -> (0,2,7) as in the lucebox blog's
    # compact-batch example; outputs are identical.
    w2 = make_custom(base, seed=41, d=16)
    w2.history = [(2 if s == 3 else s, k, v) for s, k, v in w2.history]
    for seg in w2.steps[0].segments:
        seg.slot = 2 if seg.slot == 3 else seg.slot
    r2, _ = run_step0(w2)
    assert np.array_equal(r1["out"], r2["out"])


def test_free_and_reuse_isolation():
    """Release one slot, reuse its blocks for a new prompt; the other slots'
    replayed rows and their pool bytes are unchanged (lucebox blog §Paged KV:
    blocks of a finished sequence go to a new request without moving others)."""
    from workloads.configs import Segment, Step
    w = make_custom([(0, 30, 4), (1, 50, 4), (2, 20, 4)], seed=51, d=16, pool_slack=1.0, num_blocks=40)
    s1 = w.steps[0]
    rng = np.random.default_rng(52)
    nk = bf16_bits_from_f32(rng.standard_normal((40, 2, 16), dtype=np.float32))
    nq = bf16_bits_from_f32(rng.standard_normal((40, 4, 16), dtype=np.float32))
    ops = [("release", 1), ("truncate", 0, 30), ("truncate", 2, 20), ("acquire", 1)]
    segs = [Segment(0, 4), Segment(1, 40), Segment(2, 4)]
    w.steps.append(Step(ops=ops, segments=segs,
                        k_new=np.concatenate([s1.k_new[0:4], nk, s1.k_new[8:12]]),
                        v_new=np.concatenate([s1.v_new[0:4], nk, s1.v_new[8:12]]),
                        q=np.concatenate([s1.q[0:4], nq, s1.q[8:12]])))
    res, _ = run_workload(w)
    a, b = res[0], res[1]
    assert np.array_equal(b["out"][0:4], a["out"][0:4])
    assert np.array_equal(b["out"][44:48], a["out"][8:12])
    old1 = set(a["meta"]["block_tables"][1][: -(-54 // 16)].tolist())
    new1 = b["meta"]["block_tables"][1][: -(-40 // 16)].tolist()
    assert set(new1) <= old1 | set(range(40))
    assert new1[0] == a["meta"]["block_tables"][1][0]         # LIFO: first freed block first


# --------------------------------------------------------------- append
def test_append_matches_token_loop_and_leaves_other_bytes():
    rng = np.random.default_rng(61)
    nb, hkv, bs, d = 9, 3, 16, 8
    pk = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint16)
    pv = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint16)
    sm = rng.choice(nb * bs, size=37, replace=False).astype(np.int32)
    kn = rng.integers(0, 2 ** 16, size=(37, hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, size=(37, hkv, d), dtype=np.uint16)
    k2, v2 = pa.append_reference(pk, pv, sm, kn, vn, bs)
    ek, ev = pk.copy(), pv.copy()
    touched = np.zeros((nb, bs), bool)
    for t in range(37):
        blk, off = int(sm[t]) // bs, int(sm[t]) % bs
        touched[blk, off] = True
        for h in range(hkv):
            for e in range(d):
                ek[blk, h, off, e] = kn[t, h, e]
                ev[blk, h, off, e] = vn[t, h, e]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert np.array_equal(k2.transpose(0, 2, 1, 3)[~touched], pk.transpose(0, 2, 1, 3)[~touched])
    k3, v3 = pa.append_reference(k2, v2, sm, kn, vn, bs)           # idempotent
    assert np.array_equal(k3, k2) and np.array_equal(v3, v2)


# --------------------------------------------------------------- block pool
def _golden_tables():
    rows = {}
    with open(os.path.join(GOLDEN, "worked_block_tables.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                rows[key] = [int(x) for x in vals]
    return rows


def test_worked_block_table_example():
    g = _golden_tables()
    order = g["A"] + g["B"] + g["free"]
    alloc = BlockPool(10, 16, 4, 8, order)
    alloc.acquire(0)
    alloc.reserve(0, 4 * 16)
    alloc.acquire(1)
    alloc.reserve(1, 2 * 16)
    assert alloc.tables[0] == g["A"] and alloc.tables[1] == g["B"]
    assert list(reversed(alloc.free)) == g["free"]
    alloc.release(1)
    alloc.acquire(2)
    alloc.reserve(2, 2 * 16)
    assert alloc.tables[2] == g["after_B_finishes_new_request"]
    assert alloc.tables[0] == g["A"]


def test_reserve_is_all_or_nothing():
    alloc = BlockPool(10, 16, 4, 16, np.arange(10))
    alloc.acquire(0)
    alloc.acquire(1)
    alloc.reserve(0, 100)                       # 7 blocks
    before = (list(alloc.free), {k: list(v) for k, v in alloc.tables.items()}, dict(alloc.lengths))
    with pytest.raises(NoSpace):
        alloc.reserve(1, 4 * 16)                # needs 4, 3 free
    with pytest.raises(NoSpace):
        alloc.lower_step([(0, 13), (1, 49)])    # 0 + 4 blocks > 3 free
    assert before == (list(alloc.free), {k: list(v) for k, v in alloc.tables.items()}, dict(alloc.lengths))


def test_slot_mapping_roundtrip_and_uniqueness():
    """Every appended token lands at a distinct pool position, and walking the
    block table gives the tokens back in logical order."""
    w = make_custom(MIXED, dtype="f32", hq=2, hkv=1, d=4, seed=71)
    r, (pk, _) = run_step0(w)
    kv = logical_kv(w)
    ctx, tables = r["meta"]["context_lens"], r["meta"]["block_tables"]
    for slot, (k, _) in kv.items():
        got = pa.gather_sequence(pk, tables[slot], int(ctx[slot]), w.block_size)
        assert np.array_equal(got, k)
    sm = r["meta"]["slot_mapping"]
    assert len(set(sm.tolist())) == len(sm)


def test_pool_rounding_to_whole_blocks():
    assert pool_blocks_for_tokens(98304, 16) == 6144
    assert pool_blocks_for_tokens(100, 16) == 7
    assert pool_blocks_for_tokens(0, 16) == 0


# --------------------------------------------------------------- planted mistakes
def _pins_fail(monkeypatch_target, name, bad):
    w = make_custom(MIXED, dtype="f32", hq=8, hkv=2, d=16, seed=81)
    orig = getattr(monkeypatch_target, name)
    setattr(monkeypatch_target, name, bad)
    try:
        r, _ = run_step0(w)
        out = r["out"]
    except (IndexError, ValueError):
        return True                      # the mistake cannot even run
    finally:
        setattr(monkeypatch_target, name, orig)
    ref = sdpa_reference(w)
    return not np.allclose(out, ref, rtol=0, atol=1e-12, equal_nan=False)


def test_planted_mistakes_are_caught():
    assert _pins_fail(pa, "kv_head_for", lambda h, g: h % 2)                     # wrong GQA map
    assert _pins_fail(pa, "visible", lambda pos, L: np.arange(L)[None] < pos[:, None])   # off by one
    assert _pins_fail(pa, "visible", lambda pos, L: np.ones((len(pos), L), bool))        # no causal mask
    assert _pins_fail(pa, "block_and_offset", lambda s, bs: (s % bs, s // bs))          # swapped
    orig_gather = pa.gather_sequence
    assert _pins_fail(pa, "gather_sequence",
                      lambda pool, t, L, bs: orig_gather(pool, np.roll(np.asarray(t), 1), L, bs))
    orig_attend = pa.attend_rows
    assert _pins_fail(pa, "attend_rows", lambda q, k, v, s, p: orig_attend(q, k, v, 1.0, p))  # scale dropped
    assert _pins_fail(pa, "attend_rows", lambda q, k, v, s, p: orig_attend(q, v, k, s, p))    # K/V swapped


# --------------------------------------------------------------- shared prefixes
def _assert_refcounts(pool: BlockPool):
    """Brute-force recount: a block's count is the number of tables holding it,
    and the free list is exactly the blocks no table holds, each once."""
    counts = [0] * pool.num_blocks
    for table in pool.tables.values():
        for b in table:
            counts[b] += 1
    assert counts == pool.refs
    assert sorted(pool.free) == [b for b in range(pool.num_blocks) if counts[b] == 0]


def _golden_saving():
    vals = {}
    with open(os.path.join(GOLDEN, "prefix_sharing_saving.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def test_prefix_sharing_saving_matches_worked_example():
    """The page's 8 requests over a 1024-token prefix: adopting stores the
    prefix blocks once; the blocks not stored, at the page's KV bytes per
    token, give its 784 MiB."""
    g = _golden_saving()
    n, p, bs = g["requests"], g["prefix_tokens"], 16
    used = {}
    for adopt in (False, True):
        pool = BlockPool(n * p // bs + 8, bs, n, p // bs + 1)
        for s in range(n):
            pool.acquire(s)
        if adopt:
            pool.lower_step([(0, p)])
            for s in range(1, n):
                pool.adopt(s, 0, p)
        else:
            pool.lower_step([(s, p) for s in range(n)])
        _assert_refcounts(pool)
        used[adopt] = pool.num_blocks - pool.free_count()
        # every request then decodes one token; a block-aligned prefix needs no copy
        meta = pool.lower_step([(s, 1) for s in range(n)])
        assert len(meta["copy_src"]) == 0
        _assert_refcounts(pool)
    saved_tokens = (used[False] - used[True]) * bs
    assert saved_tokens == (n - 1) * p
    assert saved_tokens * g["kib_per_token"] / 1024 == g["saved_mib"]


def test_prefix_adoption_decodes_like_cold_bitwise():
    """An adopting request's outputs equal a cold prefill's, bit for bit, over
    three steps (suffix chunks that diverge inside the shared partial block,
    decodes, and the donor's release); the prefix is stored once."""
    wa, wc = make_workload("prefix"), make_workload("prefix-cold")
    ra, _ = run_workload(wa)
    rc, _ = run_workload(wc)
    assert len(ra) == len(rc) == 3
    for a, c in zip(ra, rc):
        assert np.isfinite(a["out"]).all()
        assert np.array_equal(a["out"], c["out"])
    # slots 0..6 copy the shared partial block; slot 7, last to write, then
    # holds it alone and writes in place
    assert len(ra[0]["meta"]["copy_src"]) == 7 and len(rc[0]["meta"]["copy_src"]) == 0
    assert len(set(ra[0]["meta"]["copy_dst"].tolist())) == 7
    assert all(len(r["meta"]["copy_src"]) == 0 for r in ra[1:] + rc)


def test_shared_blocks_are_never_written():
    """Random slot lifecycles with adoption: after every lowering, no token
    of the step lands in a block that two tables hold, and the reference
    counts match a brute-force recount."""
    rng = np.random.default_rng(5)
    nb, bs, slots, maxb = 80, 16, 6, 10
    pool = BlockPool(nb, bs, slots, maxb, rng.permutation(nb))
    live = set()
    copies = 0
    both = [0]
    for _ in range(400):
        kind = int(rng.integers(0, 5))
        if kind == 0 and len(live) < slots:
            s = int(rng.choice([x for x in range(slots) if x not in live]))
            pool.acquire(s)
            donors = [x for x in live if pool.lengths[x] > 0]
            live.add(s)
            if donors and rng.random() < 0.8:
                src = int(rng.choice(donors))
                pool.adopt(s, src, int(rng.integers(0, pool.lengths[src] + 1)))
        elif kind == 1 and live:
            s = int(rng.choice(sorted(live)))
            pool.release(s)
            live.discard(s)
        elif kind == 2 and live:
            s = int(rng.choice(sorted(live)))
            pool.truncate(s, int(rng.integers(0, pool.lengths[s] + 1)))
        elif live:
            ent = [(s, int(rng.integers(1, 20))) for s in sorted(live)
                   if pool.lengths[s] + 20 <= maxb * bs and rng.random() < 0.7]
            if not ent:
                continue
            try:
                meta = pool.lower_step(ent)
            except NoSpace:
                continue
            copies += len(meta["copy_src"])
            written = set((meta["slot_mapping"] // bs).tolist())
            assert all(pool.refs[b] == 1 for b in written)
            # a copy source may still be written in this step by its last
            # holder (two writers shared it; the first copied it out), which
            # is why the copies run before the append
            both[0] += bool(written & set(meta["copy_src"].tolist()))
        _assert_refcounts(pool)
    assert copies > 10


def _prefix_pins_fail(patch):
    """Run the adopting workload with one planted mistake; True when the
    adopted outputs no longer equal the cold run's."""
    wa, wc = make_workload("prefix"), make_workload("prefix-cold")
    rc, _ = run_workload(wc)
    undo = patch()
    try:
        ra, _ = run_workload(wa)
    except (IndexError, ValueError, KeyError):
        return True
    finally:
        undo()
    return not all(np.array_equal(a["out"], c["out"]) for a, c in zip(ra, rc))


def test_planted_prefix_mistakes_are_caught():
    import oracle.step as ostep

    def swap(obj, name, bad):
        def apply():
            orig = getattr(obj, name)
            setattr(obj, name, bad)
            return lambda: setattr(obj, name, orig)
        return apply

    # the copy-on-write copy skipped: adopters read the fresh block's poison
    assert _prefix_pins_fail(swap(ostep, "copy_blocks_reference", lambda k, v, s, d: (k, v)))
    # no copy-on-write at all: adopters write into the shared block
    assert _prefix_pins_fail(swap(BlockPool, "_shared_write_index", lambda self, slot: None))
    # adoption sharing one block too few (floor instead of ceil)
    orig_adopt = BlockPool.adopt

    def short_adopt(self, slot, src, n):
        orig_adopt(self, slot, src, n)
        b = self.tables[slot].pop()
        self.refs[b] -= 1
    assert _prefix_pins_fail(swap(BlockPool, "adopt", short_adopt))


# --------------------------------------------------------------- 8-bit KV rows
from fractions import Fraction  # noqa: E402

from oracle import quant as pq  # noqa: E402


def _f32_nearest(r: Fraction) -> np.float32:
    """The float32 nearest the rational r (ties to even), by exact comparison
    of the neighbours of a first guess (no double rounding)."""
    c = np.float32(float(r))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    def key(f):
        return (abs(Fraction(float(f)) - r), int(np.array(f, np.float32).view(np.uint32)) & 1)
    return min(cands, key=key)


def _round_half_even(r: Fraction) -> int:
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def _q8_brute(x_bits):
    """The format's definition evaluated with exact rationals: every float32
    rounding done by nearest-neighbour search, the integer rounding by hand."""
    x = [Fraction(float(v)) for v in pa.decode_values(x_bits, "bf16")]
    amax = max(abs(v) for v in x)
    if amax == 0:
        return [0] * len(x), np.float32(0)
    inv = _f32_nearest(Fraction(127) / amax)
    scale = _f32_nearest(amax / 127)
    codes = []
    for v in x:
        prod = _f32_nearest(v * Fraction(float(inv)))
        codes.append(max(-127, min(127, _round_half_even(Fraction(float(prod))))))
    return codes, scale


def test_q8_hand_cases():
    """Hand-computed rows: ties go to the even code; a zero row is all zeros
    with scale 0; a row whose largest magnitude is 127 keeps its integers."""
    row = bf16_bits_from_f32(np.array([[254, 1, 3, 5, -3, -1, 0, 7]], np.float32))
    codes, scale = pq.quantize_rows(row)            # inv = 1/2, scale = 2
    assert codes.tolist() == [[127, 0, 2, 2, -2, 0, 0, 4]] and scale.tolist() == [2.0]
    codes, scale = pq.quantize_rows(np.zeros((1, 8), np.uint16))
    assert codes.tolist() == [[0] * 8] and scale.tolist() == [0.0]
    ints = np.array([[-127, -64, -1, 0, 1, 2, 100, 127]], np.float32)
    codes, scale = pq.quantize_rows(bf16_bits_from_f32(ints))
    assert codes.tolist() == ints.astype(int).tolist() and scale.tolist() == [1.0]


def test_q8_matches_exact_rational_brute_force():
    rng = np.random.default_rng(17)
    rows = bf16_bits_from_f32(rng.standard_normal((24, 64), dtype=np.float32) *
                              np.exp2(rng.integers(-6, 7, size=(24, 1))).astype(np.float32))
    codes, scales = pq.quantize_rows(rows)
    for i in range(rows.shape[0]):
        want_c, want_s = _q8_brute(rows[i])
        assert codes[i].tolist() == want_c, i
        assert scales[i].view(np.uint32) == np.float32(want_s).view(np.uint32), i


def test_q8_properties():
    """Codes within [-127, 127], the largest magnitude at +-127, signs kept,
    dequantization error within half a step, and scaling a row by a power of
    two scales its scale and keeps its codes."""
    rng = np.random.default_rng(19)
    x = rng.standard_normal((200, 128), dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    xf = pa.decode_values(bits, "bf16")
    codes, scales = pq.quantize_rows(bits)
    assert np.abs(codes.astype(int)).max() <= 127
    assert (np.abs(codes.astype(int)).max(axis=1) == 127).all()
    assert (codes.astype(float) * xf >= 0).all()
    err = np.abs(xf - pq.dequantize(codes, scales))
    assert (err <= scales[:, None].astype(np.float64) * (0.5 + 1e-4)).all()
    for k in (-5, 3):
        c2, s2 = pq.quantize_rows(bf16_bits_from_f32(pa.decode_values(bits, "bf16").astype(np.float32) * 2.0 ** k))
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, (scales * np.float32(2.0 ** k)).astype(np.float32))


def test_q8_append_and_attention():
    """The 8-bit append stores each token's codes and scale at its slot and
    touches nothing else; attention over the codes equals attention over a
    pool already holding their values, and stays within a few hundredths of
    the unquantized attention on N(0, 1) data."""
    w = make_custom([(0, 40, 1), (1, 70, 3), (2, 5, 1)], dtype="bf16", hq=8, hkv=2, d=64, seed=5)
    w.kv_quant = "q8"
    res, (pk, pv) = run_workload(w)
    out = res[0]["out"]
    meta = res[0]["meta"]
    # scatter: every written position holds the row's own quantization
    st = w.steps[0]
    ck, sk = pk
    for t, slot in enumerate(meta["slot_mapping"].tolist()):
        b, o = divmod(slot, w.block_size)
        c, s = pq.quantize_rows(st.k_new[t])
        assert np.array_equal(ck[b, :, o, :], c) and np.array_equal(sk[b, :, o], s)
    hist_rows = sum(len(k) for _, k, _ in w.history)
    assert np.isnan(sk).sum() == sk.size - (hist_rows + len(meta["slot_mapping"])) * w.num_kv_heads
    # attention over the dequantized pools through the plain path
    deq_k = pq.dequantize(pk[0], np.nan_to_num(pk[1]))
    deq_v = pq.dequantize(pv[0], np.nan_to_num(pv[1]))
    plain = pa.paged_attention(st.q, deq_k, deq_v, "bf16", w.block_size, meta["block_tables"],
                               meta["context_lens"], meta["row_to_slot"], meta["query_start"],
                               meta["query_len"], w.scale, kv_dtype="f64")
    assert np.array_equal(out, plain)
    w.kv_quant = ""
    ref, _ = run_workload(w)
    err = np.abs(out - ref[0]["out"]).max()
    assert 0 < err < 0.05, err


def test_planted_q8_mistakes_are_caught():
    row = bf16_bits_from_f32(np.array([[254, 1, 3, 5, -3, -1, 0, 7]], np.float32))
    orig_rint = np.rint
    try:
        pq.np.rint = lambda a: np.floor(a + 0.5)              # ties away from even
        assert pq.quantize_rows(row)[0].tolist() != [[127, 0, 2, 2, -2, 0, 0, 4]]
    finally:
        pq.np.rint = orig_rint
    orig_q = pq.quantize_rows

    def scale_128(bits):                                     # wrong divisor
        c, s = orig_q(bits)
        return c, (s * np.float32(127) / np.float32(128)).astype(np.float32)
    pq.quantize_rows = scale_128
    try:
        rng = np.random.default_rng(3)
        bits = bf16_bits_from_f32(rng.standard_normal((4, 64), dtype=np.float32))
        assert any(pq.quantize_rows(bits[i:i + 1])[1][0].view(np.uint32) !=
                   np.float32(_q8_brute(bits[i])[1]).view(np.uint32) for i in range(4))
    finally:
        pq.quantize_rows = orig_q
