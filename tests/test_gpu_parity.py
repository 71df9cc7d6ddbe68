"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* kv_append: bit-exact over the whole pool (NaN-poisoned positions included);
* paged_attend: max-abs error <= 1e-4 (fp32 pool) / 1e-2 (bf16 pool, fp32
  accumulation, fp32 output) on every config, plus edge cases;
* bitwise invariants the design promises: batch composition, physical block
  placement, slot reuse.
"""
import functools
import os
import sys

import numpy as np
import pytest

import paged_kv_attention_slot_amd as pk
from oracle.step import run_workload
from workloads import make_custom, make_workload
from workloads.drive import make_engine, place_history, run_step, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def _workload(name):
    return make_workload(name)


@functools.lru_cache(maxsize=4)
def _oracle(name):
    res, pools = run_workload(_workload(name))
    return res, pools


def _pool_bits(t):
    import torch
    a = t.detach().cpu()
    return (a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)).numpy()


def _oracle_bits(a):
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


def _run_gpu(w, steps=None, out_dtype=None, free_order=None, fused=False):
    import torch
    eng = make_engine(pk.PagedKVEngine, w, free_order=free_order)
    place_history(eng, w)
    outs = []
    for i in range(len(w.steps)):
        if steps is not None and i not in steps:
            break
        out, meta = run_step(eng, w, i, out_dtype=out_dtype, fused=fused)
        torch.cuda.synchronize()
        outs.append((out, meta))
    return eng, outs


def _check_close(name, got, want, tol):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape
    assert np.isfinite(g).all(), f"{name}: non-finite output"
    err = np.abs(g - want)
    _log(f"{name}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= tol, f"{name}: max-abs {err.max()} > {tol}"


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
@pytest.mark.parametrize("name", ["1", "2", "4b", "5"])
def test_kv_append_bit_exact_whole_pool(name, fused, gpu_available):
    _log(f"append config {name} fused={fused}")
    w = _workload(name)
    eng, _ = _run_gpu(w, fused=fused)
    _, (ok, ov) = _oracle(name)
    assert np.array_equal(_pool_bits(eng.pool.k), _oracle_bits(ok))
    assert np.array_equal(_pool_bits(eng.pool.v), _oracle_bits(ov))


def test_kv_append_skips_out_of_pool_entries_and_empty(gpu_available):
    import torch
    w = make_custom([(0, 20, 1)], dtype="bf16", hq=4, hkv=2, d=64)
    eng = make_engine(pk.PagedKVEngine, w)
    before_k = _pool_bits(eng.pool.k).copy()
    sm = torch.tensor([-1, w.num_blocks * 16, 5], dtype=torch.int32, device="cuda")
    kn = torch.ones((3, 2, 64), dtype=torch.bfloat16, device="cuda")
    pk.kv_append(sm, kn, kn, eng.pool)
    pk.kv_append(sm[:0], kn[:0], kn[:0], eng.pool)
    torch.cuda.synchronize()
    after = _pool_bits(eng.pool.k)
    changed = np.argwhere(after != before_k)
    assert set(map(tuple, changed[:, :3].tolist())) == {(0, 0, 5), (0, 1, 5)}


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_empty_step_changes_nothing(fused, gpu_available):
    """A step with no segments (nothing appended, nothing attended) returns
    an empty output and leaves the pool bit for bit as it was."""
    import torch
    w = make_custom([(0, 20, 1), (1, 40, 1)], dtype="bf16", hq=4, hkv=2, d=64)
    eng = make_engine(pk.PagedKVEngine, w)
    place_history(eng, w)
    torch.cuda.synchronize()
    before_k, before_v = _pool_bits(eng.pool.k).copy(), _pool_bits(eng.pool.v).copy()
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    if fused:
        out, _ = eng.fused_step([], e, e, q, 0.125)
    else:
        meta = eng.lower([])
        eng.append(meta, e, e)
        out = eng.attend(meta, q, 0.125)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 4, 64)
    assert np.array_equal(_pool_bits(eng.pool.k), before_k)
    assert np.array_equal(_pool_bits(eng.pool.v), before_v)


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
@pytest.mark.parametrize("name", ["1", "1+1", "3", "3v", "2", "4a", "4b", "5"])
def test_attention_matches_oracle(name, fused, gpu_available):
    _log(f"attention config {name} fused={fused}")
    w = _workload(name)
    _, outs = _run_gpu(w, fused=fused)
    res, _ = _oracle(name)
    for i, ((out, _), r) in enumerate(zip(outs, res)):
        _check_close(f"config {name} step {i}", out, r["out"], TOL[w.dtype])


EDGE_SEQS = [
    [(0, 0, 1)],                                  # L = 1: output is V0
    [(0, 15, 1), (1, 16, 1), (2, 31, 1)],         # L = 16, 17, 32 block edges
    [(0, 511, 1), (1, 512, 1), (2, 1023, 1), (3, 1024, 1), (4, 2047, 1), (5, 2048, 1)],   # partition edges
    [(5, 3000, 1), (2, 7, 1)],                    # slots out of order
    [(0, 0, 5), (1, 40, 1), (2, 3, 2)],           # tiny prompt, decode, 2 drafts
    [(0, 700, 16), (1, 3000, 3), (2, 200, 40), (3, 1300, 1)],   # key-range splits of short segments
    [(0, 2500, 2), (1, 510, 3), (2, 40, 4), (3, 1021, 4)],     # short drafts whose rows straddle partitions
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 8, 8), (128, 40, 8), (64, 8, 1),
                                      (128, 24, 8), (64, 12, 2), (128, 14, 2)])   # G 4, 1, 5, 8, 3, 6, 7
@pytest.mark.parametrize("case", range(len(EDGE_SEQS)))
def test_edge_cases(dtype, d, hq, hkv, case, gpu_available):
    seqs = EDGE_SEQS[case]
    _log(f"edge case {case} {dtype} D{d} {hq}/{hkv}")
    w = make_custom(seqs, dtype=dtype, hq=hq, hkv=hkv, d=d, seed=100 + case)
    _, outs = _run_gpu(w)
    res, _ = run_workload(w)
    _check_close(f"edge {case}", outs[0][0], res[0]["out"], TOL[dtype])


def _rising_scores(w, seed, top=24.0, spike=12.0, spikes=3):
    """Rewrite Q and K of a one-step bf16 workload so that each sequence's
    scores (log2 units: q.k * scale * log2 e) climb about `top` from its first
    key to its last, with `spikes` isolated keys `spike` above the climb.  The
    running max then moves past any rescale slack in tiles well after the
    first, and some of those moves happen inside one tile."""
    from workloads.configs import bf16_bits_from_f32
    rng = np.random.default_rng(seed)
    d, hkv, hq = w.head_dim, w.num_kv_heads, w.num_q_heads
    to_qk = 1.0 / (w.scale * np.log2(np.e))            # log2 units -> q.k units
    u = rng.standard_normal((hkv, d)).astype(np.float32)
    unit = u / (u * u).sum(-1, keepdims=True)            # q . (b unit) = b for q = u
    step = w.steps[0]
    k_new = np.zeros(step.k_new.shape, np.float32)
    q = np.zeros(step.q.shape, np.float32)
    hist = {slot: kh for slot, kh, _ in w.history}
    new_k_hist = {}
    off = 0
    for seg in step.segments:
        h = hist[seg.slot].shape[0]
        L = h + seg.n
        b = top * np.arange(L) / max(L - 1, 1)
        b[rng.choice(L, size=min(spikes, L), replace=False)] += spike
        keys = (b * to_qk)[:, None, None] * unit[None] + 0.1 * rng.standard_normal((L, hkv, d))
        new_k_hist[seg.slot] = keys[:h]
        k_new[off:off + seg.n] = keys[h:]
        q[off:off + seg.n] = u[np.arange(hq) // (hq // hkv)][None] + 0.1 * rng.standard_normal((seg.n, hq, d))
        off += seg.n
    conv = bf16_bits_from_f32 if w.dtype == "bf16" else (lambda x: x.astype(np.float32))
    w.history = [(slot, conv(new_k_hist[slot].astype(np.float32)), vh) for slot, _, vh in w.history]
    step.k_new = conv(k_new)
    step.q = conv(q)
    return w


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (64, 8, 8), (128, 40, 8), (128, 8, 1)])
@pytest.mark.parametrize("seed", [0, 1])
def test_rising_scores_move_the_running_max(d, hq, hkv, seed, gpu_available):
    """Scores that climb along the sequence, with isolated spikes: every
    kernel's lazy rescale (and any vote that triggers it) fires repeatedly
    after the first tile, for a prompt chunk, short drafts and decode rows."""
    seqs = [(0, 900, 300), (1, 2000, 40), (2, 60, 5), (3, 3000, 1), (4, 0, 200)]
    _log(f"rising scores D{d} {hq}/{hkv} seed {seed}")
    w = _rising_scores(make_custom(seqs, dtype="bf16", hq=hq, hkv=hkv, d=d, seed=300 + seed), seed)
    _, outs = _run_gpu(w)
    res, _ = run_workload(w)
    _check_close("rising", outs[0][0], res[0]["out"], TOL["bf16"])


def test_single_token_context_is_v0(gpu_available):
    """One visible key: the output is that key's V, bit for bit (one weight,
    normalised by the same bf16-rounded weight the product consumed)."""
    w = make_custom([(0, 0, 1)], dtype="bf16", hq=8, hkv=2, d=128, seed=5)
    _, outs = _run_gpu(w)
    out = outs[0][0].cpu().numpy()
    v = w.steps[0].v_new.astype(np.uint32) << 16
    v = v.view(np.float32)
    for h in range(8):
        assert np.array_equal(out[0, h], v[0, h // 4])


@pytest.mark.parametrize("name", ["3", "3v", "2", "4a", "4b", "5", "3q", "5q"])
def test_bf16_output(name, gpu_available):
    """bf16 output on every store path - decode rows (direct and through the
    partition reduce), chunks (direct and through the key-range merge), short
    drafts (verify direct and merge), 8-bit pools - is the fp32 result
    rounded to nearest even, bit for bit, and within 1e-2 + half a bf16 ulp
    of the oracle (the bound for a bf16-rounded result)."""
    import torch
    _log(f"bf16 output config {name}")
    w = _workload(name)
    _, o32 = _run_gpu(w)
    _, o16 = _run_gpu(w, out_dtype=torch.bfloat16)
    res, _ = _oracle(name)
    for i, ((a, _), (b, _), r) in enumerate(zip(o32, o16, res)):
        assert b.dtype == torch.bfloat16
        assert torch.equal(b.cpu(), a.cpu().to(torch.bfloat16)), f"step {i}"
        got = b.float().cpu().numpy().astype(np.float64)
        want = r["out"]
        half_ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 9)
        err = np.abs(got - want)
        err32 = np.abs(a.float().cpu().numpy().astype(np.float64) - want)
        _log(f"config {name} step {i}: fp32 max-abs {err32.max():.3e} mean-abs {err32.mean():.3e}; "
             f"bf16 max-abs {err.max():.3e}")
        assert (err <= 1e-2 + half_ulp).all(), f"step {i}: max-abs {err.max()}"


def _scale_qk(w, factor):
    """Multiply every Q and K value of a one-step workload by a power of two
    (exact in bf16): scores grow by factor^2."""
    from workloads.configs import bf16_bits_from_f32

    def mul(a):
        x = (a.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
        return bf16_bits_from_f32(x)
    w.history = [(slot, mul(kh), vh) for slot, kh, vh in w.history]
    st = w.steps[0]
    st.k_new, st.q = mul(st.k_new), mul(st.q)
    return w


LARGE_LOGIT_SEQS = [(0, 3000, 1), (1, 700, 1), (2, 1200, 4), (3, 900, 16), (4, 1024, 512), (5, 40, 100)]


@pytest.mark.parametrize("kind", ["bf16", "q8"])
@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 32, 8), (128, 40, 8)])
def test_large_logits(kind, d, hq, hkv, gpu_available):
    """Q and K drawn N(0, 4^2): scores 16x larger than N(0,1) data, a sharply
    peaked softmax where any rounding of q or of the scaled score shows up.
    Decode rows, short drafts (verify kernel), 16-row drafts and chunks
    (chunk kernel, split and unsplit) stay within the 1e-2 bound."""
    _log(f"large logits {kind} D{d} {hq}/{hkv}")
    w = _scale_qk(make_custom(LARGE_LOGIT_SEQS, dtype="bf16", hq=hq, hkv=hkv, d=d, seed=400 + d + hq), 4.0)
    if kind == "q8":
        w.kv_quant = "q8"
    _, outs = _run_gpu(w)
    res, _ = run_workload(w)
    _check_close(f"large logits {kind}", outs[0][0], res[0]["out"], TOL["bf16"])


# ------------------------------------------------------------------ invariants
def test_decode_batch_composition_invariance_bitwise(gpu_available):
    """A row's output does not depend on which other rows share the step."""
    import torch
    base = [(3, 700, 1), (0, 5000, 1), (7, 100, 1), (2, 2047, 1), (9, 1, 1)]
    w1 = make_custom(base, dtype="bf16", hq=32, hkv=8, d=128, seed=61)
    _, o1 = _run_gpu(w1)
    w2 = make_custom(base, dtype="bf16", hq=32, hkv=8, d=128, seed=61)
    # same data, step holds only rows 1 and 3 in reverse order
    keep = [3, 1]
    st = w2.steps[0]
    st.segments = [st.segments[i] for i in keep]
    st.q, st.k_new, st.v_new = st.q[keep], st.k_new[keep], st.v_new[keep]
    _, o2 = _run_gpu(w2)
    a, b = o1[0][0].cpu(), o2[0][0].cpu()
    assert torch.equal(a[3], b[0]) and torch.equal(a[1], b[1])


def test_chunk_batch_composition_invariance_bitwise(gpu_available):
    """Multi-row segments (split and unsplit) give the same bits whatever
    else shares the step."""
    import torch
    base = [(0, 900, 16), (1, 50, 1), (2, 100, 300), (3, 2000, 1)]
    w1 = make_custom(base, dtype="bf16", hq=32, hkv=8, d=128, seed=81)
    _, o1 = _run_gpu(w1)
    w2 = make_custom(base, dtype="bf16", hq=32, hkv=8, d=128, seed=81)
    st = w2.steps[0]
    keep = [2, 0]
    rows = {0: slice(0, 16), 2: slice(17, 317)}
    st.segments = [st.segments[i] for i in keep]
    st.q = np.concatenate([st.q[rows[i]] for i in keep])
    st.k_new = np.concatenate([st.k_new[rows[i]] for i in keep])
    st.v_new = np.concatenate([st.v_new[rows[i]] for i in keep])
    _, o2 = _run_gpu(w2)
    a, b = o1[0][0].cpu(), o2[0][0].cpu()
    assert torch.equal(a[17:317], b[0:300]) and torch.equal(a[0:16], b[300:316])


@pytest.mark.parametrize("kind", ["f32", "q8"])
def test_decode_path_multirow_composition_invariance_bitwise(kind, gpu_available):
    """Multi-row segments of fp32 and 8-bit pools give the same bits
    whatever else shares the step, and match the oracle.  On the fp32 pool
    they take the decode path and their rows straddle a partition edge
    (512), so some rows are written directly and others merged from per-row
    partials; on the 8-bit pool they take the chunk kernel's 8-bit form
    (200 and 115 (row, head) pairs: two row tiles and one, the second tile
    partly empty) while the decode rows take the 8-bit decode kernel."""
    import torch
    if kind == "f32":
        base = [(0, 505, 12), (1, 50, 1), (2, 1000, 7), (3, 2000, 1)]
        rows = {0: slice(0, 12), 2: slice(13, 20)}
        hq, hkv, d = 8, 2, 64
    else:
        base = [(0, 480, 40), (1, 50, 1), (2, 1000, 23), (3, 2000, 1)]
        rows = {0: slice(0, 40), 2: slice(41, 64)}
        hq, hkv, d = 40, 8, 128

    def build():
        w = make_custom(base, dtype="f32" if kind == "f32" else "bf16", hq=hq, hkv=hkv, d=d, seed=83)
        if kind == "q8":
            w.kv_quant = "q8"
        return w

    w1 = build()
    _, o1 = _run_gpu(w1)
    res, _ = run_workload(w1)
    _check_close(f"decode-path multi-row {kind}", o1[0][0], res[0]["out"], TOL["f32"] if kind == "f32" else TOL["bf16"])
    w2 = build()
    st = w2.steps[0]
    keep = [2, 0]
    st.segments = [st.segments[i] for i in keep]
    st.q = np.concatenate([st.q[rows[i]] for i in keep])
    st.k_new = np.concatenate([st.k_new[rows[i]] for i in keep])
    st.v_new = np.concatenate([st.v_new[rows[i]] for i in keep])
    _, o2 = _run_gpu(w2)
    a, b = o1[0][0].cpu(), o2[0][0].cpu()
    n2 = rows[2].stop - rows[2].start
    assert torch.equal(a[rows[2]], b[0:n2]) and torch.equal(a[rows[0]], b[n2:n2 + rows[0].stop - rows[0].start])


def test_block_permutation_invariance_bitwise(gpu_available):
    import torch
    w = make_custom([(0, 900, 1), (1, 40, 1), (2, 1500, 1)], dtype="bf16", hq=32, hkv=8, d=128, seed=71)
    _, o1 = _run_gpu(w)
    other = np.random.default_rng(5).permutation(w.num_blocks).astype(np.int32)
    _, o2 = _run_gpu(w, free_order=other)
    assert torch.equal(o1[0][0].cpu(), o2[0][0].cpu())


def test_pool_beyond_4gib_bitwise(gpu_available):
    """Pool tensors over 4 GiB with every block of the step allocated above
    the 4 GiB mark give bitwise the outputs of a small pool: the chunk
    kernel's 64-bit tile addressing (used only for such pools) against its
    32-bit form, and the decode path's addressing at large offsets."""
    import copy
    import torch
    w = make_custom([(0, 500, 200), (1, 3000, 1), (2, 100, 64), (3, 2000, 16)], dtype="bf16", hq=32, hkv=8,
                    d=64, seed=73)
    _, small = _run_gpu(w, fused=True)
    big = copy.copy(w)
    big.num_blocks = 300_000       # 300K blocks x 8 heads x 16 x 64 x 2 B = 4.9 GB per tensor
    order = np.arange(big.num_blocks - 1, -1, -1, dtype=np.int32)    # highest blocks first
    eng, large = _run_gpu(big, free_order=order, fused=True)
    assert eng.pool.k.numel() * eng.pool.k.element_size() > 2 ** 32
    assert torch.equal(small[0][0].cpu(), large[0][0].cpu())
    del eng, large
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_slot_reuse_leaves_other_slots_bitwise_unchanged(fused, gpu_available):
    """Config 5: after slot 3 is released and its blocks reused by a new
    prompt, the replayed rows of slots 0, 1, 2, 4 are bitwise unchanged."""
    import torch
    w = _workload("5")
    _, outs = _run_gpu(w, fused=fused)
    s1, s2 = outs[0][0].cpu(), outs[1][0].cpu()
    for i in (0, 1, 2):
        assert torch.equal(s2[16 * i:16 * i + 16], s1[16 * i:16 * i + 16])
    assert torch.equal(s2[3048:3064], s1[64:80])


# ------------------------------------------------------------------ shared prefixes
def test_copy_blocks_bit_exact(gpu_available):
    """pkv_copy_blocks against the oracle's block copy over the whole pool;
    pairs with an id outside the pool are skipped."""
    import torch
    from oracle.attention import copy_blocks_reference
    from workloads import bf16_bits_from_f32
    from workloads.drive import torch_dtype
    rng = np.random.default_rng(11)
    for dtype, d, hkv in [("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 1)]:
        _log(f"copy_blocks {dtype} D{d} Hkv{hkv}")
        nb = 40
        shape = (nb, hkv, 16, d)
        raw = [rng.standard_normal(shape, dtype=np.float32) for _ in range(2)]
        if dtype == "bf16":
            raw = [bf16_bits_from_f32(x) for x in raw]
        pool = pk.KVPool(nb, hkv, d, torch_dtype(dtype), poison=False)
        pool.k.copy_(to_device(raw[0], dtype, "cuda").view(shape))
        pool.v.copy_(to_device(raw[1], dtype, "cuda").view(shape))
        src = rng.choice(20, size=7).astype(np.int32)                # repeats allowed
        dst = rng.choice(np.arange(20, nb), size=7, replace=False).astype(np.int32)
        spare = [b for b in range(20, nb) if b not in dst][0]          # must stay untouched
        bad_src = np.array([nb + 3, 5], np.int32)
        bad_dst = np.array([spare, -1], np.int32)
        all_src = torch.from_numpy(np.concatenate([src, bad_src])).cuda()
        all_dst = torch.from_numpy(np.concatenate([dst, bad_dst])).cuda()
        pk.copy_blocks(all_src, all_dst, pool)
        pk.copy_blocks(all_src[:0], all_dst[:0], pool)                # no-op
        torch.cuda.synchronize()
        wk, wv = copy_blocks_reference(raw[0], raw[1], src, dst)
        assert np.array_equal(_pool_bits(pool.k), _oracle_bits(wk))
        assert np.array_equal(_pool_bits(pool.v), _oracle_bits(wv))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_prefix_adoption_matches_oracle_and_cold_bitwise(fused, gpu_available):
    """Eight requests over one 1000-token prefix: adopted by reference (seven
    copy-on-write copies in step 0) versus prefilled cold.  Every step's output
    is within tolerance of the oracle and bit-identical to the cold run's; the
    pool after the adopting run equals the oracle's bit for bit."""
    _log(f"prefix adoption fused={fused}")
    wa, wc = _workload("prefix"), _workload("prefix-cold")
    ea, oa = _run_gpu(wa, fused=fused)
    _, oc = _run_gpu(wc, fused=fused)
    res, (ok, ov) = _oracle("prefix")
    assert len(oa) == len(oc) == len(res) == 3
    for i, ((a, ma), (c, _), r) in enumerate(zip(oa, oc, res)):
        _check_close(f"prefix step {i}", a, r["out"], TOL[wa.dtype])
        assert np.array_equal(a.cpu().numpy().view(np.int32), c.cpu().numpy().view(np.int32)), f"step {i}"
        assert np.array_equal(ma.host["copy_src"], r["meta"]["copy_src"])
        assert np.array_equal(ma.host["copy_dst"], r["meta"]["copy_dst"])
    assert np.array_equal(_pool_bits(ea.pool.k), _oracle_bits(ok))
    assert np.array_equal(_pool_bits(ea.pool.v), _oracle_bits(ov))


# ------------------------------------------------------------------ gather ablation
def _gather_then_attend(w, eng, meta, q):
    """Rebuild every segment's window contiguously in a second (poisoned)
    pool with pkv_gather_kv, then attend over it through identity tables.
    Returns (out, gathered pool, per-segment first block, block counts)."""
    import torch
    from workloads.drive import pool_torch_dtype
    h = meta.host
    r2s, ctx = h["row_to_slot"], h["context_lens"]
    nbs = [-(-int(ctx[s]) // 16) for s in r2s]
    start = np.concatenate([[0], np.cumsum(nbs)[:-1]]).astype(np.int32)
    dst = pk.KVPool(int(sum(nbs)) + 1, w.num_kv_heads, w.head_dim, pool_torch_dtype(w))
    dense = np.zeros((w.max_slots, max(nbs)), np.int32)
    for b, s in enumerate(r2s):
        dense[s, :nbs[b]] = start[b] + np.arange(nbs[b])
    pk.gather_kv(meta.row_to_slot, meta.context_lens, eng.d_block_tables, torch.from_numpy(start).cuda(),
                 eng.pool, dst, max_context_len=meta.max_context_len)
    out = torch.empty((meta.total_q, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    pk.paged_attend(q, meta.row_to_slot, meta.query_start, meta.query_len, meta.context_lens,
                    torch.from_numpy(dense).cuda(), dst, w.scale, max_query_len=meta.max_query_len,
                    max_context_len=meta.max_context_len, out=out, workspace=eng.workspace_for(meta))
    torch.cuda.synchronize()
    return out, dst, start, nbs


@pytest.mark.parametrize("name", ["3", "gather-mixed"])
def test_gather_then_attend_equals_paged_bitwise(name, gpu_available):
    """The gather path (rebuild each window contiguously, then attend through
    identity tables) gives the block-table path's output bit for bit, and the
    rebuilt windows equal the oracle's logical gather of each sequence."""
    from oracle.attention import gather_sequence
    from workloads.drive import step_tensors
    _log(f"gather ablation parity {name}")
    if name == "gather-mixed":
        w = make_custom([(0, 700, 16), (1, 3000, 3), (2, 200, 40), (3, 1300, 1), (4, 0, 1)],
                        dtype="bf16", hq=32, hkv=8, d=128, seed=23)
        res, (ok, ov) = run_workload(w)
    else:
        w = _workload(name)
        res, (ok, ov) = _oracle(name)
    eng, outs = _run_gpu(w)
    out_paged, meta = outs[-1]
    _, _, q = step_tensors(w, len(w.steps) - 1)
    out, dst, start, nbs = _gather_then_attend(w, eng, meta, q)
    assert np.array_equal(out.cpu().numpy().view(np.int32), out_paged.cpu().numpy().view(np.int32))
    tables = res[-1]["meta"]["block_tables"]
    gk, gv = _pool_bits(dst.k), _pool_bits(dst.v)
    for b, s in enumerate(meta.host["row_to_slot"].tolist()):
        L = int(meta.host["context_lens"][s])
        for got_pool, want_pool in ((gk, ok), (gv, ov)):
            got = got_pool[start[b]:start[b] + nbs[b]].transpose(0, 2, 1, 3).reshape(-1, w.num_kv_heads,
                                                                                    w.head_dim)[:L]
            want = gather_sequence(want_pool, tables[s], L, 16)
            assert np.array_equal(got, _oracle_bits(want)), f"segment {b}"


# ------------------------------------------------------------------ 8-bit KV
Q8_EDGE = [
    [(0, 0, 1)],                                  # L = 1
    [(0, 15, 1), (1, 16, 1), (2, 31, 1)],         # block edges
    [(0, 511, 1), (1, 512, 1), (2, 1023, 1), (3, 1024, 1), (4, 2047, 1), (5, 2048, 1)],   # partition edges
    [(5, 3000, 1), (2, 7, 1)],                    # slots out of order
]


def _q8_workload(seqs, d, hq, hkv, seed=7):
    w = make_custom(seqs, dtype="bf16", hq=hq, hkv=hkv, d=d, seed=seed)
    w.kv_quant = "q8"
    return w


def _q8_pool_check(eng, pools):
    (ck, sk), (cv, sv) = pools
    assert np.array_equal(eng.pool.k.cpu().numpy(), ck)
    assert np.array_equal(eng.pool.v.cpu().numpy(), cv)
    assert np.array_equal(eng.pool.k_scale.cpu().numpy().view(np.uint32), sk.view(np.uint32))
    assert np.array_equal(eng.pool.v_scale.cpu().numpy().view(np.uint32), sv.view(np.uint32))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_q8_config3_append_bit_exact_and_attention(fused, gpu_available):
    """Config 3 with an 8-bit pool: codes and scales bit-exact with the
    oracle's quantizer over the whole pool (poison included); attention
    within 1e-2 of the oracle's fp64 attention over code * scale."""
    _log(f"q8 config 3q fused={fused}")
    w = _workload("3q")
    eng, outs = _run_gpu(w, fused=fused)
    res, pools = _oracle("3q")
    _q8_pool_check(eng, pools)
    _check_close("config 3q", outs[0][0], res[0]["out"], TOL["bf16"])


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 8, 8), (128, 40, 8), (64, 8, 1), (128, 32, 4),
                                      (128, 24, 8), (64, 14, 2)])   # G 4, 1, 5, 8, 8, 3, 7
@pytest.mark.parametrize("case", range(len(Q8_EDGE)))
def test_q8_edge_cases(d, hq, hkv, case, gpu_available):
    _log(f"q8 edge case {case} D{d} {hq}/{hkv}")
    w = _q8_workload(Q8_EDGE[case], d, hq, hkv, seed=40 + case)
    eng, outs = _run_gpu(w)
    res, pools = run_workload(w)
    _q8_pool_check(eng, pools)
    _check_close(f"q8 edge {case}", outs[0][0], res[0]["out"], TOL["bf16"])


def test_q8_zero_rows_and_bf16_output(gpu_available):
    """Rows of zeros quantize to codes 0 with scale 0 and attend as zeros;
    bf16 output is the fp32 result rounded to nearest even."""
    import torch
    w = _q8_workload([(0, 300, 1), (1, 40, 1)], 128, 16, 8, seed=61)
    for slot, hk, hv in w.history:
        hk[::7] = 0                               # every 7th token's K rows all zero
        hv[::5] = 0
    _, outs = _run_gpu(w)
    _, outs_b = _run_gpu(w, out_dtype=torch.bfloat16)
    res, _ = run_workload(w)
    _check_close("q8 zero rows", outs[0][0], res[0]["out"], TOL["bf16"])
    f = outs[0][0].cpu()
    assert torch.equal(outs_b[0][0].cpu(), f.to(torch.bfloat16))


def test_q8_copy_on_write_and_gather(gpu_available):
    """On an 8-bit pool the copy-on-write copies and the gather carry the
    scales with the codes: the prefix workload matches the oracle and the
    cold run bit for bit, and gather-then-attend equals paged attention."""
    from workloads import make_prefix_share
    # one-token suffixes: 8-bit pools attend decode rows only
    wa, wc = make_prefix_share(False, suffixes=(1,) * 8), make_prefix_share(True, suffixes=(1,) * 8)
    wa.kv_quant = wc.kv_quant = "q8"
    _log("q8 prefix adoption")
    ea, oa = _run_gpu(wa, fused=True)
    _, oc = _run_gpu(wc, fused=True)
    res, pools = run_workload(wa)
    _q8_pool_check(ea, pools)
    assert len(res[0]["meta"]["copy_src"]) == 7
    for i, ((a, _), (c, _), r) in enumerate(zip(oa, oc, res)):
        _check_close(f"q8 prefix step {i}", a, r["out"], TOL["bf16"])
        assert np.array_equal(a.cpu().numpy().view(np.int32), c.cpu().numpy().view(np.int32))
    from workloads.drive import step_tensors
    out_paged, meta = oa[-1]
    _, _, q = step_tensors(wa, len(wa.steps) - 1)
    out, _, _, _ = _gather_then_attend(wa, ea, meta, q)
    assert np.array_equal(out.cpu().numpy().view(np.int32), out_paged.cpu().numpy().view(np.int32))


@pytest.mark.parametrize("case", [4, 5, 6])
@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 40, 8)])
def test_q8_multirow_edge_cases(case, d, hq, hkv, gpu_available):
    """Multi-row segments on an 8-bit pool (the chunk kernel's 8-bit form):
    tiny prompts, drafts, and chunks whose rows span several key ranges."""
    _log(f"q8 multirow case {case} D{d} {hq}/{hkv}")
    w = _q8_workload(EDGE_SEQS[case], d, hq, hkv, seed=70 + case)
    eng, outs = _run_gpu(w)
    res, pools = run_workload(w)
    _q8_pool_check(eng, pools)
    _check_close(f"q8 multirow {case}", outs[0][0], res[0]["out"], TOL["bf16"])


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_q8_config5(fused, gpu_available):
    """Config 5 on an 8-bit pool: 16-row drafts, then rollback, slot reuse
    and a 3000-row prompt, all on the chunk kernel's 8-bit form."""
    _log(f"q8 config 5 fused={fused}")
    w = _workload("5q")
    eng, outs = _run_gpu(w, fused=fused)
    res, pools = _oracle("5q")
    _q8_pool_check(eng, pools)
    for i, ((out, _), r) in enumerate(zip(outs, res)):
        _check_close(f"q8 config 5 step {i}", out, r["out"], TOL["bf16"])


# ------------------------------------------------------------------ randomized mixes
def _random_mix(seed):
    """A seeded random step: 1-9 segments mixing decode rows, short drafts
    and chunks, random contexts (block and partition edges likely), a random
    head layout, head dim, pool type and slot numbering."""
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 5, 8]))
    kind = ["f32", "bf16", "bf16", "q8"][int(rng.integers(0, 4))]
    nseg = int(rng.integers(1, 10))
    slots = rng.choice(32, size=nseg, replace=False)
    seqs = []
    for s in slots:
        r = rng.random()
        n = 1 if r < 0.5 else (int(rng.integers(2, 17)) if r < 0.8 else int(rng.integers(17, 200)))
        if kind == "f32" and n > 1:
            n = min(n, 8)
        edge = int(rng.choice([0, 1, 15, 16, 17, 511, 512, 513, 1023, 1024]))
        hist = int(rng.integers(0, 2500)) if rng.random() < 0.6 else edge
        seqs.append((int(s), hist, n))
    w = make_custom(seqs, dtype="f32" if kind == "f32" else "bf16", hq=g * hkv, hkv=hkv, d=d, seed=seed,
                    max_slots=32)
    if kind == "q8":
        w.kv_quant = "q8"
    return w, kind


@pytest.mark.parametrize("seed", range(64))
def test_random_mixed_steps(seed, gpu_available):
    w, kind = _random_mix(seed)
    _log(f"random mix {seed}: {kind} D{w.head_dim} {w.num_q_heads}/{w.num_kv_heads} "
         f"segs {[(s.slot, s.n) for s in w.steps[0].segments]}")
    fused = bool(seed % 2)
    eng, outs = _run_gpu(w, fused=fused)
    res, pools = run_workload(w)
    tol = TOL["f32"] if kind == "f32" else TOL["bf16"]
    _check_close(f"random mix {seed}", outs[0][0], res[0]["out"], tol)
    if kind == "q8":
        _q8_pool_check(eng, pools)
    else:
        ok, ov = pools
        assert np.array_equal(_pool_bits(eng.pool.k), _oracle_bits(ok))
        assert np.array_equal(_pool_bits(eng.pool.v), _oracle_bits(ov))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_pool_past_4gib_equals_small_pool_bitwise(fused, gpu_available):
    """K and V tensors of more than 4 GiB each, with the step's blocks at the
    top of the pool (the allocator hands them out from the end): tile
    addresses no longer fit 32 bits, and the chunk kernel takes its 64-bit
    form.  A prompt chunk, decode rows and a draft give the same bits as on
    a small pool, and match the oracle."""
    import copy
    seqs = [(0, 3000, 200), (1, 2000, 1), (2, 1500, 3), (3, 5000, 1)]
    w = make_custom(seqs, dtype="bf16", hq=32, hkv=8, d=128, seed=91)
    _, small = _run_gpu(w, fused=fused)
    per_block = w.num_kv_heads * 16 * w.head_dim * 2
    wb = copy.copy(w)
    wb.num_blocks = (1 << 32) // per_block + w.num_blocks + 64
    assert wb.num_blocks * per_block > (1 << 32)
    _log(f"pool past 4 GiB: {wb.num_blocks} blocks, {wb.num_blocks * per_block / 2**30:.2f} GiB per tensor")
    order = np.arange(wb.num_blocks - 1, -1, -1, dtype=np.int32)
    big, outs = _run_gpu(wb, fused=fused, free_order=order)
    assert int(big.d_block_tables.max()) * per_block >= (1 << 32)   # tiles past 4 GiB are in use
    assert np.array_equal(outs[0][0].cpu().numpy().view(np.int32), small[0][0].cpu().numpy().view(np.int32))
    res, _ = run_workload(w)
    _check_close("pool past 4 GiB", outs[0][0], res[0]["out"], TOL["bf16"])
    del big, outs


@functools.lru_cache(maxsize=2)
def _long_contexts(kind):
    """Contexts past 32768 tokens, where a row has more than one wavefront's
    worth (64) of 512-token partitions: decode rows at ~33K, 40K and 70K
    (up to 137 partitions), a 3-row draft at 45K (verify path on bf16) and a
    40-row chunk at 36K (16 key ranges on bf16); on an 8-bit pool all of
    them run on the 8-bit decode kernel."""
    seqs = [(0, 40000, 1), (1, 70000, 1), (2, 45000, 3), (3, 36000, 40), (4, 33000, 1)]
    w = make_custom(seqs, dtype="bf16", hq=32, hkv=8, d=128, seed=77)
    if kind == "q8":
        w.kv_quant = "q8"
    res, pools = run_workload(w)
    return w, res, pools


@pytest.mark.parametrize("kind,fused", [("bf16", False), ("bf16", True), ("q8", True)],
                         ids=["bf16-separate", "bf16-mixed_step", "q8-mixed_step"])
def test_long_contexts_past_64_partitions(kind, fused, gpu_available):
    _log(f"long contexts {kind} fused={fused}")
    w, res, pools = _long_contexts(kind)
    eng, outs = _run_gpu(w, fused=fused)
    _check_close(f"long contexts {kind}", outs[0][0], res[0]["out"], TOL["bf16"])
    if kind == "q8":
        _q8_pool_check(eng, pools)
    else:
        ok, ov = pools
        assert np.array_equal(_pool_bits(eng.pool.k), _oracle_bits(ok))
        assert np.array_equal(_pool_bits(eng.pool.v), _oracle_bits(ov))


def _many_segments(d, hq, hkv, seed):
    """100 segments, more than one wavefront holds: decode rows, then prompt
    chunks (cut into key ranges), then short drafts, then decode rows again,
    so that the chunk, merge and verify kernels find their segments and
    partial slots past the first 64 segments."""
    rng = np.random.default_rng(seed)
    seqs = []
    for s in range(60):
        seqs.append((s, int(rng.integers(0, 700)), 1))
    for s in range(60, 70):
        seqs.append((s, int(rng.integers(1500, 3000)), int(rng.integers(20, 81))))
    for s in range(70, 85):
        seqs.append((s, int(rng.integers(0, 1200)), int(rng.integers(2, 9))))
    for s in range(85, 100):
        seqs.append((s, int(rng.integers(0, 1100)), 1))
    order = rng.permutation(30) + 55          # shuffle the middle, across the 64-segment boundary
    seqs[55:85] = [seqs[i] for i in order]
    return make_custom(seqs, dtype="bf16", hq=hq, hkv=hkv, d=d, seed=seed, max_slots=128)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 40, 8)])
def test_many_segments_beyond_one_wavefront(d, hq, hkv, fused, gpu_available):
    _log(f"100 segments D{d} {hq}/{hkv} fused={fused}")
    w = _many_segments(d, hq, hkv, seed=4242 + d)
    eng, outs = _run_gpu(w, fused=fused)
    res, (ok, ov) = run_workload(w)
    _check_close(f"100 segments D{d}", outs[0][0], res[0]["out"], TOL["bf16"])
    assert np.array_equal(_pool_bits(eng.pool.k), _oracle_bits(ok))
    assert np.array_equal(_pool_bits(eng.pool.v), _oracle_bits(ov))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "mixed_step"])
def test_many_segments_beyond_one_wavefront_q8(fused, gpu_available):
    """The same 100-segment step over an 8-bit pool: the multi-row segments
    take the workgroup form of the 8-bit decode kernel and the decode rows
    the one-wavefront form, both finding their units past the first 64
    segments."""
    _log(f"100 segments q8 fused={fused}")
    w = _many_segments(128, 40, 8, seed=4343)
    w.kv_quant = "q8"
    eng, outs = _run_gpu(w, fused=fused)
    res, pools = run_workload(w)
    _check_close("100 segments q8", outs[0][0], res[0]["out"], TOL["bf16"])
    _q8_pool_check(eng, pools)


@pytest.mark.parametrize("name", ["1", "2", "3", "3v", "4a", "4b", "5", "3q", "5q", "prefix"])
def test_one_call_step_equals_split_calls_bitwise(name, gpu_available):
    """pkv_mixed_step picks prefetch depths, column tiles, skipped launches
    and the auxiliary stream from the host's view of the step; the split
    calls (pkv_kv_append, then pkv_paged_attend) know none of that.  Neither
    choice may change arithmetic: outputs and pools are bit-identical."""
    _log(f"one-call vs split {name}")
    w = _workload(name)
    e1, o1 = _run_gpu(w, fused=True)
    e2, o2 = _run_gpu(w, fused=False)
    for i, ((a, _), (b, _)) in enumerate(zip(o1, o2)):
        assert np.array_equal(a.cpu().numpy().view(np.int32), b.cpu().numpy().view(np.int32)), f"step {i}"
    assert np.array_equal(e1.pool.k.cpu().view(torch_int_view(e1.pool.k)).numpy(),
                          e2.pool.k.cpu().view(torch_int_view(e2.pool.k)).numpy())


def torch_int_view(t):
    import torch
    return {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int8: torch.int8}[t.dtype]
