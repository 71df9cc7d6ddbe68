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
@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 8, 8), (128, 40, 8), (64, 8, 1)])
@pytest.mark.parametrize("case", range(len(EDGE_SEQS)))
def test_edge_cases(dtype, d, hq, hkv, case, gpu_available):
    seqs = EDGE_SEQS[case]
    _log(f"edge case {case} {dtype} D{d} {hq}/{hkv}")
    w = make_custom(seqs, dtype=dtype, hq=hq, hkv=hkv, d=d, seed=100 + case)
    _, outs = _run_gpu(w)
    res, _ = run_workload(w)
    _check_close(f"edge {case}", outs[0][0], res[0]["out"], TOL[dtype])


def test_single_token_context_is_v0(gpu_available):
    """One visible key: the output is that key's V.  The kernel forms the
    softmax weight as exp2(fma(s, c, -round(s c))), i.e. 1 + (rounding residue
    of s c), so the result is V0 within one fp32 ulp rather than bit-exact."""
    w = make_custom([(0, 0, 1)], dtype="bf16", hq=8, hkv=2, d=128, seed=5)
    _, outs = _run_gpu(w)
    out = outs[0][0].cpu().numpy()
    v = w.steps[0].v_new.astype(np.uint32) << 16
    v = v.view(np.float32)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], v[0, h // 4], rtol=2.0 ** -22, atol=0)


def test_bf16_output(gpu_available):
    import torch
    w = _workload("3")
    _, outs = _run_gpu(w, out_dtype=torch.bfloat16)
    res, _ = _oracle("3")
    got = outs[0][0].float().cpu().numpy()
    want = res[0]["out"]
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 9)
    assert (np.abs(got - want) <= 1e-2 + half_ulp).all()


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
