"""GPU closed forms: results that plain mathematics fixes, on every kernel path.

Attention over one sequence is the plain definition (lucebox blog,
"Continuous batching: Qwen3.8-27B at 301 tok/s ...", §Paged KV and paged
attention: the block table changes only where tokens live):
    O = sum_j w_j V_j / sum_j w_j,  w_j = exp(scale q . K_j - max)
over the keys the row sees (row i of an n-row segment sits at L - n + i;
§Packing unequal prompt chunks together).  So, whatever the kernel:
  * one visible key: O = V_0 exactly (one weight, normalised by itself);
  * all V equal to c: O = c up to fp32 summation rounding;
  * q = 0: every weight is 1, O = the mean of the visible V;
  * one key scoring ~100 above the rest: O = that key's V (the other
    weights are below e^-90);
  * identical queries across a GQA group: identical outputs, bit for bit
    (each head runs the same arithmetic on the same data).
Paths: bf16 decode rows (MFMA kernel), fp32 decode rows (vector kernel),
short drafts (verify kernel), prompt chunks (chunk kernel, with and without
key-range splits), and the 8-bit pool (decode rows and multi-row segments).
The 8-bit pool's stored value is code x scale (its own format), and its
product weights that value by fp16(p v_scale) / v_scale, which the row sum
matches; its bounds say where that adds rounding.
"""
import numpy as np
import pytest

import paged_kv_attention_slot_amd as pk
from workloads import bf16_bits_from_f32, make_custom
from workloads.drive import make_engine, place_history, run_step

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24          # fp32 unit roundoff


def _log(msg):
    print(msg, flush=True)


# (label, dtype, kv_quant, hq, hkv, d, seqs): seqs are (slot, history, rows)
PATHS = [
    ("decode-bf16-mfma", "bf16", "", 32, 8, 128, [(0, 0, 1), (1, 40, 1), (2, 700, 1), (3, 2100, 1)]),
    ("decode-f32-valu", "f32", "", 8, 2, 64, [(0, 0, 1), (1, 40, 1), (2, 700, 1), (3, 1100, 1)]),
    ("verify-drafts", "bf16", "", 32, 8, 128, [(0, 0, 2), (1, 30, 3), (2, 600, 4), (3, 1500, 2)]),
    ("chunk", "bf16", "", 32, 8, 64, [(0, 0, 40), (1, 90, 200), (2, 5, 150)]),
    ("chunk-split", "bf16", "", 8, 8, 128, [(0, 0, 2048), (1, 2000, 40), (2, 3000, 16)]),
    ("chunk-d128-g5", "bf16", "", 40, 8, 128, [(0, 0, 16), (1, 1000, 16), (2, 77, 16)]),
    ("q8-decode", "bf16", "q8", 32, 8, 128, [(0, 0, 1), (1, 40, 1), (2, 700, 1), (3, 2100, 1)]),
    ("q8-multirow", "bf16", "q8", 16, 8, 64, [(0, 0, 5), (1, 40, 3), (2, 600, 24)]),
]


def _to_f32(w, a):
    if w.dtype == "f32":
        return np.asarray(a, np.float32)
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _from_f32(w, x):
    x = np.ascontiguousarray(x, np.float32)
    return x.copy() if w.dtype == "f32" else bf16_bits_from_f32(x)


def _make(path, seed):
    label, dtype, quant, hq, hkv, d, seqs = path
    w = make_custom(seqs, dtype=dtype, hq=hq, hkv=hkv, d=d, seed=seed)
    if quant:
        w.kv_quant = quant
    return w


def _run(w, out_dtype=None, fused=False):
    import torch
    eng = make_engine(pk.PagedKVEngine, w)
    place_history(eng, w)
    out, meta = run_step(eng, w, 0, out_dtype=out_dtype, fused=fused)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), eng


def _segments(w):
    """(row0, n, history, slot) per segment, in packed order."""
    hist = {slot: len(k) for slot, k, _ in w.history}
    out, r0 = [], 0
    for seg in w.steps[0].segments:
        out.append((r0, seg.n, hist[seg.slot], seg.slot))
        r0 += seg.n
    return out


def _logical(w, which):
    """Per slot, the float32 K or V of every token after the step (history
    then the step's new rows): [L][Hkv][D]."""
    idx = 1 if which == "k" else 2
    new = w.steps[0].k_new if which == "k" else w.steps[0].v_new
    res = {}
    for (r0, n, h, slot), (s2, *kv) in zip(_segments(w), w.history):
        assert s2 == slot
        res[slot] = np.concatenate([_to_f32(w, kv[idx - 1]), _to_f32(w, new[r0:r0 + n])])
    return res


def _stored_v(w, v_by_slot):
    """The values the pool stores for V: the inputs themselves, or code x
    scale on an 8-bit pool (the oracle's quantizer, pinned on the CPU)."""
    if not w.kv_quant:
        return {s: v.astype(np.float64) for s, v in v_by_slot.items()}
    from oracle.quant import dequantize, quantize_rows
    res = {}
    for s, v in v_by_slot.items():
        bits = bf16_bits_from_f32(v)                   # inputs are bf16 already: exact
        codes, scales = quantize_rows(bits)
        res[s] = dequantize(codes, scales)
    return res


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_first_row_of_each_sequence_start_sees_v0(path, gpu_available):
    """A row that sees one key (position 0: a decode row at L = 1, or row 0
    of a segment starting at offset 0) returns that key's V: bit for bit on
    bf16 and fp32 pools; to fp32 rounding of code x scale on 8-bit pools."""
    import torch
    w = _make(path, seed=11)
    _log(f"one visible key: {path[0]}")
    g = w.num_q_heads // w.num_kv_heads
    v = _stored_v(w, _logical(w, "v"))
    for out_dtype in ((None,) if w.dtype == "f32" else (None, torch.bfloat16)):
        got, _ = _run(w, out_dtype=out_dtype)
        checked = 0
        for r0, n, h, slot in _segments(w):
            if h != 0:
                continue
            want = v[slot][0][np.arange(w.num_q_heads) // g]          # [Hq][D]
            if w.kv_quant:
                tol = 8 * U32 * np.abs(want)
                if out_dtype is not None:                              # plus half a bf16 ulp
                    tol = tol + np.ldexp(1.0, np.frexp(np.abs(want))[1] - 9)
                assert (np.abs(got[r0] - want) <= tol).all(), f"row {r0}"
            else:
                assert np.array_equal(got[r0], want), f"row {r0}"
            checked += 1
        assert checked


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_constant_v_gives_that_value(path, gpu_available):
    """Every V of a sequence equal to one vector c (per KV head): each
    output row is c up to fp32 summation rounding, (2 keys + 16) ulp."""
    w = _make(path, seed=12)
    _log(f"constant V: {path[0]}")
    rng = np.random.default_rng(5)
    g = w.num_q_heads // w.num_kv_heads
    st = w.steps[0]
    segs = _segments(w)
    consts = {}
    for i, (slot, kh, vh) in enumerate(w.history):
        c = rng.standard_normal((w.num_kv_heads, w.head_dim)).astype(np.float32)
        consts[slot] = c
        w.history[i] = (slot, kh, _from_f32(w, np.broadcast_to(c, (len(vh),) + c.shape)))
    vn = _to_f32(w, st.v_new).copy()
    for r0, n, h, slot in segs:
        vn[r0:r0 + n] = consts[slot]
    st.v_new = _from_f32(w, vn)
    stored = _stored_v(w, _logical(w, "v"))
    got, _ = _run(w)
    for r0, n, h, slot in segs:
        c = stored[slot][0][np.arange(w.num_q_heads) // g]             # [Hq][D] (all tokens equal)
        # 8-bit pool: codes enter the product as fp16 1152 + code and the
        # constant is taken out in fp32 afterwards, which leaves up to
        # (keys) ulp of 1152 x v_scale (the row's scale is max|c| / 127)
        vscale = np.abs(c).max(-1, keepdims=True) / 127.0
        for i in range(n):
            keys = h + i + 1
            tol = (2 * keys + 16) * U32 * np.abs(c)
            if w.kv_quant:
                tol = tol + 2.0 ** -21 * np.abs(c) + (2 * keys + 16) * U32 * 1152.0 * vscale
            err = np.abs(got[r0 + i] - c)
            assert (err <= tol + 1e-30).all(), f"row {r0 + i}: max err {err.max()}"


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_zero_query_gives_mean_of_visible_v(path, gpu_available):
    """q = 0 makes every weight exactly 1: each row returns the mean of the
    V it sees (fp32 summation bound; on an 8-bit pool the weights are
    fp16(v_scale) / v_scale, within 2^-11 of 1)."""
    w = _make(path, seed=13)
    _log(f"zero query: {path[0]}")
    st = w.steps[0]
    st.q = _from_f32(w, np.zeros(_to_f32(w, st.q).shape, np.float32))
    stored = _stored_v(w, _logical(w, "v"))
    g = w.num_q_heads // w.num_kv_heads
    got, _ = _run(w)
    heads = np.arange(w.num_q_heads) // g
    for r0, n, h, slot in _segments(w):
        vs = stored[slot][:, heads]                                    # [L][Hq][D]
        csum = np.cumsum(vs, axis=0)
        cabs = np.cumsum(np.abs(vs), axis=0)
        for i in range(n):
            keys = h + i + 1
            mean = csum[keys - 1] / keys
            bound = 2 * (keys + 16) * U32 * cabs[keys - 1] / keys + 4 * U32 * np.abs(mean)
            if w.kv_quant:
                bound = bound + 2.0 ** -10 * np.abs(vs[:keys] - mean).max(0)
            err = np.abs(got[r0 + i] - mean)
            assert (err <= bound + 1e-30).all(), f"row {r0 + i}: max err {err.max()}"


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_dominant_key_gives_its_v(path, gpu_available):
    """One key of each sequence (visible to every row) scores ~100 (natural
    log units) above all others: every row returns that key's V."""
    w = _make(path, seed=14)
    _log(f"dominant key: {path[0]}")
    rng = np.random.default_rng(6)
    g = w.num_q_heads // w.num_kv_heads
    st = w.steps[0]
    segs = _segments(w)
    d = w.head_dim
    u = rng.standard_normal((w.num_kv_heads, d)).astype(np.float32)
    u = _to_f32(w, _from_f32(w, u / np.linalg.norm(u, axis=1, keepdims=True) * np.sqrt(d)))
    beta = 100.0 / (w.scale * (u * u).sum(1))                          # score of the chosen key: 100
    chosen = {}
    kn = _to_f32(w, st.k_new).copy()
    qn = _to_f32(w, st.q).copy()
    for (r0, n, h, slot), i in zip(segs, range(len(segs))):
        L = h + n
        j = int(rng.integers(0, L - n + 1))                            # seen by row 0, hence by all
        chosen[slot] = j
        keys = 0.02 * rng.standard_normal((L, w.num_kv_heads, d)).astype(np.float32)
        keys[j] = beta[:, None] * u
        slot_, kh, vh = w.history[i]
        w.history[i] = (slot_, _from_f32(w, keys[:h]), vh)
        kn[r0:r0 + n] = keys[h:]
        qn[r0:r0 + n] = u[np.arange(w.num_q_heads) // g]
    st.k_new, st.q = _from_f32(w, kn), _from_f32(w, qn)
    stored = _stored_v(w, _logical(w, "v"))
    got, _ = _run(w)
    for r0, n, h, slot in segs:
        want = stored[slot][chosen[slot]][np.arange(w.num_q_heads) // g]
        for i in range(n):
            np.testing.assert_allclose(got[r0 + i], want, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
def test_gqa_twins_are_bitwise_identical(path, gpu_available):
    """The same query on every head of a KV head's group: the group's outputs
    are identical bit for bit (split-key merges and partitions included)."""
    w = _make(path, seed=15)
    _log(f"GQA twins: {path[0]}")
    g = w.num_q_heads // w.num_kv_heads
    if g == 1:
        pytest.skip("one query head per KV head")
    st = w.steps[0]
    q = _to_f32(w, st.q).copy()
    t = q.shape[0]
    q = q.reshape(t, w.num_kv_heads, g, w.head_dim)
    q[:] = q[:, :, :1].copy()
    st.q = _from_f32(w, q.reshape(t, w.num_q_heads, w.head_dim))
    for fused in (False, True):
        got, _ = _run(w, fused=fused)
        o = got.reshape(t, w.num_kv_heads, g, w.head_dim)
        assert np.array_equal(o, np.broadcast_to(o[:, :, :1], o.shape))
