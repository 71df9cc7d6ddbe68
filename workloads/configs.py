"""The five seeded synthetic step configurations, plus small custom ones.

Shapes follow the pages' workloads:
  * "Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog),
    §Chunked prefill is a slot phase: a prompt slice C[1024:1536] advancing
    while other sequences decode (config 2), and §Keeping track of each
    request: a compact batch over non-contiguous slots (config 3);
  * mlxcel user guide "연속 배칭" (continuous batching), §청크 프리필
    (chunked prefill): four decoding streams while an 8192-token prompt is
    admitted in 2048- or 512-token chunks (config 4);
  * the lucebox blog's five clients with speculative verification
    (§Packing unequal prompt chunks together) and slot reuse after a
    sequence finishes (§Paged KV and paged attention) (config 5).

Random draws use numpy PCG64 with seed 1000+k for config k, in the order
lengths -> slot ids -> free-block permutation -> per-sequence history K, V
(packed sequence order) -> new K, V -> Q.  Values are N(0,1) float32; bf16
configs round them to bf16 by round-to-nearest-even on the bit pattern and
carry the raw uint16 patterns.  No public dataset or benchmark is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = ("1", "2", "3", "4a", "4b", "5")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Segment:
    """One entry of the packed batch: `n` rows for sequence slot `slot`.
    Each row is one new token of that sequence (appended this step)."""
    slot: int
    n: int


@dataclass
class Step:
    """One scheduler step.  `ops` are slot lifecycle events applied before the
    step: ("acquire", slot), ("release", slot), ("truncate", slot, new_len)
    (speculative drafts rejected) or ("adopt", slot, src_slot, num_tokens)
    (an empty slot shares src_slot's first num_tokens tokens).  Slots named in Workload.history are
    acquired when the history is placed, before the first step.  `k_new`/`v_new` are [T][Hkv][D] and `q` is
    [T][Hq][D], packed in segment order."""
    ops: list
    segments: list
    k_new: np.ndarray
    v_new: np.ndarray
    q: np.ndarray


@dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"; raw arrays are float32 / uint16
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_slots: int
    max_blocks_per_seq: int
    scale: float
    free_order: np.ndarray     # int32 permutation of [0, num_blocks): hand-out order
    history: list              # [(slot, k_hist [h][Hkv][D], v_hist)] placed before step 0
    steps: list                # [Step]
    description: str = ""
    notes: dict = field(default_factory=dict)
    kv_quant: str = ""         # "" (pool holds `dtype` values) or "q8" (8-bit codes + scales; inputs bf16)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


class _Draw:
    def __init__(self, seed: int, dtype: str):
        self.rng = np.random.default_rng(np.random.PCG64(seed))
        self.dtype = dtype

    def values(self, shape):
        x = self.rng.standard_normal(shape, dtype=np.float32)
        return x if self.dtype == "f32" else bf16_bits_from_f32(x)


def _blocks(tokens: int, bs: int) -> int:
    return -(-tokens // bs)


def _build(name, seed, dtype, hq, hkv, d, bs, seqs, *, num_blocks=None, pool_slack=1.1,
           max_slots=None, draw=None, description=""):
    """seqs: list of (slot, hist_len, new_len) in packed segment order.
    Draws the free-block permutation, then history K/V per sequence, then new
    K/V, then Q (all from `draw`, which may already have drawn lengths)."""
    draw = draw or _Draw(seed, dtype)
    need = sum(_blocks(h + n, bs) for _, h, n in seqs)
    if num_blocks is None:
        num_blocks = math.ceil(pool_slack * need)
    free_order = draw.rng.permutation(num_blocks).astype(np.int32)
    history = []
    for slot, h, _ in seqs:
        history.append((slot, draw.values((h, hkv, d)), draw.values((h, hkv, d))))
    t = sum(n for _, _, n in seqs)
    k_new = draw.values((t, hkv, d))
    v_new = draw.values((t, hkv, d))
    q = draw.values((t, hq, d))
    segs = [Segment(slot, n) for slot, _, n in seqs]
    step = Step(ops=[], segments=segs, k_new=k_new, v_new=v_new, q=q)
    maxb = max(_blocks(h + n, bs) for _, h, n in seqs)
    return Workload(
        name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
        num_blocks=num_blocks, max_slots=max_slots or (max(s for s, _, _ in seqs) + 1),
        max_blocks_per_seq=maxb, scale=1.0 / math.sqrt(d), free_order=free_order,
        history=history, steps=[step], description=description)


def make_custom(seqs, *, dtype="bf16", hq=4, hkv=2, d=64, bs=16, seed=7, num_blocks=None,
                pool_slack=1.5, max_slots=None, name="custom"):
    """Small workload: seqs = [(slot, hist_len, new_len)] in packed order."""
    return _build(name, seed, dtype, hq, hkv, d, bs, seqs, num_blocks=num_blocks,
                  pool_slack=pool_slack, max_slots=max_slots)


def _config1(variant_plus_one=False):
    # Tiny decode-only, fp32: 4 sequences, context lengths {17, 64, 130, 255}
    # after this step's single appended token (the other reading adds 1).
    lens = [17, 64, 130, 255]
    if variant_plus_one:
        lens = [x + 1 for x in lens]
    seqs = [(i, L - 1, 1) for i, L in enumerate(lens)]
    return _build("1+1" if variant_plus_one else "1", 1001, "f32", 8, 2, 64, 16, seqs,
                  num_blocks=64, description="decode-only fp32, 4 seqs, GQA 8/2, D64")


def _config2():
    draw = _Draw(1002, "bf16")
    lens = draw.rng.integers(200, 4001, size=8)
    # P1's "C[1024:1536] + decode(A, B)", widened to 8 decode rows; prompt first.
    seqs = [(8, 1024, 512)] + [(i, int(L) - 1, 1) for i, L in enumerate(lens)]
    return _build("2", 1002, "bf16", 32, 8, 128, 16, seqs, num_blocks=8192, draw=draw,
                  description="mixed: 8 decode rows + 512-row chunk at offset 1024, 32/8/128")


def _config3():
    draw = _Draw(1003, "bf16")
    z = draw.rng.standard_normal(64)
    lens = np.clip(np.round(np.exp(math.log(2048.0) + 1.0 * z)), 16, 32768).astype(np.int64)
    slots = draw.rng.choice(128, size=64, replace=False)
    seqs = [(int(s), int(L) - 1, 1) for s, L in zip(slots, lens)]
    return _build("3", 1003, "bf16", 32, 8, 128, 16, seqs, max_slots=128, draw=draw,
                  description="64 decode rows, lognormal context (median 2048), slots from 0..127")


def _config3v():
    """Config 3's sequences (same seed, lengths and slots), each verifying 2
    speculative draft rows in this step instead of decoding one token: the
    short multi-row segments of a multi-token-prediction verify step."""
    draw = _Draw(1003, "bf16")
    z = draw.rng.standard_normal(64)
    lens = np.clip(np.round(np.exp(math.log(2048.0) + 1.0 * z)), 16, 32768).astype(np.int64)
    slots = draw.rng.choice(128, size=64, replace=False)
    seqs = [(int(s), max(int(L) - 2, 0), 2) for s, L in zip(slots, lens)]
    return _build("3v", 1003, "bf16", 32, 8, 128, 16, seqs, max_slots=128, draw=draw,
                  description="64 sequences x 2 draft rows (verify), lognormal context (median 2048)")


def _config3q():
    """Config 3 (same seed, lengths, slots and values) with the KV pool held
    as 8-bit codes with one scale per (token, KV head): the bf16 K/V rows are
    quantized on append."""
    w = _config3()
    w.name = "3q"
    w.kv_quant = "q8"
    w.description = "64 decode rows, lognormal context (median 2048), 8-bit KV"
    return w


def _config5q():
    """Config 5 (same seed and values) with an 8-bit pool."""
    w = _config5()
    w.name = "5q"
    w.kv_quant = "q8"
    w.description = "speculative verify + slot reuse on an 8-bit KV pool"
    return w


def _config4(chunk):
    draw = _Draw(1004, "bf16")
    if chunk == 2048:
        prompt = (4, 6144, 2048)
    else:
        prompt = (4, 7680, 512)
    seqs = [prompt] + [(i, 8191, 1) for i in range(4)]
    nb = math.ceil(1.1 * 5 * 512)
    return _build("4a" if chunk == 2048 else "4b", 1004, "bf16", 32, 8, 64, 16, seqs,
                  num_blocks=nb, draw=draw,
                  description=f"4 decode rows at 8192 + {chunk}-row chunk of an 8192-token prompt, 32/8/64")


def _config5():
    draw = _Draw(1005, "bf16")
    lens = draw.rng.integers(1000, 16001, size=5)
    hq, hkv, d, bs = 40, 8, 128, 16
    seqs = [(i, int(L) - 16, 16) for i, L in enumerate(lens)]
    need = sum(_blocks(int(L), bs) for L in lens) + _blocks(3000, bs)
    nb = math.ceil(1.1 * need)
    w = _build("5", 1005, "bf16", hq, hkv, d, bs, seqs, num_blocks=nb, draw=draw,
               description="speculative verify: 5 seqs x 16 draft rows, 40/8/128; then slot 3 reused")
    s1 = w.steps[0]
    # Step 2: slot 3 finishes and is released; the other slots reject all 16
    # drafts (rolled back) and verify the same drafts again; a new 3000-token
    # prompt takes slot 3 and reuses its freed blocks first.
    new3_k = draw.values((3000, hkv, d))
    new3_v = draw.values((3000, hkv, d))
    new3_q = draw.values((3000, hq, d))
    ks, vs, qs, segs = [], [], [], []
    for i in range(5):
        if i == 3:
            ks.append(new3_k); vs.append(new3_v); qs.append(new3_q); segs.append(Segment(3, 3000))
        else:
            r = slice(16 * i, 16 * i + 16)
            ks.append(s1.k_new[r]); vs.append(s1.v_new[r]); qs.append(s1.q[r]); segs.append(Segment(i, 16))
    ops = [("release", 3)] + [("truncate", i, int(lens[i]) - 16) for i in (0, 1, 2, 4)] + [("acquire", 3)]
    w.steps.append(Step(ops=ops, segments=segs, k_new=np.concatenate(ks), v_new=np.concatenate(vs),
                        q=np.concatenate(qs)))
    w.max_blocks_per_seq = max(w.max_blocks_per_seq, _blocks(3000, bs))
    return w


def make_prefix_share(cold=False, *, dtype="bf16", hq=16, hkv=8, d=128, prefix=1000,
                      suffixes=(1, 5, 24, 1, 50, 16, 2, 9), seed=1010):
    """Eight requests with one shared prompt prefix (mlxcel user guide "연속
    배칭" §Paged KV 캐시와 프리픽스 공유: 8 requests over a 1024-token prefix;
    head counts of a 0.6B Qwen3, 16/8/128).

    Adopting (cold=False): slot 0 holds the prefix; before step 0 slots 1..7
    are acquired and adopt its `prefix` tokens by reference.  Cold (True): all
    eight slots prefill the same prefix themselves.  Then, identically:
    step 0 - slot s appends its own suffixes[s] rows (slot 0 decodes one);
    step 1 - every slot decodes one token; step 2 - slot 0 finishes
    (released) and slots 1..7 decode one more.  The prefix is 1000 tokens,
    not 1024, so that its last block is partial: every adopter's first write
    lands in a shared block (copy-on-write); at 1024 adopters would only
    append to fresh blocks.  Both variants draw the same values in the same
    order, so a slot's data are identical in the two."""
    n = len(suffixes)
    bs = 16
    draw = _Draw(seed, dtype)
    maxb = _blocks(prefix + max(suffixes) + 2, bs)
    num_blocks = math.ceil(1.2 * n * maxb)
    free_order = draw.rng.permutation(num_blocks).astype(np.int32)
    pk = draw.values((prefix, hkv, d))
    pv = draw.values((prefix, hkv, d))
    history = [(s, pk, pv) for s in range(n)] if cold else [(0, pk, pv)]
    steps = []
    plan = [list(enumerate(suffixes)), [(s, 1) for s in range(n)], [(s, 1) for s in range(1, n)]]
    for i, segs in enumerate(plan):
        t = sum(m for _, m in segs)
        k_new, v_new, q = draw.values((t, hkv, d)), draw.values((t, hkv, d)), draw.values((t, hq, d))
        ops = []
        if i == 0 and not cold:
            for s in range(1, n):
                ops += [("acquire", s), ("adopt", s, 0, prefix)]
        if i == 2:
            ops = [("release", 0)]
        steps.append(Step(ops=ops, segments=[Segment(s, m) for s, m in segs], k_new=k_new, v_new=v_new, q=q))
    name = "prefix-cold" if cold else "prefix"
    return Workload(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                    num_blocks=num_blocks, max_slots=n, max_blocks_per_seq=maxb, scale=1.0 / math.sqrt(d),
                    free_order=free_order, history=history, steps=steps,
                    description=f"{n} requests sharing a {prefix}-token prefix ({'cold' if cold else 'adopted'})")


def make_gather_ablation(prompt: int, batch: int = 4) -> Workload:
    """Decode step of `batch` sequences after a `prompt`-token prompt (mlxcel
    user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유 compares block-table
    and gather decode at batch 4 with 512- and 4096-token prompts).  The page
    names no model for that figure; the head layout is that of the 0.6B Qwen3
    its paragraph uses (16 query / 8 KV heads, head_dim 128), bf16."""
    seqs = [(i, prompt, 1) for i in range(batch)]
    return _build(f"gather-{prompt}", 1020 + prompt, "bf16", 16, 8, 128, 16, seqs,
                  description=f"decode, batch {batch}, {prompt}-token prompts, 16/8/128")


def make_workload(name: str) -> Workload:
    if name == "1":
        return _config1()
    if name == "1+1":
        return _config1(True)
    if name == "2":
        return _config2()
    if name == "3":
        return _config3()
    if name == "3v":
        return _config3v()
    if name == "3q":
        return _config3q()
    if name == "4a":
        return _config4(2048)
    if name == "4b":
        return _config4(512)
    if name == "5":
        return _config5()
    if name == "5q":
        return _config5q()
    if name.startswith("gather-"):
        return make_gather_ablation(int(name.split("-", 1)[1]))
    if name == "prefix":
        return make_prefix_share(False)
    if name == "prefix-cold":
        return make_prefix_share(True)
    raise ValueError(f"unknown config {name!r}")
