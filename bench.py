#!/usr/bin/env python3
"""Benchmark of the paged-KV mixed step on one MI355X.

Default workload: 64 decode sequences (bf16, 32 query / 8 KV heads, head_dim
128, block size 16), context lengths lognormal with median 2048 clipped to
[16, 32768], slots drawn from 0..127, block tables fragmented by a seeded
random free order.  A step is the whole hot path: host reservation and
lowering of the step plan, one async copy of the metadata, kv_append of the
64 new tokens, and paged attention (decode kernel + split-context reduce).
The device half is one library call (pkv_mixed_step): the append kernel also
stages the step's metadata from pinned host memory, then attention runs.
Each timed step is a real decode step: every sequence grows by one token.

Prints one JSON line:
  value        = decode KV bytes read per step x steps / wall time  (GB/s)
  ms_per_step  = wall time / steps (host lowering included)
  step_gpu_ms  = each step's GPU work (append + attention) between HIP events
                 on the stream, p10 / p50 / p90, in as many steps run after
                 the timed ones (the timed steps record no events)
  host_ms_per_step = host time inside the step calls (lowering, the library
                 call, staging-ring waits)
  roofline     = the attention launch (decode kernel + partition reduce),
                 replayed 20 times on the last step's metadata after the timed
                 steps with the caches flushed before each call (a 1 GiB
                 read, outside the events), each call bracketed by HIP events
                 on its stream; algorithmic bytes per call / mean duration vs
                 8 TB/s (attend_ms_warm_avg: the same calls back to back)
  cpu_baseline = the CPU oracle on a bounded sample of the same step (with
                 the host's CPU model, core count and BLAS)
  extras       = after the headline, on the same GPU: config 4a's prompt
                 chunk alone (the chunk kernel's TFLOP/s against the bf16
                 peak: a one-call step holding only the chunk, minus its
                 append timed alone, both cold); the whole one-call step of
                 configs 2, 4a, 4b, 5 and 5 step 2, cold, against its
                 roofline time t_roof (the sum over its kernels of
                 max(bytes / 8 TB/s, flops / 2.5 PF)); the append kernel's
                 GB/s on three step sizes
  cpu_baseline_configs = the oracle on configs 1, 2, 5, 4b and 4a (1-thread
                 runs for 1 and 2)

    python bench.py [--steps K] [--warmup W] [--config 3] [--step N] [--no-cpu-baseline] [--no-extras]
    python bench.py --ablation gather|prefix     (one JSON line of ablation rows)
"""
from __future__ import annotations

import argparse
import gc
import ctypes
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
# Sources of the measured attention launch: a counter summary in
# profiles/traffic.json counts only while these files are unchanged.
TRAFFIC_SOURCES = ("decode_mfma.hip", "decode.hip", "pkv_device.h", "pkv_internal.h")
TRAFFIC_SOURCES_Q8 = ("decode_q8.hip", "decode.hip", "pkv_device.h", "pkv_internal.h")
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="3")
    ap.add_argument("--step", type=int, default=0,
                    help="mixed-step configs: time this step of the workload (earlier steps run once first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the chunk-kernel, mixed-step and append lines after the headline")
    ap.add_argument("--cpu-sample-rows", type=int, default=64)
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--sdpa-reference", action="store_true",
                    help="only time torch's flash-attention backend on contiguous dense shapes like the "
                         "prompt-chunk configs (context for the chunk kernel's TFLOP/s)")
    ap.add_argument("--ablation", choices=["gather", "prefix"], default=None,
                    help="gather: block-table decode vs gather-then-attend; prefix: adopted vs cold "
                         "shared-prefix step")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="how cold calls evict the caches: read 1 GiB (default) or fill it; a fill leaves dirty "
                         "lines whose write-back lands inside the next call's timing")
    ap.add_argument("--event-fence", choices=["none", "system"], default="none",
                    help="timing events: fence-free HIP events (default) or torch's events, whose record adds a "
                         "system-scope cache writeback to the timed interval")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 3 times (a plain copy of known size for counter scaling)")
    return ap.parse_args()


def decode_bytes(w, lens, elem):
    """Algorithmic bytes of the decode rows: K and V of every cached token
    once (an 8-bit pool: head_dim codes plus one float32 scale per token and
    KV head), plus Q in, fp32 O out and the block-table entries walked."""
    hkv, hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    row = d + 4 if getattr(w, "kv_quant", "") == "q8" else d * elem
    kv = sum(2 * L * hkv * row for L in lens)
    other = sum(hq * d * 2 + hq * d * 4 + 4 * (-(-L // 16)) for L in lens)
    return kv, kv + other


def chunk_flops(w, segments, lens):
    """Causal-visible flops of the multi-row segments: q.k and p.v over the
    keys each row sees, 2 flops per multiply-add each."""
    tot = 0
    for seg, L in zip(segments, lens):
        if seg.n > 1:
            visible = sum(L - seg.n + i + 1 for i in range(seg.n))
            tot += 4 * w.head_dim * w.num_q_heads * visible
    return tot


def multirow_bytes(w, segments, lens):
    """Algorithmic bytes of the multi-row segments: K and V of every token
    each segment sees, once, plus Q in and fp32 O out."""
    row = w.head_dim + 4 if getattr(w, "kv_quant", "") == "q8" else w.head_dim * w.elem_bytes
    tot = 0
    for seg, L in zip(segments, lens):
        if seg.n > 1:
            tot += 2 * L * w.num_kv_heads * row + seg.n * w.num_q_heads * w.head_dim * (2 + 4)
    return tot


def append_bytes(w, num_tokens):
    """Algorithmic bytes of kv_append: K and V rows read and written once,
    plus the 4-byte slot index per token (8-bit pools write codes and a
    4-byte scale per row)."""
    hkv, d = w.num_kv_heads, w.head_dim
    if getattr(w, "kv_quant", "") == "q8":
        return num_tokens * (2 * hkv * d * 2 + 2 * hkv * (d + 4) + 4)
    return num_tokens * (4 * hkv * d * w.elem_bytes + 4)


def step_roofline(w, segments, lens):
    """t_roof of one mixed step: the sum over its kernels of max(bytes / HBM
    peak, flops / bf16 peak) - the append, the decode rows (HBM), the
    multi-row segments (HBM or matrix, whichever binds).  Seconds."""
    t_app = append_bytes(w, sum(s.n for s in segments)) / (HBM_PEAK_GBS * 1e9)
    dec_lens = [L for s, L in zip(segments, lens) if s.n == 1]
    _, dec_alg = decode_bytes(w, dec_lens, w.elem_bytes)
    t_dec = dec_alg / (HBM_PEAK_GBS * 1e9)
    mr_b = multirow_bytes(w, segments, lens)
    mr_f = chunk_flops(w, segments, lens)
    t_mr = max(mr_b / (HBM_PEAK_GBS * 1e9), mr_f / (BF16_PEAK_TFLOPS * 1e12))
    return t_app + t_dec + t_mr, {"append_s": t_app, "decode_s": t_dec, "multirow_s": t_mr,
                                  "multirow_bound": "mfma" if mr_f / (BF16_PEAK_TFLOPS * 1e12) >
                                  mr_b / (HBM_PEAK_GBS * 1e9) else "hbm"}


FLUSH_KIND = "read"
EVENT_FENCE = "none"     # timing events: "none" (fence-free HIP events) or "system" (torch's default)
_HIP = None


class TimingEvent:
    """A HIP event made only for timing (hipEventDisableSystemFence): its
    record performs no system-scope cache writeback and invalidate, a cost
    that would otherwise land inside the interval it brackets and slow the
    work after it.  Same interface as torch.cuda.Event(enable_timing=True);
    read it only after a synchronize."""

    def __init__(self):
        global _HIP
        if _HIP is None:
            import torch
            torch.cuda.init()
            path = [ln.split()[-1] for ln in open("/proc/self/maps").read().splitlines()
                    if "libamdhip64" in ln][0]
            _HIP = ctypes.CDLL(path)       # the runtime torch loaded: the same stream handles
            _HIP.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            _HIP.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            _HIP.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = _HIP
        self.handle = ctypes.c_void_p()
        if _HIP.hipEventCreateWithFlags(ctypes.byref(self.handle), 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._hip.hipEventRecord(self.handle, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self.handle:
            self._hip.hipEventDestroy(self.handle)


def timing_event(torch):
    return TimingEvent() if EVENT_FENCE == "none" else torch.cuda.Event(enable_timing=True)




def evict_caches(flush, i):
    """Push the next call's inputs out of the L2s and the 256 MB Infinity
    Cache by streaming the 1 GiB buffer `flush` through them, on the current
    stream.  "read" sums it (one small result written); "write" fills it,
    which leaves dirty lines behind whose write-back then runs inside the
    next call's timing window."""
    if FLUSH_KIND == "write":
        flush.fill_(i & 0xFF)
    else:
        import torch
        flush.view(torch.int64).sum()


def _cold_times(torch, stream, fn, reps, flush):
    """Durations of fn() (seconds), each bracketed by HIP events on `stream`
    with the caches flushed before it (evict_caches, outside the events)."""
    ev = [(timing_event(torch), timing_event(torch)) for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        evict_caches(flush, i)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)


def mixed_step_stats(w, step, pk, torch, dev, reps, flush):
    """One workload step replayed through the one-call path: its GPU time
    cold (median of `reps`) against its roofline time."""
    from workloads.drive import apply_ops, make_engine, place_history, run_step, step_tensors
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    for i in range(step):
        run_step(eng, w, i, device=dev)
    st = w.steps[step]
    apply_ops(eng, st.ops)
    k_new, v_new, q = step_tensors(w, step, device=dev)
    prep = eng.prepare_fused([(s.slot, s.n) for s in st.segments], k_new, v_new, q, w.scale)
    for _ in range(3):
        eng.run_prepared(prep)
    stream = torch.cuda.current_stream()
    t = _cold_times(torch, stream, lambda: eng.run_prepared(prep), reps, flush)
    lens = [int(prep.meta.host["context_lens"][s.slot]) for s in st.segments]
    t_roof, parts = step_roofline(w, st.segments, lens)
    med = t[len(t) // 2]
    res = {"step_gpu_ms_cold": round(med * 1e3, 4), "t_roof_ms": round(t_roof * 1e3, 4),
           "frac": round(t_roof / med, 4), "bound_of_multirow": parts["multirow_bound"],
           "chunk_causal_gflop": round(chunk_flops(w, st.segments, lens) / 1e9, 2),
           "kv_mb": round((decode_bytes(w, [L for s, L in zip(st.segments, lens) if s.n == 1], w.elem_bytes)[0]
                           + multirow_bytes(w, st.segments, lens)) / 1e6, 1)}
    del eng, prep
    torch.cuda.empty_cache()
    return res


def chunk_kernel_stats(w, pk, torch, dev, reps, flush):
    """The chunk kernel on one config's multi-row segment alone: a one-call
    step holding only that segment (append + chunk kernels), minus the same
    append timed alone, both cold (medians).  Returns TFLOP/s over the
    causal-visible flops."""
    from workloads import Step, Workload  # noqa: F401  (types only)
    from workloads.drive import make_engine, place_history, to_device
    st = w.steps[0]
    seg_i = next(i for i, s in enumerate(st.segments) if s.n > 1)
    r0 = sum(s.n for s in st.segments[:seg_i])
    seg = st.segments[seg_i]
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    rows = slice(r0, r0 + seg.n)
    k_new = to_device(st.k_new[rows], w.dtype, dev)
    v_new = to_device(st.v_new[rows], w.dtype, dev)
    q = to_device(st.q[rows], w.dtype, dev)
    prep = eng.prepare_fused([(seg.slot, seg.n)], k_new, v_new, q, w.scale)
    for _ in range(3):
        eng.run_prepared(prep)
    stream = torch.cuda.current_stream()
    meta = prep.meta
    t_step = _cold_times(torch, stream, lambda: eng.run_prepared(prep), reps, flush)
    t_app = _cold_times(torch, stream, lambda: pk.kv_append(meta.slot_mapping, k_new, v_new, eng.pool), reps, flush)
    L = int(meta.host["context_lens"][seg.slot])
    fl = chunk_flops(w, [seg], [L])
    t_chunk = t_step[len(t_step) // 2] - t_app[len(t_app) // 2]
    del eng, prep
    torch.cuda.empty_cache()
    return {"kernel": "pkv chunk_kernel (+ its key-range merge when the segment is cut)",
            "workload": f"config {w.name}'s {seg.n}-row chunk at offset {L - seg.n} (context {L}), alone",
            "causal_gflop": round(fl / 1e9, 2), "ms": round(t_chunk * 1e3, 4),
            "step_ms_cold": round(t_step[len(t_step) // 2] * 1e3, 4),
            "append_ms_cold": round(t_app[len(t_app) // 2] * 1e3, 4),
            "tflops": round(fl / t_chunk / 1e12, 1),
            "frac_bf16_peak": round(fl / t_chunk / 1e12 / BF16_PEAK_TFLOPS, 4)}


def append_kernel_stats(w, step, pk, torch, dev, reps, flush):
    """kv_append alone on one step's new tokens (idempotent: the same rows to
    the same positions), cold median: algorithmic GB/s."""
    from workloads.drive import apply_ops, make_engine, place_history, run_step, step_tensors
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    for i in range(step):
        run_step(eng, w, i, device=dev)
    st = w.steps[step]
    apply_ops(eng, st.ops)
    k_new, v_new, _ = step_tensors(w, step, device=dev)
    meta = eng.lower([(s.slot, s.n) for s in st.segments])
    for _ in range(3):
        pk.kv_append(meta.slot_mapping, k_new, v_new, eng.pool)
    stream = torch.cuda.current_stream()
    t = _cold_times(torch, stream, lambda: pk.kv_append(meta.slot_mapping, k_new, v_new, eng.pool), reps, flush)
    med = t[len(t) // 2]
    nb = append_bytes(w, meta.total_q)
    del eng
    torch.cuda.empty_cache()
    return {"kernel": "pkv kv_append_kernel", "tokens": meta.total_q, "bytes": nb, "ms_cold": round(med * 1e3, 4),
            "gbs": round(nb / med / 1e9, 1), "frac_hbm_peak": round(nb / med / 1e9 / HBM_PEAK_GBS, 4)}


def run_mixed(args, w, pk, torch, dev):
    """Replay one mixed step - the one-call pkv_mixed_step (append, then
    attention) on fixed lowered metadata - and time it; for the chunk-bearing
    configs.  Steps before `args.step` run once, untimed."""
    from workloads.drive import apply_ops, make_engine, place_history, run_step, step_tensors
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    if not 0 <= args.step < len(w.steps):
        raise SystemExit(f"config {w.name} has steps 0..{len(w.steps) - 1}")
    for i in range(args.step):
        run_step(eng, w, i, device=dev)
    st = w.steps[args.step]
    apply_ops(eng, st.ops)
    k_new, v_new, q = step_tensors(w, args.step, device=dev)
    prep = eng.prepare_fused([(s.slot, s.n) for s in st.segments], k_new, v_new, q, w.scale)
    meta = prep.meta
    stream = torch.cuda.current_stream()
    ev = [(timing_event(torch), timing_event(torch)) for _ in range(args.steps)]
    # collect before the warm-up, not after it: a collection leaves the host
    # caches cold for the first timed step
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        eng.run_prepared(prep)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        eng.run_prepared(prep)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    att = sum(a.elapsed_time(b) for a, b in ev) / len(ev) / 1e3
    # the same step with the caches flushed before each call (evict_caches,
    # outside the events)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold_ev = [(timing_event(torch), timing_event(torch)) for _ in range(10)]
    for i, (a_, b_) in enumerate(cold_ev):
        evict_caches(flush, i)
        a_.record(stream)
        eng.run_prepared(prep)
        b_.record(stream)
    torch.cuda.synchronize()
    del flush
    att_cold = sorted(a_.elapsed_time(b_) for a_, b_ in cold_ev)[len(cold_ev) // 2] / 1e3
    lens = [int(meta.host["context_lens"][s.slot]) for s in st.segments]
    dec_lens = [L for s, L in zip(st.segments, lens) if s.n == 1]
    kv, _ = decode_bytes(w, dec_lens, w.elem_bytes)
    fl = chunk_flops(w, st.segments, lens)
    # K and V of every cached token of the multi-row segments, once
    row = w.head_dim + 4 if getattr(w, "kv_quant", "") == "q8" else w.head_dim * w.elem_bytes
    mr_kv = sum(2 * L * w.num_kv_heads * row for seg, L in zip(st.segments, lens) if seg.n > 1)
    t_roof, parts = step_roofline(w, st.segments, lens)
    name = w.name if args.step == 0 else f"{w.name} step {args.step + 1}"
    line = {"metric": f"mixed-step latency, config {name}", "value": round(wall / args.steps * 1e3, 4),
            "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall / args.steps * 1e3, 4), "step_gpu_ms_avg": round(att * 1e3, 4),
            "step_gpu_ms_cold_p50": round(att_cold * 1e3, 4),
            "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": f"config {name}: {w.description}", "decode_rows": len(dec_lens),
                       "chunk_rows": int(sum(s.n for s in st.segments if s.n > 1))},
            "decode_kv_bytes": kv, "chunk_causal_flops": fl, "multi_row_kv_bytes": mr_kv,
            "step_kv_gbs": round((kv + mr_kv) / att / 1e9, 1),
            "step_tflops_if_all_chunk": round(fl / att / 1e12, 2),
            # sum over the step's kernels of max(bytes / 8 TB/s, flops / 2.5 PF)
            "step_roofline": {"t_roof_ms": round(t_roof * 1e3, 4),
                              "frac_cold": round(t_roof / att_cold, 4), "frac_warm": round(t_roof / att, 4),
                              "parts_ms": {k: round(v * 1e3, 4) for k, v in parts.items() if k.endswith("_s")},
                              "multirow_bound": parts["multirow_bound"]}}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_step(w, args.step, 1 if fl > 50e9 else 3)
    return line


def cpu_baseline_step(w, step, repeats):
    """The oracle on one whole step of a workload (numpy fp64), best of
    `repeats`, setup excluded: step time and the same step's algorithmic rate."""
    from oracle.block_pool import BlockPool
    from oracle.step import append_kv, apply_ops, attend_step, copy_kv, place_history, poisoned_pool
    alloc = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
    pk_, pv_ = place_history(w, alloc, poisoned_pool(w), poisoned_pool(w))
    for i, st in enumerate(w.steps[:step + 1]):
        apply_ops(alloc, st.ops)
        meta = alloc.lower_step([(s.slot, s.n) for s in st.segments])
        pk_, pv_ = copy_kv(w, pk_, pv_, meta["copy_src"], meta["copy_dst"])
        pk_, pv_ = append_kv(w, pk_, pv_, meta["slot_mapping"], st.k_new, st.v_new)
        if i < step:
            continue
        dt = float("inf")
        for _ in range(repeats):
            t0 = time.perf_counter()
            attend_step(w, st, pk_, pv_, meta)
            dt = min(dt, time.perf_counter() - t0)
    st = w.steps[step]
    lens = [int(meta["context_lens"][s.slot]) for s in st.segments]
    kv = decode_bytes(w, [L for s, L in zip(st.segments, lens) if s.n == 1], w.elem_bytes)[0] + \
        multirow_bytes(w, st.segments, lens)
    host = _host_description()
    return {"value": round(dt * 1e3, 2), "unit": "ms per step", "cores": host["blas_threads"] or host["os_cpu_count"],
            "kind": "oracle", "sample": f"numpy fp64 oracle over the whole step, best of {repeats}",
            "kv_gbs": round(kv / dt / 1e9, 4), **host}


def _event_time(torch, stream, fn, reps):
    """Mean duration of fn() over reps calls, each bracketed by HIP events on
    `stream` (seconds)."""
    ev = [(timing_event(torch), timing_event(torch)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps / 1e3


def run_gather_ablation(args, pk, torch, dev):
    """mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유 reports the
    block-table decode kernel 1.9x (512-token prompts) to 10.9x (4096) faster
    than a gather path that rebuilds every visible window each step (batch
    4).  Here both paths run the same attention kernels; the gather path
    first copies each window into contiguous blocks (pkv_gather_kv) and then
    attends through identity tables, so the ratio prices the rebuild alone."""
    from workloads import make_workload
    from workloads.drive import make_engine, place_history, pool_torch_dtype, step_tensors
    rows = []
    stream = torch.cuda.current_stream()
    reps = max(args.steps, 5)
    for name in ("gather-512", "gather-4096", "3"):
        w = make_workload(name)
        eng = make_engine(pk.PagedKVEngine, w, device=dev)
        place_history(eng, w, device=dev)
        st = w.steps[0]
        k_new, v_new, q = step_tensors(w, 0, device=dev)
        meta = eng.lower([(s.slot, s.n) for s in st.segments])
        eng.append(meta, k_new, v_new)
        h = meta.host
        nbs = [-(-int(h["context_lens"][s]) // 16) for s in h["row_to_slot"]]
        start = torch.tensor([0] + list(itertools.accumulate(nbs))[:-1], dtype=torch.int32, device=dev)
        dst = pk.KVPool(sum(nbs), w.num_kv_heads, w.head_dim, pool_torch_dtype(w), device=dev, poison=False)
        dense = torch.zeros((w.max_slots, max(nbs)), dtype=torch.int32)
        off = 0
        for b, s in enumerate(h["row_to_slot"].tolist()):
            dense[s, :nbs[b]] = torch.arange(off, off + nbs[b], dtype=torch.int32)
            off += nbs[b]
        dense = dense.to(dev)
        out = torch.empty((meta.total_q, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        ws = eng.workspace_for(meta)

        def paged():
            eng.attend(meta, q, w.scale, out=out)

        def gather():
            pk.gather_kv(meta.row_to_slot, meta.context_lens, eng.d_block_tables, start, eng.pool, dst,
                         max_context_len=meta.max_context_len)

        def gather_attend():
            gather()
            pk.paged_attend(q, meta.row_to_slot, meta.query_start, meta.query_len, meta.context_lens, dense, dst,
                            w.scale, max_query_len=meta.max_query_len, max_context_len=meta.max_context_len,
                            out=out, workspace=ws)

        for fn in (paged, gather_attend):
            for _ in range(args.warmup):
                fn()
        torch.cuda.synchronize()
        t_paged = _event_time(torch, stream, paged, reps)
        t_gather = _event_time(torch, stream, gather, reps)
        t_both = _event_time(torch, stream, gather_attend, reps)
        moved = 2 * 2 * sum(nbs) * 16 * w.num_kv_heads * w.head_dim * w.elem_bytes   # K+V, read+write
        # a plain contiguous device copy of the same bytes, for scale
        csrc = torch.empty(moved // 2, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        t_copy = _event_time(torch, stream, lambda: cdst.copy_(csrc), reps)
        del csrc, cdst
        kv = sum(2 * int(h["context_lens"][s]) * w.num_kv_heads * w.head_dim * w.elem_bytes
                 for s in h["row_to_slot"])
        rows.append({"workload": f"{name}: {w.description}", "paged_attend_ms": round(t_paged * 1e3, 4),
                     "gather_ms": round(t_gather * 1e3, 4), "gather_then_attend_ms": round(t_both * 1e3, 4),
                     "ratio": round(t_both / t_paged, 3), "gather_gbs": round(moved / t_gather / 1e9, 1),
                     "plain_copy_gbs": round(moved / t_copy / 1e9, 1),
                     "paged_kv_gbs": round(kv / t_paged / 1e9, 1)})
        del eng, dst
        torch.cuda.empty_cache()
    return {"metric": "gather-then-attend / block-table attention time (ablation)", "unit": "x",
            "higher_is_better": False, "n_gpus": 1, "reps": reps, "warmup": args.warmup, "dtype": "bf16",
            "data": "synthetic", "rows": rows}


def run_prefix_ablation(args, pk, torch, dev):
    """mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유: eight
    requests over one prompt prefix, adopted by reference (seven copy-on-write
    block copies in the first step) or prefilled cold.  Times the first step
    (suffix chunks + decode) of each through the one-call path and reports
    the blocks each holds after it; also times the prefill that adoption
    skips (the seven adopters' prefix rows appended and attended causally in
    one step)."""
    from workloads import make_custom, make_workload
    from workloads.drive import apply_ops, make_engine, place_history, step_tensors
    rows = []
    stream = torch.cuda.current_stream()
    reps = max(args.steps, 5)

    def timed_step0(w):
        eng = make_engine(pk.PagedKVEngine, w, device=dev)
        place_history(eng, w, device=dev)         # acquires the slots; appends any history
        st = w.steps[0]
        apply_ops(eng, st.ops)
        k_new, v_new, q = step_tensors(w, 0, device=dev)
        prep = eng.prepare_fused([(s.slot, s.n) for s in st.segments], k_new, v_new, q, w.scale)
        for _ in range(args.warmup):
            eng.run_prepared(prep)
        t = _event_time(torch, stream, lambda: eng.run_prepared(prep), reps)
        return t, prep.meta.num_copies, w.num_blocks - eng.alloc.free_blocks()

    for name in ("prefix", "prefix-cold"):
        w = make_workload(name)
        t, nc, used = timed_step0(w)
        rows.append({"workload": f"{name}: {w.description}", "step0_ms": round(t * 1e3, 4),
                     "copies_in_step0": nc, "blocks_held": used,
                     "kv_bytes_held": used * 2 * 16 * w.num_kv_heads * w.head_dim * w.elem_bytes})
        torch.cuda.empty_cache()
    w = make_workload("prefix")
    pre = len(w.history[0][1])
    wp = make_custom([(s, 0, pre) for s in range(1, w.max_slots)], dtype=w.dtype, hq=w.num_q_heads,
                     hkv=w.num_kv_heads, d=w.head_dim, seed=31)
    t, _, _ = timed_step0(wp)
    rows.append({"workload": f"prefill skipped by adoption: {w.max_slots - 1} x {pre} prefix rows, one step",
                 "step0_ms": round(t * 1e3, 4)})
    return {"metric": "shared-prefix adoption vs cold prefill (ablation)", "unit": "ms",
            "higher_is_better": False, "n_gpus": 1, "reps": reps, "warmup": args.warmup, "dtype": "bf16",
            "data": "synthetic", "rows": rows}


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_attention_slot_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, sample_rows, repeats):
    """Time the oracle (numpy fp64) on the first `sample_rows` decode rows of
    the step: block-table walk + fp64 attention, best of `repeats`.  Setup is
    not timed."""
    from oracle.block_pool import BlockPool
    from oracle.step import append_kv, attend_step, place_history, poisoned_pool
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    alloc = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
    pk_, pv_ = place_history(w, alloc, poisoned_pool(w), poisoned_pool(w))
    st = w.steps[0]
    meta = alloc.lower_step([(s.slot, s.n) for s in st.segments])
    pk_, pv_ = append_kv(w, pk_, pv_, meta["slot_mapping"], st.k_new, st.v_new)
    rows = min(sample_rows, len(st.segments))
    sample = dict(meta, row_to_slot=meta["row_to_slot"][:rows], query_start=meta["query_start"][:rows],
                  query_len=meta["query_len"][:rows])
    dt = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        attend_step(w, st, pk_, pv_, sample)
        dt = min(dt, time.perf_counter() - t0)
    lens = [int(meta["context_lens"][s]) for s in meta["row_to_slot"][:rows]]
    kv, _ = decode_bytes(w, lens, w.elem_bytes)
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 oracle over the first {rows} of {len(st.segments)} decode rows of one step "
                      f"({sum(lens)} cached tokens), best of {repeats}: {dt:.2f} s"}


def _host_description():
    """CPU model, logical CPU count and the BLAS numpy uses (with its threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas": blas, "blas_threads": threads}


def cpu_baseline_configs():
    """The oracle (numpy fp64: block-table walk + attention) on the mixed-step
    configs, timed over attention only (setup excluded): best of 3 for the
    small configs 1, 2 and 5, one run for 4a and 4b; configs 1 and 2 also
    with BLAS held to one thread.  Effective rates use the same algorithmic
    bytes and flops as the GPU lines."""
    from threadpoolctl import threadpool_limits
    from oracle.block_pool import BlockPool
    from oracle.step import append_kv, attend_step, place_history, poisoned_pool
    from workloads import make_workload
    rows = {}

    def prepared(name):
        w = make_workload(name)
        alloc = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
        pk_, pv_ = place_history(w, alloc, poisoned_pool(w), poisoned_pool(w))
        st = w.steps[0]
        meta = alloc.lower_step([(s.slot, s.n) for s in st.segments])
        pk_, pv_ = append_kv(w, pk_, pv_, meta["slot_mapping"], st.k_new, st.v_new)
        return w, st, pk_, pv_, meta

    for name, repeats, one_thread in (("1", 3, True), ("2", 3, True), ("5", 3, False), ("4b", 1, False),
                                      ("4a", 1, False)):
        w, st, pk_, pv_, meta = prepared(name)
        lens = [int(meta["context_lens"][s.slot]) for s in st.segments]
        kv = decode_bytes(w, [L for s, L in zip(st.segments, lens) if s.n == 1], w.elem_bytes)[0] + \
            multirow_bytes(w, st.segments, lens)
        fl = chunk_flops(w, st.segments, lens)

        def best(n):
            dt = float("inf")
            for _ in range(n):
                t0 = time.perf_counter()
                attend_step(w, st, pk_, pv_, meta)
                dt = min(dt, time.perf_counter() - t0)
            return dt
        dt = best(repeats)
        row = {"seconds": round(dt, 4), "repeats": repeats, "kv_gbs": round(kv / dt / 1e9, 4),
               "gflops_causal": round(fl / dt / 1e9, 2) if fl else None}
        if one_thread:
            with threadpool_limits(limits=1):
                dt1 = best(repeats)
            row["seconds_1_thread"] = round(dt1, 4)
        rows[f"config {name}"] = row
    return {"kind": "oracle", **_host_description(), "per_config": rows}


def run_extras(pk, torch, dev, args):
    """The second target and the mixed steps, on the same run as the
    headline: config 4a's chunk kernel alone (TFLOP/s against bf16 peak),
    each chunk-bearing config's whole one-call step against its roofline,
    and the append kernel's rate."""
    from workloads import make_workload
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    reps = 10
    out = {"chunk_kernel": chunk_kernel_stats(make_workload("4a"), pk, torch, dev, reps, flush)}
    steps = {}
    for name, step in (("2", 0), ("4a", 0), ("4b", 0), ("5", 0), ("5", 1)):
        label = f"config {name}" + (f" step {step + 1}" if step else "")
        steps[label] = mixed_step_stats(make_workload(name), step, pk, torch, dev, reps, flush)
    out["mixed_steps"] = steps
    out["append_kernel"] = {
        "config 5 step 2": append_kernel_stats(make_workload("5"), 1, pk, torch, dev, reps, flush),
        "config 4a": append_kernel_stats(make_workload("4a"), 0, pk, torch, dev, reps, flush),
        "config 3": append_kernel_stats(make_workload("3"), 0, pk, torch, dev, reps, flush)}
    del flush
    torch.cuda.empty_cache()
    return out


def sdpa_reference(torch, dev, reps=20):
    """torch's scaled_dot_product_attention, flash backend only (no fallback),
    on contiguous bf16 Q, K, V with every query head's K/V expanded: dense
    shapes like the prompt-chunk configs, and two causal ones.  Flops count
    the visible pairs (4 D per pair per head); median of `reps` calls, each
    bracketed by timing-only HIP events."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    shapes = [("dense 2048 x 8192, D 64 (config 4a's rows and keys)", 32, 2048, 8192, 64, False),
              ("dense 512 x 8192, D 64 (config 4b)", 32, 512, 8192, 64, False),
              ("dense 512 x 1536, D 128 (config 2)", 32, 512, 1536, 128, False),
              ("causal 8192 x 8192, D 64", 32, 8192, 8192, 64, True),
              ("causal 3000 x 3000, D 128, 40 heads (config 5 step 2's prompt)", 40, 3000, 3000, 128, True)]
    stream = torch.cuda.current_stream()
    out = {"kind": "torch SDPBackend.FLASH_ATTENTION on contiguous K/V (not paged)", "torch": torch.__version__}
    for name, hq, lq, lk, d, causal in shapes:
        g = torch.Generator(device=dev).manual_seed(1)
        q, k, v = (torch.randn(1, hq, n, d, device=dev, dtype=torch.bfloat16, generator=g) for n in (lq, lk, lk))
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(3):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
            ev = [(timing_event(torch), timing_event(torch)) for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
                b.record(stream)
            torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2] / 1e3
        flops = 4 * d * hq * (lq * (lq + 1) // 2 if causal else lq * lk)
        out[name] = {"ms": round(t * 1e3, 4), "tflops": round(flops / t / 1e12, 1),
                     "frac_bf16_peak": round(flops / t / (BF16_PEAK_TFLOPS * 1e12), 4)}
    return out


def main():
    global FLUSH_KIND, EVENT_FENCE
    args = parse_args()
    FLUSH_KIND = args.flush
    EVENT_FENCE = args.event_fence
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              "mode", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda:0")     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 2, "launches": 3}))
        return
    import paged_kv_attention_slot_amd as pk
    from workloads import make_workload
    from workloads.drive import make_engine, place_history, step_tensors

    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.sdpa_reference:
        print(json.dumps(sdpa_reference(torch, dev)), flush=True)
        return
    if args.ablation == "gather":
        print(json.dumps(run_gather_ablation(args, pk, torch, dev)), flush=True)
        return
    if args.ablation == "prefix":
        print(json.dumps(run_prefix_ablation(args, pk, torch, dev)), flush=True)
        return
    w = make_workload(args.config)
    st = w.steps[0]
    if any(s.n != 1 for s in st.segments) or args.step:
        print(json.dumps(run_mixed(args, w, pk, torch, dev)), flush=True)
        return
    # warmup, the timed steps, then as many again with per-step events
    total_steps = args.warmup + 2 * args.steps
    w.max_blocks_per_seq += -(-total_steps // 16) + 1
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    k_new, v_new, q = step_tensors(w, 0, device=dev)
    entries = [(s.slot, s.n) for s in st.segments]
    # rolling decode headroom for every step of the run, reserved up front
    for slot, hk, _ in w.history:
        eng.reserve(slot, len(hk) + total_steps)
    out = torch.empty((len(entries), w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    kv_total, lens_hist = 0, []

    def one_step():
        _, meta = eng.fused_step(entries, k_new, v_new, q, w.scale, out=out)
        return meta

    # No collector pauses in the warm-up or the timed region.  The collection
    # runs before the warm-up: right before the timed steps it left the host
    # caches cold, and the first timed step's host work took ~190 us instead
    # of ~25 us.
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    metas = []
    host = 0.0
    t0 = time.perf_counter()
    for i in range(args.steps):
        h0 = time.perf_counter()
        metas.append(one_step())
        host += time.perf_counter() - h0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Each step's GPU work (append + attention) bracketed by HIP events, in
    # as many further steps after the timed ones: an event record costs the
    # stream several microseconds, so the timed steps carry none.
    step_ev = [(timing_event(torch), timing_event(torch))
               for _ in range(args.steps)]
    for i in range(args.steps):
        step_ev[i][0].record(stream)
        one_step()
        step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    step_gpu = sorted(a_.elapsed_time(b_) for a_, b_ in step_ev)
    for meta in metas:
        lens = meta.host["context_lens"][meta.host["row_to_slot"]].tolist()
        kv, alg = decode_bytes(w, lens, w.elem_bytes)
        kv_total += kv
        lens_hist.append(sum(lens))
    # Roofline of the attention launch (decode kernel + partition reduce):
    # replay it on the last step's metadata, each call bracketed by HIP events
    # recorded on the stream the kernels run on.  Cold: before each call a
    # 1 GiB read (4x the 256 MB Infinity Cache) evicts the caches, outside
    # the events; the roofline uses the cold calls.  Warm: back to back.
    last = metas[-1]
    lens = last.host["context_lens"][last.host["row_to_slot"]].tolist()
    _, alg_attend = decode_bytes(w, lens, w.elem_bytes)
    reps = 20
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def replay(cold):
        ev = [(timing_event(torch), timing_event(torch)) for _ in range(reps)]
        for i, (a_, b_) in enumerate(ev):
            if cold:
                evict_caches(flush, i)
            a_.record(stream)
            eng.attend(last, q, w.scale, out=out)
            b_.record(stream)
        torch.cuda.synchronize()
        return sorted(a_.elapsed_time(b_) for a_, b_ in ev)

    warm_ms = replay(False)
    cold_ms = replay(True)
    del flush
    attend_avg_s = sum(cold_ms) / reps / 1e3
    achieved = alg_attend / attend_avg_s / 1e9

    def pct(v, f):
        return round(v[min(len(v) - 1, int(f * len(v)))], 4)
    q8 = getattr(w, "kv_quant", "") == "q8"
    src = source_hash(*(TRAFFIC_SOURCES_Q8 if q8 else TRAFFIC_SOURCES))
    traffic = measured_traffic(f"decode_config{w.name}", src)
    line = {
        "metric": "paged-attn decode KV GB/s (% HBM peak); mixed-step latency at 64 seqs",
        "value": round(kv_total / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 KV (bf16 Q, fp32 accumulate)" if q8 else ("bf16" if w.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": f"config {w.name}: {w.description}", "decode_rows": len(entries),
                   "heads_q_kv": [w.num_q_heads, w.num_kv_heads], "head_dim": w.head_dim, "block_size": 16,
                   "cached_tokens_per_step": int(sum(lens_hist) / len(lens_hist)),
                   "decode_partition_tokens": pk.decode_partition_tokens()},
        "pct_hbm_peak": round(100.0 * kv_total / wall / 1e9 / HBM_PEAK_GBS, 2),
        "step_gpu_ms": {"p10": pct(step_gpu, 0.1), "p50": pct(step_gpu, 0.5), "p90": pct(step_gpu, 0.9)},
        "host_ms_per_step": round(host / args.steps * 1e3, 4),
        "attend_ms_avg": round(attend_avg_s * 1e3, 4),
        "attend_ms_cold": {"p10": pct(cold_ms, 0.1), "p50": pct(cold_ms, 0.5), "p90": pct(cold_ms, 0.9)},
        "attend_ms_warm_avg": round(sum(warm_ms) / reps, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("pkv decode_q8_kernel" if q8 else "pkv decode_mfma_kernel")
                     + " + reduce_kernel (one paged_attend launch)",
                     "cold_flush": f"1 GiB {FLUSH_KIND} before each timed call",
                     "timing_events": "HIP events without the system-scope fence" if EVENT_FENCE == "none"
                     else "torch events (system-scope fence on record)"},
    }
    if not args.no_extras:
        line["extras"] = run_extras(pk, torch, dev, args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows, args.cpu_repeats)
        line["cpu_baseline"].update(_host_description())
        if not args.no_extras:
            line["cpu_baseline_configs"] = cpu_baseline_configs()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
