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
  roofline     = the attention launch (decode kernel + partition reduce),
                 replayed 20 times on the last step's metadata after the timed
                 steps, each call bracketed by HIP events on its stream;
                 algorithmic bytes per call / mean duration vs 8 TB/s
  cpu_baseline = the CPU oracle on a bounded sample of the same step

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
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
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=64)
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 3 times (a plain copy of known size for counter scaling)")
    return ap.parse_args()


def decode_bytes(w, lens, elem):
    """Algorithmic bytes of the decode rows: K and V of every cached token
    once, plus Q in, fp32 O out and the block-table entries walked."""
    hkv, hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    kv = sum(2 * L * hkv * d * elem for L in lens)
    other = sum(hq * d * elem + hq * d * 4 + 4 * (-(-L // 16)) for L in lens)
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


def run_mixed(args, w, pk, torch, dev):
    """Replay one mixed step - the one-call pkv_mixed_step (append, then
    attention) on fixed lowered metadata - and time it; for the chunk-bearing
    configs."""
    from workloads.drive import make_engine, place_history, step_tensors
    eng = make_engine(pk.PagedKVEngine, w, device=dev)
    place_history(eng, w, device=dev)
    st = w.steps[0]
    k_new, v_new, q = step_tensors(w, 0, device=dev)
    prep = eng.prepare_fused([(s.slot, s.n) for s in st.segments], k_new, v_new, q, w.scale)
    meta = prep.meta
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for _ in range(args.warmup):
        eng.run_prepared(prep)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        eng.run_prepared(prep)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    att = sum(a.elapsed_time(b) for a, b in ev) / len(ev) / 1e3
    lens = [int(meta.host["context_lens"][s.slot]) for s in st.segments]
    dec_lens = [L for s, L in zip(st.segments, lens) if s.n == 1]
    kv, alg = decode_bytes(w, dec_lens, w.elem_bytes)
    fl = chunk_flops(w, st.segments, lens)
    # K and V of every cached token of the multi-row segments, once
    mr_kv = sum(2 * L * w.num_kv_heads * w.head_dim * w.elem_bytes for seg, L in zip(st.segments, lens) if seg.n > 1)
    return {"metric": f"mixed-step latency, config {w.name}", "value": round(wall / args.steps * 1e3, 4),
            "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall / args.steps * 1e3, 4), "step_gpu_ms_avg": round(att * 1e3, 4),
            "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": f"config {w.name}: {w.description}", "decode_rows": len(dec_lens),
                       "chunk_rows": int(sum(s.n for s in st.segments if s.n > 1))},
            "decode_kv_bytes": kv, "chunk_causal_flops": fl, "multi_row_kv_bytes": mr_kv,
            "step_kv_gbs": round((kv + mr_kv) / att / 1e9, 1),
            "step_tflops_if_all_chunk": round(fl / att / 1e12, 2),
            "roofline_step_ms": round((alg / HBM_PEAK_GBS / 1e9 + fl / BF16_PEAK_TFLOPS / 1e12) * 1e3, 4)}


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
    import numpy as np
    from oracle.attention import paged_attention
    from oracle.step import place_history, poisoned_pool
    from oracle.block_pool import BlockPool
    from oracle.attention import append_reference
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    alloc = BlockPool(w.num_blocks, w.block_size, w.max_slots, w.max_blocks_per_seq, w.free_order)
    pk_, pv_ = place_history(w, alloc, poisoned_pool(w), poisoned_pool(w))
    st = w.steps[0]
    meta = alloc.lower_step([(s.slot, s.n) for s in st.segments])
    pk_, pv_ = append_reference(pk_, pv_, meta["slot_mapping"], st.k_new, st.v_new, w.block_size)
    rows = min(sample_rows, len(st.segments))
    dt = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        paged_attention(st.q[:rows], pk_, pv_, w.dtype, w.block_size, meta["block_tables"], meta["context_lens"],
                        meta["row_to_slot"][:rows], meta["query_start"][:rows], meta["query_len"][:rows], w.scale)
        dt = min(dt, time.perf_counter() - t0)
    lens = [int(meta["context_lens"][s]) for s in meta["row_to_slot"][:rows]]
    kv, _ = decode_bytes(w, lens, w.elem_bytes)
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 oracle over the first {rows} of {len(st.segments)} decode rows of one step "
                      f"({sum(lens)} cached tokens), best of {repeats}: {dt:.2f} s"}


def main():
    args = parse_args()
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
    w = make_workload(args.config)
    st = w.steps[0]
    if any(s.n != 1 for s in st.segments):
        print(json.dumps(run_mixed(args, w, pk, torch, dev)), flush=True)
        return
    total_steps = args.warmup + args.steps
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

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    metas = []
    gc.collect()
    gc.disable()            # no collector pauses inside the timed region
    t0 = time.perf_counter()
    for i in range(args.steps):
        metas.append(one_step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    for meta in metas:
        lens = meta.host["context_lens"][meta.host["row_to_slot"]].tolist()
        kv, alg = decode_bytes(w, lens, w.elem_bytes)
        kv_total += kv
        lens_hist.append(sum(lens))
    # Roofline of the attention launch (decode kernel + partition reduce):
    # replay it on the last step's metadata, each call bracketed by HIP events
    # recorded on the stream the kernels run on.
    last = metas[-1]
    lens = last.host["context_lens"][last.host["row_to_slot"]].tolist()
    _, alg_attend = decode_bytes(w, lens, w.elem_bytes)
    reps = 20
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in ev:
        a_.record(stream)
        eng.attend(last, q, w.scale, out=out)
        b_.record(stream)
    torch.cuda.synchronize()
    attend_avg_s = sum(a_.elapsed_time(b_) for a_, b_ in ev) / reps / 1e3
    achieved = alg_attend / attend_avg_s / 1e9
    src = source_hash(*TRAFFIC_SOURCES)
    traffic = measured_traffic("decode_config3", src)
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
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"config {w.name}: {w.description}", "decode_rows": len(entries),
                   "heads_q_kv": [w.num_q_heads, w.num_kv_heads], "head_dim": w.head_dim, "block_size": 16,
                   "cached_tokens_per_step": int(sum(lens_hist) / len(lens_hist)),
                   "decode_partition_tokens": pk.decode_partition_tokens()},
        "pct_hbm_peak": round(100.0 * kv_total / wall / 1e9 / HBM_PEAK_GBS, 2),
        "attend_ms_avg": round(attend_avg_s * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "pkv decode_kernel + reduce_kernel (one paged_attend launch)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows, args.cpu_repeats)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
