"""Paged KV append and paged attention, fp64 (oracle side, test infrastructure).

"Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog):
  * §Paged KV and paged attention: attention reads a sequence's cached
    history by following its block table, visiting blocks in logical token
    order, over a shared pool, with no gather or relocation of the cache
    (here: the oracle does materialise the contiguous history - it is the
    plain definition the kernels must agree with);
  * §Chunked prefill is a slot phase: each selected chunk appends directly to
    its slot's paged KV;
  * §Packing unequal prompt chunks together: prompt chunks and decode rows
    share one packed token axis; per-query causal positions plus block-table
    metadata let both kinds of rows attend in one pass.

Pool layout (the pages leave it to the backend): K and V are separate arrays,
each [num_blocks][num_kv_heads][block_size][head_dim].  bf16 values are held
as their uint16 bit patterns; fp32 as float32.

Readings where the pages are silent:
  * segment b has n = query_len[b] rows; its slot s = row_to_slot[b] holds
    L = context_lens[s] tokens (this step's included); row i sits at position
    L - n + i and sees keys 0 .. L - n + i (a decode row, n = 1, sees all L);
  * query head h uses KV head h // (Hq / Hkv) (consecutive heads share);
  * plain softmax with the running maximum subtracted; no sliding window, no
    soft-cap, no sinks.
"""
from __future__ import annotations

import numpy as np


def decode_values(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element storage -> fp64 (exact).  bf16 is the high half of an fp32."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f64":                  # values already decoded (a dequantized pool)
        return np.asarray(raw, dtype=np.float64)
    raise ValueError(dtype)


def block_and_offset(slot_index: int, block_size: int):
    """A flat pool token slot -> (physical block, position inside the block)."""
    return slot_index // block_size, slot_index % block_size


def append_reference(pool_k, pool_v, slot_mapping, k_new, v_new, block_size):
    """Scatter token t's K/V [Hkv][D] into pool position slot_mapping[t].
    Returns new arrays; a pure copy of element bits, no conversion."""
    k = pool_k.copy()
    v = pool_v.copy()
    sm = np.asarray(slot_mapping, dtype=np.int64)
    if sm.size:
        blk, off = block_and_offset(sm, block_size)
        k[blk, :, off, :] = k_new
        v[blk, :, off, :] = v_new
    return k, v


def copy_blocks_reference(pool_k, pool_v, copy_src, copy_dst):
    """Copy-on-write (mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스
    공유): block copy_dst[c] receives all of block copy_src[c], K and V, every
    head and position.  Returns new arrays; a pure copy of element bits."""
    k = pool_k.copy()
    v = pool_v.copy()
    for src, dst in zip(np.asarray(copy_src).tolist(), np.asarray(copy_dst).tolist()):
        k[dst] = pool_k[src]
        v[dst] = pool_v[src]
    return k, v


def gather_sequence(pool, block_table, num_tokens, block_size):
    """Visit the first ceil(L / block_size) entries of the block table in
    logical order and return the sequence's first L tokens as [L][Hkv][D]."""
    nb = -(-num_tokens // block_size)
    tiles = [pool[int(block_table[j])] for j in range(nb)]          # each [Hkv][BS][D]
    if not tiles:
        return pool[:0, :, 0, :].copy().reshape(0, pool.shape[1], pool.shape[3])
    seq = np.concatenate(tiles, axis=1)                              # [Hkv][nb*BS][D]
    return np.ascontiguousarray(seq[:, :num_tokens, :].transpose(1, 0, 2))


def kv_head_for(h: int, group: int) -> int:
    """Query head h reads KV head h // G."""
    return h // group


def visible(positions: np.ndarray, num_keys: int) -> np.ndarray:
    """mask[i, j] is True when key j is visible to the row at positions[i]."""
    return np.arange(num_keys)[None, :] <= positions[:, None]


def attend_rows(q, k, v, scale, positions):
    """q [n][Hq][D], k/v [L][Hkv][D] (fp64); softmax attention of each row over
    its visible keys.  Returns [n][Hq][D] fp64."""
    n, hq, d = q.shape
    num_keys, hkv, _ = k.shape
    group = hq // hkv
    mask = visible(positions, num_keys)
    out = np.empty((n, hq, d), dtype=np.float64)
    for h in range(hq):
        g = kv_head_for(h, group)
        s = scale * (q[:, h, :] @ k[:, g, :].T)                      # [n][L]
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)                                            # masked keys -> 0
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def paged_attention(q_raw, pool_k, pool_v, dtype, block_size, block_tables, context_lens,
                    row_to_slot, query_start, query_len, scale, num_kv_heads=None, kv_dtype=None):
    """Mixed-step paged attention over a packed batch.  Returns fp64
    [total_q][Hq][D]; rows not covered by any segment stay NaN.  `kv_dtype`
    (default `dtype`) is the pools' element type ("f64" for pools already
    dequantized)."""
    q = decode_values(q_raw, dtype)
    kv_dtype = kv_dtype or dtype
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for b in range(len(row_to_slot)):
        s = int(row_to_slot[b])
        L = int(context_lens[s])
        n = int(query_len[b])
        r0 = int(query_start[b])
        k = decode_values(gather_sequence(pool_k, block_tables[s], L, block_size), kv_dtype)
        v = decode_values(gather_sequence(pool_v, block_tables[s], L, block_size), kv_dtype)
        positions = L - n + np.arange(n)
        out[r0:r0 + n] = attend_rows(q[r0:r0 + n], k, v, float(scale), positions)
    return out
