"""8-bit KV rows with one float32 scale each (oracle side, test infrastructure).

"Continuous batching: Qwen3.8-27B at 301 tok/s ..." (lucebox blog),
§Qwen3.8-27B DFlash2 on the R9700 (vs llama.cpp) and its launch example: the
server keeps its KV cache in an 8-bit format (Q8_0).  The pages name the
format without defining it, so this repository defines its own, written out
here as the definition the kernels must reproduce:

  * a row is the head_dim values of one (token, KV head), given as bf16;
  * amax = the largest |x| of the row (x read as float32, exact);
  * amax == 0: every code is 0 and the scale is 0;
  * otherwise inv = 127 / amax and scale = amax / 127, each a correctly
    rounded float32 division; code = round-half-to-even(x * inv), the
    product first rounded to float32, then clamped to [-127, 127];
  * a code stands for the value code * scale (exact in fp64).

Rounding decides integers here, so the precision is part of the definition:
IEEE float32 with round-to-nearest-even at every step, which numpy's float32
arithmetic and the GPU's both follow.  Inputs are finite.

Pool layout: codes int8 [num_blocks][num_kv_heads][block_size][head_dim]
(the bf16 pool's layout with one byte per element); scales float32
[num_blocks][num_kv_heads][block_size].
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, block_and_offset, decode_values, gather_sequence


def quantize_rows(x_bits: np.ndarray):
    """bf16 bit patterns [..., D] -> (int8 codes [..., D], float32 scales [...])."""
    x = decode_values(x_bits, "bf16").astype(np.float32)        # exact
    amax = np.max(np.abs(x), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = (np.float32(127) / safe).astype(np.float32)
    scale = np.where(nz, safe / np.float32(127), np.float32(0)).astype(np.float32)
    prod = (x * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127)
    codes = np.where(nz[..., None], codes, 0)
    return codes.astype(np.int8), scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The values the codes stand for, fp64 (code * scale, exact)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def append_reference_q8(codes_k, scale_k, codes_v, scale_v, slot_mapping, k_new_bits, v_new_bits, block_size):
    """Quantize token t's K/V rows [Hkv][D] and store codes and scales at pool
    position slot_mapping[t].  Returns new arrays."""
    ck, sk, cv, sv = codes_k.copy(), scale_k.copy(), codes_v.copy(), scale_v.copy()
    sm = np.asarray(slot_mapping, dtype=np.int64)
    if sm.size:
        blk, off = block_and_offset(sm, block_size)
        qk, qks = quantize_rows(k_new_bits)
        qv, qvs = quantize_rows(v_new_bits)
        ck[blk, :, off, :] = qk
        sk[blk, :, off] = qks
        cv[blk, :, off, :] = qv
        sv[blk, :, off] = qvs
    return ck, sk, cv, sv


def gather_dequantized(codes, scales, block_table, num_tokens, block_size):
    """A sequence's first L tokens as fp64 [L][Hkv][D]: its codes and scales
    walked through the block table in logical order, then dequantized."""
    c = gather_sequence(codes, block_table, num_tokens, block_size)
    s = gather_sequence(scales[..., None], block_table, num_tokens, block_size)[..., 0]
    return dequantize(c, s)


def paged_attention_q8(q_raw, pool_k, pool_v, block_size, block_tables, context_lens, row_to_slot,
                       query_start, query_len, scale):
    """Mixed-step paged attention over 8-bit pools (pool_k = (codes, scales),
    likewise pool_v): the bf16 queries attend, in fp64, over the values the
    codes stand for.  Returns fp64 [total_q][Hq][D]; uncovered rows NaN."""
    q = decode_values(q_raw, "bf16")
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for b in range(len(row_to_slot)):
        s = int(row_to_slot[b])
        L = int(context_lens[s])
        n = int(query_len[b])
        r0 = int(query_start[b])
        k = gather_dequantized(pool_k[0], pool_k[1], block_tables[s], L, block_size)
        v = gather_dequantized(pool_v[0], pool_v[1], block_tables[s], L, block_size)
        positions = L - n + np.arange(n)
        out[r0:r0 + n] = attend_rows(q[r0:r0 + n], k, v, float(scale), positions)
    return out
