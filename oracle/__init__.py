"""CPU oracle for the paged-KV mixed step.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the C-ABI library and its Python
binding) never calls it and shares no code with it.

What it computes, in plain numpy (fp64 for all floating point):
  * block_pool.BlockPool   - a block-pool allocator with stable sequence
    slots, per-slot block tables, atomic reservation and LIFO reuse, and the
    lowering of one step into slot_mapping / query_start / query_len /
    row_to_slot / context_lens / block_tables;
  * block_pool.BlockPool.adopt and the copy-on-write pairs of lower_step -
    shared prompt-prefix blocks with reference counts;
  * attention.append_reference - the KV append scatter (a byte copy);
  * attention.copy_blocks_reference - the copy-on-write block copy;
  * quant.quantize_rows / append_reference_q8 / paged_attention_q8 - the
    8-bit KV format (one float32 scale per (token, KV head) row), its append
    and attention over the values the codes stand for;
  * attention.paged_attention  - walks each block table in logical
    order, materialises that sequence's contiguous K/V, and computes causal
    softmax attention in fp64.

Sources: "Continuous batching: Qwen3.8-27B at 301 tok/s across five clients,
up to 1.97x llama.cpp" (lucebox blog) §Keeping track of each request,
§Paged KV and paged attention, §Chunked prefill is a slot phase, §Packing
unequal prompt chunks together, §Admission and step planning are different
decisions; mlxcel user guide "연속 배칭" §Paged KV 캐시와 프리픽스 공유.

Every function is pinned by the `-m "not gpu"` tests in tests/test_oracle_*.py
(brute force, closed forms, a library routine, invariants, the pages' worked
block-table example).  No function here is "parity unpinned".
"""
from .block_pool import BlockPool, NoSpace, pool_blocks_for_tokens  # noqa: F401
from .attention import (  # noqa: F401
    append_reference,
    copy_blocks_reference,
    decode_values,
    gather_sequence,
    paged_attention,
)
