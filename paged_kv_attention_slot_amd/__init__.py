"""MI355X-native paged KV append and mixed-step paged attention.

The compute lives in libpagedkv.so (HIP kernels for gfx950 behind the C ABI
declared in include/pagedkv.h; a C++ block-pool allocator and step lowering).
This package is the Python binding over it.  There is no fallback: if the
library has not been built, the first call raises.
"""
from .binding import (  # noqa: F401
    BlockAllocator,
    KVPool,
    NoSpace,
    PagedKVError,
    PKV_BF16,
    PKV_F32,
    PKV_I8,
    copy_blocks,
    decode_partition_tokens,
    gather_kv,
    header_symbols,
    kv_append,
    lib,
    paged_attend,
    paged_attend_noalloc,
    pool_blocks_for_tokens,
    validate_step,
    workspace_bytes,
)
from .engine import PagedKVEngine, StepMeta  # noqa: F401
