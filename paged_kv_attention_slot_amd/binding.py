"""ctypes binding for libpagedkv.so: argument marshalling only.

Every computation runs in the library (HIP kernels for append and attention,
C++ for the block-pool allocator and the step lowering).  PyTorch supplies
device memory and the current stream; nothing else from it is used here.
Importing this module does not load the library; the first call does, and
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

# PKV_LIBRARY may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libpagedkv.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pagedkv.h")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_NO_SPACE = -3
PKV_ERR_WORKSPACE = -4
PKV_ERR_HIP = -5
PKV_ERR_STATE = -6
PKV_F32 = 0
PKV_BF16 = 1
PKV_I8 = 2

_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)


class PoolDesc(ctypes.Structure):
    _fields_ = [("k", _p), ("v", _p), ("num_blocks", _i32), ("block_size", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("dtype", _i32),
                ("scales", _p)]


class StepDesc(ctypes.Structure):
    _fields_ = [("host_meta", _p), ("dev_meta", _p), ("meta_len", _i32),
                ("slot_mapping_off", _i32), ("query_start_off", _i32), ("query_len_off", _i32),
                ("row_to_slot_off", _i32), ("context_lens_off", _i32),
                ("num_tokens", _i32), ("num_segments", _i32), ("num_slots", _i32), ("total_q", _i32),
                ("num_q_heads", _i32), ("max_blocks_per_seq", _i32), ("max_query_len", _i32),
                ("max_context_len", _i32), ("k_new", _p), ("v_new", _p), ("q_packed", _p),
                ("block_tables", _p), ("scale", ctypes.c_float), ("out", _p), ("out_dtype", _i32),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
                ("copy_off", _i32), ("num_copies", _i32),
                ("aux_stream", _p), ("aux_fork_event", _p), ("aux_join_event", _p)]


class PagedKVError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class NoSpace(PagedKVError):
    pass


_LIB = None

_SIGNATURES = {
    "pkv_kv_append": (_i32, [_p, _p, _p, _i32, ctypes.POINTER(PoolDesc), _p]),
    "pkv_paged_attend": (_i32, [_p, _i32, _i32, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                                ctypes.POINTER(PoolDesc), ctypes.c_float, _p, _i32, _p, ctypes.c_size_t, _p]),
    "pkv_paged_attend_noalloc": (_i32, [_p, _i32, _i32, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32,
                                        ctypes.POINTER(PoolDesc), ctypes.c_float, _p, _i32, _p]),
    "pkv_paged_attend_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(PoolDesc)]),
    "pkv_decode_partition_tokens": (_i32, []),
    "pkv_mixed_step": (_i32, [ctypes.POINTER(StepDesc), ctypes.POINTER(PoolDesc), _p]),
    "pkv_copy_blocks": (_i32, [_p, _p, _i32, ctypes.POINTER(PoolDesc), _p]),
    "pkv_gather_kv": (_i32, [_p, _i32, _p, _p, _i32, _i32, _i32, _p, ctypes.POINTER(PoolDesc),
                             ctypes.POINTER(PoolDesc), _p]),
    "pkv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_alloc_create": (_i32, [_i32, _i32, _i32, _i32, _pi32, ctypes.POINTER(_p)]),
    "pkv_alloc_destroy": (None, [_p]),
    "pkv_slot_acquire": (_i32, [_p, _i32]),
    "pkv_slot_release": (_i32, [_p, _i32]),
    "pkv_slot_truncate": (_i32, [_p, _i32, _i32]),
    "pkv_reserve": (_i32, [_p, _i32, _i32]),
    "pkv_lower_step": (_i32, [_p, _i32, _pi32, _pi32, _pi32, _i32, _pi32, _pi32, _pi32, _pi32, _pi32]),
    "pkv_lower_step_cow": (_i32, [_p, _i32, _pi32, _pi32, _pi32, _i32, _pi32, _pi32, _pi32, _pi32, _pi32,
                                  _pi32, _pi32, _i32, _pi32]),
    "pkv_slot_adopt": (_i32, [_p, _i32, _i32, _i32]),
    "pkv_block_refs": (_i32, [_p, _i32]),
    "pkv_free_blocks": (_i32, [_p]),
    "pkv_slot_info": (_i32, [_p, _i32, _pi32, _pi32]),
    "pkv_slot_table": (_i32, [_p, _i32, _pi32, _i32]),
    "pkv_pool_blocks_for_tokens": (ctypes.c_int64, [ctypes.c_int64, _i32]),
    "pkv_validate_step": (_i32, [_i32, _i32, _pi32, _pi32, _pi32, _i32, _pi32, _pi32, _i32, _i32, _i32,
                                 _pi32, _i32, _pi32]),
}


def lib():
    """Load libpagedkv.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_attention_slot_amd.build` (there is no fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        # pkv_lower_step_cow once more with its arrays as plain addresses
        # (a staging buffer's base plus offsets: no per-call pointer objects)
        raw = handle["pkv_lower_step_cow"]
        raw.restype = _i32
        raw.argtypes = [_p, _i32, _p, _p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _i32, _pi32]
        handle.lower_step_cow_raw = raw
        _LIB = handle
    return _LIB


def header_symbols():
    """Function names declared in include/pagedkv.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def status_str(status: int) -> str:
    try:
        return lib().pkv_status_str(int(status)).decode()
    except Exception:  # library not loadable: still give a message
        return "status"


def _check(status, what):
    if status != PKV_OK:
        if status == PKV_ERR_NO_SPACE:
            raise NoSpace(status, what)
        raise PagedKVError(status, what)


def _ptr_i32(a):
    """Host int32 numpy array (contiguous) -> ctypes pointer, or NULL."""
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_pi32)


# --------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def pkv_dtype_of(tdtype) -> int:
    torch = _torch()
    if tdtype == torch.bfloat16:
        return PKV_BF16
    if tdtype == torch.float32:
        return PKV_F32
    if tdtype == torch.int8:
        return PKV_I8
    raise ValueError(f"unsupported dtype {tdtype}")


def current_stream_handle(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_HIP_RT = None


class StreamEvent:
    """A HIP event for ordering one stream after another on the same GPU:
    created with hipEventDisableTiming | hipEventDisableSystemFence, so a
    record takes no system-scope cache writeback and invalidate (the device
    work that waits on it still follows the recorded work, and sees its
    writes).  Host-side waits on it (query, synchronize) tell that the
    recorded work has finished, not that its device writes are visible to
    the host.  Made on the HIP runtime PyTorch loaded, so torch stream
    handles apply."""

    _FLAGS = 0x2 | 0x20000000   # hipEventDisableTiming | hipEventDisableSystemFence

    def __init__(self):
        global _HIP_RT
        if _HIP_RT is None:
            _torch().cuda.init()
            path = [ln.split()[-1] for ln in open("/proc/self/maps").read().splitlines()
                    if "libamdhip64" in ln][0]
            rt = ctypes.CDLL(path)
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_p), ctypes.c_uint]
            rt.hipEventDestroy.argtypes = [_p]
            rt.hipEventRecord.argtypes = [_p, _p]
            rt.hipEventQuery.argtypes = [_p]
            rt.hipEventSynchronize.argtypes = [_p]
            _HIP_RT = rt
        self._rt = _HIP_RT
        self.handle = _p()
        if self._rt.hipEventCreateWithFlags(ctypes.byref(self.handle), self._FLAGS) != 0:
            raise PagedKVError("hipEventCreateWithFlags failed")

    def __del__(self):
        if getattr(self, "handle", None):
            self._rt.hipEventDestroy(self.handle)

    # Host-side waits, for work that only reads host memory (a pinned staging
    # buffer may be rewritten once the kernels that read it have finished;
    # no device writes need to become visible to the host).
    def record(self, stream):
        if self._rt.hipEventRecord(self.handle, _p(stream.cuda_stream)) != 0:
            raise PagedKVError("hipEventRecord failed")

    def query(self):
        return self._rt.hipEventQuery(self.handle) == 0       # hipSuccess: the recorded work is done

    def synchronize(self):
        if self._rt.hipEventSynchronize(self.handle) != 0:
            raise PagedKVError("hipEventSynchronize failed")


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class KVPool:
    """The shared pool: K and V, each [num_blocks][num_kv_heads][16][head_dim].
    dtype torch.int8 makes an 8-bit pool: int8 codes plus float32 scales
    [num_blocks][num_kv_heads][2][16] (K's 16 then V's 16 per block and head;
    see pkv_pool); k_scale / v_scale are views of its two halves.  Poison
    fills unwritten positions with NaN (codes: -128, never a valid code)."""

    def __init__(self, num_blocks, num_kv_heads, head_dim, dtype, block_size=16, device="cuda", poison=True):
        torch = _torch()
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k = torch.empty(shape, dtype=dtype, device=device)
        self.v = torch.empty(shape, dtype=dtype, device=device)
        self.scales = self.k_scale = self.v_scale = None
        if dtype == torch.int8:
            self.scales = torch.empty((num_blocks, num_kv_heads, 2, block_size), dtype=torch.float32, device=device)
            self.k_scale = self.scales[:, :, 0]
            self.v_scale = self.scales[:, :, 1]
        if poison:
            if dtype == torch.int8:
                self.k.fill_(-128)
                self.v.fill_(-128)
                self.scales.fill_(float("nan"))
            else:
                self.k.fill_(float("nan"))
                self.v.fill_(float("nan"))
        self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size = num_blocks, num_kv_heads, head_dim, block_size
        self.dtype = dtype
        self._desc = PoolDesc(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.block_size,
                              self.num_kv_heads, self.head_dim, pkv_dtype_of(self.dtype),
                              self.scales.data_ptr() if self.scales is not None else None)
        self._desc_ref = ctypes.byref(self._desc)

    def desc(self) -> PoolDesc:
        return self._desc


def kv_append(slot_mapping, k_new, v_new, pool: KVPool, stream=None):
    """Scatter k_new/v_new [T][Hkv][D] into the pool at slot_mapping [T] (device int32)."""
    t = int(slot_mapping.shape[0])
    st = lib().pkv_kv_append(_dptr(slot_mapping), _dptr(k_new), _dptr(v_new), t, pool._desc_ref,
                             stream if stream is not None else current_stream_handle())
    _check(st, "pkv_kv_append")


def copy_blocks(src_blocks, dst_blocks, pool: KVPool, stream=None):
    """Copy whole blocks src_blocks[c] -> dst_blocks[c] (device int32 tensors)."""
    n = int(src_blocks.shape[0])
    st = lib().pkv_copy_blocks(_dptr(src_blocks), _dptr(dst_blocks), n, pool._desc_ref,
                               stream if stream is not None else current_stream_handle())
    _check(st, "pkv_copy_blocks")


def gather_kv(row_to_slot, context_lens, block_tables, dst_block_start, src: KVPool, dst: KVPool, *,
              max_context_len, stream=None):
    """Rebuild each segment's visible window contiguously in `dst` (the
    gather ablation); device int32 metadata as for paged_attend."""
    st = lib().pkv_gather_kv(_dptr(row_to_slot), int(row_to_slot.shape[0]), _dptr(context_lens),
                             _dptr(block_tables), int(block_tables.shape[0]), int(block_tables.shape[1]),
                             int(max_context_len), _dptr(dst_block_start), src._desc_ref, dst._desc_ref,
                             stream if stream is not None else current_stream_handle())
    _check(st, "pkv_gather_kv")


def workspace_bytes(num_segments, total_q, num_q_heads, max_query_len, max_context_len, pool: KVPool) -> int:
    n = lib().pkv_paged_attend_workspace_bytes(num_segments, total_q, num_q_heads, max_query_len,
                                               max_context_len, pool._desc_ref)
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID_ARG, "pkv_paged_attend_workspace_bytes")
    return int(n)


def paged_attend(q_packed, row_to_slot, query_start, query_len, context_lens, block_tables, pool: KVPool,
                 scale, *, max_query_len, max_context_len, out, workspace=None, stream=None):
    """Mixed-step paged attention; all tensors on the device, metadata int32.
    `out` [total_q][Hq][D] is float32 or the pool dtype."""
    total_q, hq = int(q_packed.shape[0]), int(q_packed.shape[1])
    nseg = int(row_to_slot.shape[0])
    num_slots, maxb = int(block_tables.shape[0]), int(block_tables.shape[1])
    ws_ptr = _dptr(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().pkv_paged_attend(_dptr(q_packed), total_q, hq, _dptr(row_to_slot), _dptr(query_start),
                                _dptr(query_len), nseg, _dptr(context_lens), _dptr(block_tables), num_slots, maxb,
                                int(max_query_len), int(max_context_len), pool._desc_ref, float(scale),
                                _dptr(out), pkv_dtype_of(out.dtype), ws_ptr, ws_bytes,
                                stream if stream is not None else current_stream_handle())
    _check(st, "pkv_paged_attend")
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20     # PKV_NOALLOC_SCRATCH_BYTES in include/pagedkv.h


def paged_attend_noalloc(q_packed, row_to_slot, query_start, query_len, context_lens, block_tables, pool: KVPool,
                         scale, *, max_query_len, max_context_len, out, stream=None):
    """paged_attend with the library's own scratch instead of a workspace
    (pkv_paged_attend_noalloc: allocates nothing; calls overlapping on one
    GPU race)."""
    total_q, hq = int(q_packed.shape[0]), int(q_packed.shape[1])
    nseg = int(row_to_slot.shape[0])
    num_slots, maxb = int(block_tables.shape[0]), int(block_tables.shape[1])
    st = lib().pkv_paged_attend_noalloc(_dptr(q_packed), total_q, hq, _dptr(row_to_slot), _dptr(query_start),
                                        _dptr(query_len), nseg, _dptr(context_lens), _dptr(block_tables), num_slots,
                                        maxb, int(max_query_len), int(max_context_len), pool._desc_ref,
                                        float(scale), _dptr(out), pkv_dtype_of(out.dtype),
                                        stream if stream is not None else current_stream_handle())
    _check(st, "pkv_paged_attend_noalloc")
    return out


def mixed_step(desc: StepDesc, pool: KVPool, stream):
    """pkv_mixed_step: staged-metadata append + paged attention (two launches)."""
    _check(lib().pkv_mixed_step(ctypes.byref(desc), pool._desc_ref, stream), "pkv_mixed_step")


def decode_partition_tokens() -> int:
    return int(lib().pkv_decode_partition_tokens())


def pool_blocks_for_tokens(tokens: int, block_size: int) -> int:
    return int(lib().pkv_pool_blocks_for_tokens(int(tokens), int(block_size)))


def validate_step(meta: dict, total_q, num_blocks, block_size, max_blocks_per_seq, num_tokens=None):
    """Check host metadata arrays; returns (ok, bad_index)."""
    bad = ctypes.c_int32(-1)
    sm = meta.get("slot_mapping")
    st = lib().pkv_validate_step(int(total_q), len(meta["row_to_slot"]), _ptr_i32(meta["row_to_slot"]),
                                 _ptr_i32(meta["query_start"]), _ptr_i32(meta["query_len"]),
                                 len(meta["context_lens"]), _ptr_i32(meta["context_lens"]),
                                 _ptr_i32(meta["block_tables"]), int(max_blocks_per_seq), int(num_blocks),
                                 int(block_size), _ptr_i32(sm), int(num_tokens if num_tokens is not None else
                                                                   (len(sm) if sm is not None else 0)),
                                 ctypes.byref(bad))
    return st == PKV_OK, int(bad.value)


class BlockAllocator:
    """Host block-pool allocator (C++), see pkv_alloc_* in include/pagedkv.h."""

    def __init__(self, num_blocks, block_size, max_slots, max_blocks_per_seq, free_order=None):
        self._lib = lib()
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.max_slots, self.max_blocks_per_seq = int(max_slots), int(max_blocks_per_seq)
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        h = ctypes.c_void_p()
        _check(self._lib.pkv_alloc_create(self.num_blocks, self.block_size, self.max_slots,
                                          self.max_blocks_per_seq, _ptr_i32(order), ctypes.byref(h)),
               "pkv_alloc_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_alloc_destroy(h)
            self._h = None

    def acquire(self, slot):
        _check(self._lib.pkv_slot_acquire(self._h, int(slot)), "pkv_slot_acquire")

    def release(self, slot):
        _check(self._lib.pkv_slot_release(self._h, int(slot)), "pkv_slot_release")

    def truncate(self, slot, new_len):
        _check(self._lib.pkv_slot_truncate(self._h, int(slot), int(new_len)), "pkv_slot_truncate")

    def reserve(self, slot, total_tokens):
        _check(self._lib.pkv_reserve(self._h, int(slot), int(total_tokens)), "pkv_reserve")

    def adopt(self, slot, src_slot, num_tokens):
        """`slot` (acquired, empty) takes src_slot's first num_tokens tokens by reference."""
        _check(self._lib.pkv_slot_adopt(self._h, int(slot), int(src_slot), int(num_tokens)), "pkv_slot_adopt")

    def block_refs(self, block) -> int:
        return int(self._lib.pkv_block_refs(self._h, int(block)))

    def free_blocks(self) -> int:
        return int(self._lib.pkv_free_blocks(self._h))

    def slot_info(self, slot):
        n, b = ctypes.c_int32(), ctypes.c_int32()
        st = self._lib.pkv_slot_info(self._h, int(slot), ctypes.byref(n), ctypes.byref(b))
        return (int(n.value), int(b.value)) if st == PKV_OK else None

    def slot_table(self, slot):
        info = self.slot_info(slot)
        if info is None:
            return None
        out = np.zeros(max(info[1], 1), dtype=np.int32)
        _check(self._lib.pkv_slot_table(self._h, int(slot), _ptr_i32(out), len(out)), "pkv_slot_table")
        return out[:info[1]].tolist()

    def lower_step_raw(self, n, slots_addr, news_addr, sm_addr, sm_len, qs_addr, ql_addr, rts_addr, cl_addr,
                       csrc_addr, cdst_addr, copy_cap):
        """pkv_lower_step_cow on raw host addresses of int32 arrays (no block
        tables out): slots / news [n] in, slot_mapping [sm_len], query_start /
        query_len / row_to_slot [n], context_lens [max_slots] and copy_src /
        copy_dst [copy_cap] out.  Returns the number of copy pairs."""
        ncopy = ctypes.c_int32(0)
        _check(self._lib.lower_step_cow_raw(self._h, n, slots_addr, news_addr, sm_addr, sm_len, qs_addr, ql_addr,
                                            rts_addr, cl_addr, None, csrc_addr, cdst_addr, copy_cap,
                                            ctypes.byref(ncopy)), "pkv_lower_step_cow")
        return ncopy.value

    def lower_step(self, entries, out=None):
        """entries: [(slot, n_new)] in packed order -> dict of host int32 arrays,
        copy-on-write pairs included (copy_src / copy_dst, trimmed to the count).
        `out` may supply preallocated arrays (same keys) to fill in place; its
        copy_src / copy_dst, when given, need room for len(entries) pairs."""
        slots = np.ascontiguousarray([e[0] for e in entries], dtype=np.int32)
        news = np.ascontiguousarray([e[1] for e in entries], dtype=np.int32)
        t = int(news.sum()) if len(news) else 0
        n = len(entries)
        if out is None:
            out = dict(slot_mapping=np.empty(t, np.int32), query_start=np.empty(n, np.int32),
                       query_len=np.empty(n, np.int32), row_to_slot=np.empty(n, np.int32),
                       context_lens=np.empty(self.max_slots, np.int32),
                       block_tables=np.empty((self.max_slots, self.max_blocks_per_seq), np.int32))
        csrc = out.get("copy_src")
        cdst = out.get("copy_dst")
        if csrc is None or cdst is None:
            csrc, cdst = np.empty(max(n, 1), np.int32), np.empty(max(n, 1), np.int32)
        ncopy = ctypes.c_int32(0)
        st = self._lib.pkv_lower_step_cow(self._h, n, _ptr_i32(slots), _ptr_i32(news),
                                          _ptr_i32(out["slot_mapping"]), len(out["slot_mapping"]),
                                          _ptr_i32(out["query_start"]), _ptr_i32(out["query_len"]),
                                          _ptr_i32(out["row_to_slot"]), _ptr_i32(out.get("context_lens")),
                                          _ptr_i32(out.get("block_tables")), _ptr_i32(csrc), _ptr_i32(cdst),
                                          min(len(csrc), len(cdst)), ctypes.byref(ncopy))
        _check(st, "pkv_lower_step_cow")
        out["copy_src"], out["copy_dst"] = csrc[:ncopy.value], cdst[:ncopy.value]
        return out
