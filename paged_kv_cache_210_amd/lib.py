"""ctypes binding of libpkv.so (the C ABI declared in include/pkv.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of the library.  torch supplies device memory and the current stream.
``load()`` raises if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_NO_BLOCKS = -3
PKV_ERR_WORKSPACE = -4
PKV_ERR_DEVICE = -5
PKV_ERR_BAD_TABLE = -6
PKV_ERR_SHARED = -7
PKV_ERR_TOO_LARGE = -8
PKV_ERR_OFFLOADED = -9
OFFLOADED = -2                      # PKV_OFFLOADED: table entry of a block in a host slot
STATIC_SCRATCH_BYTES = 16 << 20     # PKV_STATIC_SCRATCH_BYTES

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
BLOCK_SIZE = 16
SCALE_GROUP = 64

_DTYPE_CODE = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}
_CODE_DTYPE = {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16, PKV_FP8_E4M3: torch.uint8}
KV_DTYPES = {"f32": PKV_F32, "bf16": PKV_BF16, "e4m3": PKV_FP8_E4M3}


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("k_cache", c_void_p), ("v_cache", c_void_p), ("block_stride", c_int64),
                ("k_scale", c_void_p), ("v_scale", c_void_p), ("num_blocks", c_int32),
                ("num_kv_heads", c_int32), ("block_size", c_int32), ("head_dim", c_int32),
                ("kv_dtype", c_int32)]


_lib = None

_SIGS = {
    "pkv_status_str": (ctypes.c_char_p, [c_int32]),
    "pkv_allocator_create": (c_int32, [c_int32, c_void_p, POINTER(c_void_p)]),
    "pkv_allocator_reserve": (c_int32, [c_void_p, c_int32, c_int64, c_void_p, c_int32,
                                        POINTER(c_int32)]),
    "pkv_allocator_release": (c_int32, [c_void_p, c_int32]),
    "pkv_allocator_waste_slots": (c_int32, [c_void_p, c_int32, POINTER(c_int64)]),
    "pkv_allocator_free_count": (c_int32, [c_void_p, POINTER(c_int32)]),
    "pkv_allocator_destroy": (None, [c_void_p]),
    "pkv_allocator_reserve_cow": (c_int32, [c_void_p, c_int32, c_int64, c_void_p, c_int32,
                                            POINTER(c_int32), POINTER(c_int32),
                                            POINTER(c_int32)]),
    "pkv_allocator_fork": (c_int32, [c_void_p, c_int32, c_int32]),
    "pkv_allocator_publish_prefix": (c_int32, [c_void_p, c_int32, c_void_p, c_int32]),
    "pkv_allocator_match_prefix": (c_int32, [c_void_p, c_int32, c_void_p, c_int32,
                                             POINTER(c_int32)]),
    "pkv_allocator_refcount": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "pkv_allocator_set_host_slots": (c_int32, [c_void_p, c_int32]),
    "pkv_allocator_offload": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                        POINTER(c_int32)]),
    "pkv_allocator_page_in": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                        POINTER(c_int32)]),
    "pkv_allocator_touch": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64]),
    "pkv_allocator_block_state": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_int32),
                                            POINTER(c_int32), POINTER(c_int64)]),
    "pkv_allocator_table": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, POINTER(c_int32)]),
    "pkv_allocator_host_free_count": (c_int32, [c_void_p, POINTER(c_int32)]),
    "pkv_allocator_coldest": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p,
                                        POINTER(c_int32)]),
    "pkv_copy_blocks": (c_int32, [POINTER(CacheDesc), POINTER(CacheDesc), c_void_p, c_void_p,
                                  c_int32, c_void_p]),
    "pkv_kv_append": (c_int32, [POINTER(CacheDesc), c_void_p, c_void_p, c_int32, c_int32,
                                c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "pkv_fp8_group_scales": (c_int32, [POINTER(CacheDesc), c_void_p, c_void_p, c_int32, c_int32,
                                       c_int32, c_void_p, c_int32, c_void_p]),
    "pkv_kv_append_fp8_groups": (c_int32, [POINTER(CacheDesc), c_void_p, c_void_p, c_int32,
                                           c_int32, c_int32, c_void_p, c_int32, c_void_p]),
    "pkv_decode_workspace_bytes": (c_int32, [POINTER(CacheDesc), c_int32, c_int32, c_int32,
                                             c_int32, c_int32, POINTER(c_size_t)]),
    "pkv_paged_attn_decode": (c_int32, [POINTER(CacheDesc), c_void_p, c_int32, c_int32, c_int32,
                                        c_void_p, c_int32, c_void_p, c_float, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_size_t, c_void_p]),
    "pkv_paged_attn_decode_noalloc": (c_int32, [POINTER(CacheDesc), c_void_p, c_int32, c_int32,
                                                c_int32, c_void_p, c_int32, c_void_p, c_float,
                                                c_int32, c_void_p, c_void_p, c_void_p]),
    "pkv_decode_partitions": (c_int32, [POINTER(CacheDesc), c_int32, c_int32, c_int32, c_int32,
                                        c_int32, POINTER(c_int32)]),
    "pkv_paged_attn_decode_partial": (c_int32, [POINTER(CacheDesc), c_void_p, c_int32, c_int32,
                                                c_int32, c_void_p, c_int32, c_void_p, c_float,
                                                c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "pkv_paged_attn_decode_step": (c_int32, [POINTER(CacheDesc), c_void_p, c_void_p, c_void_p,
                                             c_int32, c_int32, c_int32, c_void_p, c_int32,
                                             c_void_p, c_float, c_int32, c_void_p, c_void_p,
                                             c_void_p, c_size_t, c_void_p]),
    "pkv_paged_attn_decode_step_partial": (c_int32, [POINTER(CacheDesc), c_void_p, c_void_p,
                                                     c_void_p, c_int32, c_int32, c_int32,
                                                     c_void_p, c_int32, c_void_p, c_float,
                                                     c_int32, c_void_p, c_void_p, c_void_p,
                                                     c_void_p]),
    "pkv_paged_attn_prefill": (c_int32, [POINTER(CacheDesc), c_void_p, c_int32, c_int32, c_int32,
                                         c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                         c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
    "pkv_attn_lse_merge": (c_int32, [c_int32, c_int64, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "pkv_validate_tables": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                      POINTER(c_int64), c_void_p]),
}


def load(path: str = LIB_PATH):
    """Load libpkv.so (once).  Raises FileNotFoundError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it first (python -m paged_kv_cache_210_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().pkv_status_str(status).decode()


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PkvError(status, what)


def _p(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(device) -> c_void_p:
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_q(q, cache, dtype=None):
    """q [rows, Hq, head_dim] on the cache's device, with Hq a multiple of the
    cache's kv heads and head_dim the cache's; returns its shape."""
    _need(q, dtype, "q", cache.device)
    if q.dim() != 3:
        raise ValueError(f"q must be [rows, heads, head_dim], got shape {tuple(q.shape)}")
    rows, hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError(f"q head_dim {D} != cache head_dim {cache.head_dim}")
    if hq % cache.hkv:
        raise ValueError(f"q heads {hq} not a multiple of the cache's {cache.hkv} kv heads")
    return rows, hq, D


# ---------------------------------------------------------------- cache
class PagedCache:
    """One layer's block pool: K [num_blocks, Hkv, 16, d], V [num_blocks, Hkv, d, 16]
    tensors (E4M3 pools are uint8 with fp32 scales [num_blocks, Hkv]).  f32
    pages use those shapes' natural order; bf16 and E4M3 pages hold the same
    elements in the fragment order pkv.h documents."""

    def __init__(self, k, v, kv_dtype: int, k_scale=None, v_scale=None):
        self.k, self.v = k, v
        self.kv_dtype = kv_dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.num_blocks, self.hkv = k.shape[0], k.shape[1]
        self.head_dim = k.shape[3]
        self.device = k.device

    @classmethod
    def empty(cls, num_blocks, hkv, head_dim, kv_dtype, device="cuda", fill=None, pinned=False):
        """A pool on `device`; pinned=True puts it in pinned host memory instead
        (device-addressable: the target or source of an offload)."""
        code = KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype
        dt = _CODE_DTYPE[code]
        kw = dict(device="cpu", pin_memory=True) if pinned else dict(device=device)
        k = torch.empty(num_blocks, hkv, BLOCK_SIZE, head_dim, dtype=dt, **kw)
        v = torch.empty(num_blocks, hkv, head_dim, BLOCK_SIZE, dtype=dt, **kw)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        ks = vs = None
        if code == PKV_FP8_E4M3:
            ks = torch.ones(num_blocks, hkv, dtype=torch.float32, **kw)
            vs = torch.ones(num_blocks, hkv, dtype=torch.float32, **kw)
        return cls(k, v, code, ks, vs)

    def desc(self) -> CacheDesc:
        return CacheDesc(self.k.data_ptr(), self.v.data_ptr(), self.hkv * BLOCK_SIZE * self.head_dim,
                         None if self.k_scale is None else self.k_scale.data_ptr(),
                         None if self.v_scale is None else self.v_scale.data_ptr(),
                         self.num_blocks, self.hkv, BLOCK_SIZE, self.head_dim, self.kv_dtype)


# ---------------------------------------------------------------- allocator
class Allocator:
    """Host block allocator (pkv_allocator_*)."""

    def __init__(self, num_blocks: int, free_order=None):
        lib = load()
        self._h = c_void_p()
        arr = None
        if free_order is not None:
            order = [int(b) for b in free_order]
            arr = (c_int32 * len(order))(*order)
        _check(lib.pkv_allocator_create(num_blocks, arr, ctypes.byref(self._h)), "allocator_create")
        self.num_blocks = num_blocks

    def reserve(self, seq: int, new_len: int, max_blocks: int = None):
        max_blocks = max_blocks or max(1, -(-new_len // BLOCK_SIZE))
        row = (c_int32 * max_blocks)()
        n = c_int32()
        _check(load().pkv_allocator_reserve(self._h, seq, new_len, row, max_blocks,
                                            ctypes.byref(n)), "allocator_reserve")
        return list(row[:n.value])

    def reserve_cow(self, seq: int, new_len: int, max_blocks: int = None):
        """reserve() that may first move the sequence off a shared last block;
        returns (table, (src, dst) of the block copy to make, or None)."""
        max_blocks = max_blocks or max(1, -(-new_len // BLOCK_SIZE))
        row = (c_int32 * max_blocks)()
        n, cs, cd = c_int32(), c_int32(), c_int32()
        _check(load().pkv_allocator_reserve_cow(self._h, seq, new_len, row, max_blocks,
                                                ctypes.byref(n), ctypes.byref(cs),
                                                ctypes.byref(cd)), "allocator_reserve_cow")
        return list(row[:n.value]), (None if cs.value < 0 else (cs.value, cd.value))

    def fork(self, src_seq: int, dst_seq: int):
        _check(load().pkv_allocator_fork(self._h, src_seq, dst_seq), "allocator_fork")

    def publish_prefix(self, seq: int, block_hashes):
        arr = (ctypes.c_uint64 * max(1, len(block_hashes)))(*[int(h) for h in block_hashes])
        _check(load().pkv_allocator_publish_prefix(self._h, seq, arr, len(block_hashes)),
               "allocator_publish_prefix")

    def match_prefix(self, seq: int, block_hashes) -> int:
        arr = (ctypes.c_uint64 * max(1, len(block_hashes)))(*[int(h) for h in block_hashes])
        out = c_int32()
        _check(load().pkv_allocator_match_prefix(self._h, seq, arr, len(block_hashes),
                                                 ctypes.byref(out)), "allocator_match_prefix")
        return out.value

    def refcount(self, block: int) -> int:
        out = c_int32()
        _check(load().pkv_allocator_refcount(self._h, block, ctypes.byref(out)),
               "allocator_refcount")
        return out.value

    def release(self, seq: int):
        _check(load().pkv_allocator_release(self._h, seq), "allocator_release")

    # host tier (KV offload): the C page table; data moves with copy_blocks
    def set_host_slots(self, n: int):
        _check(load().pkv_allocator_set_host_slots(self._h, n), "allocator_set_host_slots")

    def _moves(self, fn, seq, first, count, what):
        k = max(0, int(count))
        a, b = (c_int32 * max(1, k))(), (c_int32 * max(1, k))()
        n = c_int32()
        _check(fn(self._h, seq, int(first), k, a, b, ctypes.byref(n)), what)
        return list(zip(a[:n.value], b[:n.value]))

    def offload(self, seq: int, first: int, count: int):
        """[(device block, host slot)] to copy device -> host."""
        return self._moves(load().pkv_allocator_offload, seq, first, count, "allocator_offload")

    def page_in(self, seq: int, first: int, count: int):
        """[(host slot, device block)] to copy host -> device."""
        return self._moves(load().pkv_allocator_page_in, seq, first, count, "allocator_page_in")

    def touch(self, seq: int, first: int, count: int, step: int):
        _check(load().pkv_allocator_touch(self._h, seq, int(first), int(count), int(step)),
               "allocator_touch")

    def block_state(self, seq: int, block: int):
        """(device id or OFFLOADED, host slot or -1, last step read or -1)."""
        d, h, t = c_int32(), c_int32(), c_int64()
        _check(load().pkv_allocator_block_state(self._h, seq, block, ctypes.byref(d),
                                                ctypes.byref(h), ctypes.byref(t)),
               "allocator_block_state")
        return d.value, h.value, t.value

    def table(self, seq: int, max_blocks: int = 1 << 20):
        row = (c_int32 * max_blocks)()
        n = c_int32()
        _check(load().pkv_allocator_table(self._h, seq, row, max_blocks, ctypes.byref(n)),
               "allocator_table")
        return list(row[:n.value])

    def host_free_count(self) -> int:
        out = c_int32()
        _check(load().pkv_allocator_host_free_count(self._h, ctypes.byref(out)),
               "host_free_count")
        return out.value

    def coldest(self, max_n: int):
        a, b = (c_int32 * max(1, max_n))(), (c_int32 * max(1, max_n))()
        n = c_int32()
        _check(load().pkv_allocator_coldest(self._h, max_n, a, b, ctypes.byref(n)),
               "allocator_coldest")
        return list(zip(a[:n.value], b[:n.value]))

    def waste_slots(self, seq: int) -> int:
        out = c_int64()
        _check(load().pkv_allocator_waste_slots(self._h, seq, ctypes.byref(out)), "waste_slots")
        return out.value

    def free_count(self) -> int:
        out = c_int32()
        _check(load().pkv_allocator_free_count(self._h, ctypes.byref(out)), "free_count")
        return out.value

    def close(self):
        if self._h:
            load().pkv_allocator_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build_tables(seq_lens, num_blocks, free_order=None, max_blocks=None):
    """Reserve every sequence in order with the library allocator; returns
    (int32 CPU tensor [B, maxb] padded with -1, waste slots per sequence)."""
    alloc = Allocator(num_blocks, free_order)
    rows = [alloc.reserve(b, int(n)) for b, n in enumerate(seq_lens)]
    maxb = max([len(r) for r in rows] + [1]) if max_blocks is None else max_blocks
    t = torch.full((len(seq_lens), maxb), -1, dtype=torch.int32)
    for b, r in enumerate(rows):
        if r:
            t[b, :len(r)] = torch.tensor(r, dtype=torch.int32)
    waste = [alloc.waste_slots(b) for b in range(len(seq_lens))]
    alloc.close()
    return t, waste


# ---------------------------------------------------------------- device ops
def kv_append(cache: PagedCache, k_new, v_new, seq_idx, pos, block_tables):
    dev = cache.device
    T = k_new.shape[0]
    src = _DTYPE_CODE.get(k_new.dtype)
    if src is None:
        raise TypeError("k_new must be float32 or bfloat16")
    shape = (T, cache.hkv, cache.head_dim)
    _need(k_new, None, "k_new", dev, shape)
    _need(v_new, k_new.dtype, "v_new", dev, shape)
    _need(seq_idx, torch.int32, "seq_idx", dev, (T,))
    _need(pos, torch.int32, "pos", dev, (T,))
    _need(block_tables, torch.int32, "block_tables", dev)
    d = cache.desc()
    _check(load().pkv_kv_append(ctypes.byref(d), _p(k_new), _p(v_new), src, T, _p(seq_idx),
                                _p(pos), _p(block_tables), block_tables.shape[0],
                                block_tables.shape[1], _stream(dev)), "kv_append")


def fp8_group_scales(cache: PagedCache, k_src, v_src, pos0, table_row):
    dev = cache.device
    T = k_src.shape[0]
    src = _DTYPE_CODE.get(k_src.dtype)
    shape = (T, cache.hkv, cache.head_dim)
    _need(k_src, None, "k_src", dev, shape)
    _need(v_src, k_src.dtype, "v_src", dev, shape)
    _need(table_row, torch.int32, "table_row", dev)
    d = cache.desc()
    _check(load().pkv_fp8_group_scales(ctypes.byref(d), _p(k_src), _p(v_src),
                                       -1 if src is None else src, T, int(pos0), _p(table_row),
                                       table_row.numel(), _stream(dev)), "fp8_group_scales")


def kv_append_fp8_groups(cache: PagedCache, k_new, v_new, pos0, table_row):
    """pkv_kv_append_fp8_groups: the group scales and the append of one
    sequence's tokens [pos0, pos0 + T) into an E4M3 pool in one pass."""
    dev = cache.device
    T = k_new.shape[0]
    src = _DTYPE_CODE.get(k_new.dtype)
    if src is None:
        raise TypeError("k_new must be float32 or bfloat16")
    shape = (T, cache.hkv, cache.head_dim)
    _need(k_new, None, "k_new", dev, shape)
    _need(v_new, k_new.dtype, "v_new", dev, shape)
    _need(table_row, torch.int32, "table_row", dev)
    d = cache.desc()
    _check(load().pkv_kv_append_fp8_groups(ctypes.byref(d), _p(k_new), _p(v_new), src, T,
                                           int(pos0), _p(table_row), table_row.numel(),
                                           _stream(dev)), "kv_append_fp8_groups")


def decode_workspace_bytes(cache: PagedCache, q_dtype, B, hq, max_blocks, partition_blocks=0):
    out = c_size_t()
    d = cache.desc()
    code = _DTYPE_CODE[q_dtype] if isinstance(q_dtype, torch.dtype) else q_dtype
    _check(load().pkv_decode_workspace_bytes(ctypes.byref(d), code, B, hq, max_blocks,
                                             partition_blocks, ctypes.byref(out)),
           "decode_workspace_bytes")
    return out.value


def decode_workspace(cache, q, block_tables, partition_blocks=0):
    n = decode_workspace_bytes(cache, q.dtype, q.shape[0], q.shape[1], block_tables.shape[1],
                               partition_blocks)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=cache.device)


def paged_attn_decode(cache: PagedCache, q, block_tables, seq_lens, scale=0.0,
                      partition_blocks=0, out=None, out_lse=None, ws=None, with_lse=True):
    dev = cache.device
    B, hq, D = _need_q(q, cache)
    qc = _DTYPE_CODE.get(q.dtype)
    if qc is None:
        raise TypeError("q must be float32 or bfloat16")
    _need(block_tables, torch.int32, "block_tables", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.dtype, "out", dev, q.shape)
    if out_lse is None and with_lse:
        out_lse = torch.empty(B, hq, dtype=torch.float32, device=dev)
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", dev, (B, hq))
    if ws is None:
        ws = decode_workspace(cache, q, block_tables, partition_blocks)
    _need(ws, None, "ws", dev)
    d = cache.desc()
    _check(load().pkv_paged_attn_decode(ctypes.byref(d), _p(q), qc, B, hq, _p(block_tables),
                                        block_tables.shape[1], _p(seq_lens), float(scale),
                                        int(partition_blocks), _p(out), _p(out_lse), _p(ws),
                                        ws.numel() * ws.element_size(), _stream(dev)),
           "paged_attn_decode")
    return out, out_lse


def paged_attn_decode_noalloc(cache: PagedCache, q, block_tables, seq_lens, scale=0.0,
                              partition_blocks=0, out=None, out_lse=None, with_lse=True):
    """pkv_paged_attn_decode_noalloc: the decode of paged_attn_decode with its
    partials in the library's static device scratch (no workspace).  `out`
    and `out_lse` are made here when not given; a caller that must not
    allocate passes both (or with_lse=False)."""
    dev = cache.device
    B, hq, D = _need_q(q, cache)
    qc = _DTYPE_CODE.get(q.dtype)
    if qc is None:
        raise TypeError("q must be float32 or bfloat16")
    _need(block_tables, torch.int32, "block_tables", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, q.dtype, "out", dev, q.shape)
    if out_lse is None and with_lse:
        out_lse = torch.empty(B, hq, dtype=torch.float32, device=dev)
    if out_lse is not None:
        _need(out_lse, torch.float32, "out_lse", dev, (B, hq))
    d = cache.desc()
    _check(load().pkv_paged_attn_decode_noalloc(ctypes.byref(d), _p(q), qc, B, hq,
                                                _p(block_tables), block_tables.shape[1],
                                                _p(seq_lens), float(scale), int(partition_blocks),
                                                _p(out), _p(out_lse), _stream(dev)),
           "paged_attn_decode_noalloc")
    return out, out_lse


def paged_attn_decode_step(cache: PagedCache, k_new, v_new, q, block_tables, seq_lens, scale=0.0,
                           partition_blocks=0, out=None, out_lse=None, ws=None, partial=False,
                           part=None):
    """pkv_paged_attn_decode_step(_partial): append token seq_lens[b]-1 of every
    sequence from k_new / v_new ([B, Hkv, d] bf16) and decode, in the decode's
    own launches.  Returns (out, out_lse), or (part_o, part_m, part_l)."""
    dev = cache.device
    B, hq, D = _need_q(q, cache, torch.bfloat16)
    _need(k_new, torch.bfloat16, "k_new", dev, (B, cache.hkv, D))
    _need(v_new, torch.bfloat16, "v_new", dev, (B, cache.hkv, D))
    _need(block_tables, torch.int32, "block_tables", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev, (B,))
    d = cache.desc()
    head = (ctypes.byref(d), _p(k_new), _p(v_new), _p(q), PKV_BF16, B, hq, _p(block_tables),
            block_tables.shape[1], _p(seq_lens), float(scale), int(partition_blocks))
    if partial:
        P = decode_partitions(cache, q.dtype, B, hq, block_tables.shape[1], partition_blocks)
        if part is None:
            part = (torch.empty(P, B, hq, D, dtype=torch.float32, device=dev),
                    torch.empty(P, B, hq, dtype=torch.float32, device=dev),
                    torch.empty(P, B, hq, dtype=torch.float32, device=dev))
        _need(part[0], torch.float32, "part_o", dev, (P, B, hq, D))
        _need(part[1], torch.float32, "part_m", dev, (P, B, hq))
        _need(part[2], torch.float32, "part_l", dev, (P, B, hq))
        _check(load().pkv_paged_attn_decode_step_partial(*head, _p(part[0]), _p(part[1]),
                                                         _p(part[2]), _stream(dev)),
               "paged_attn_decode_step_partial")
        return part
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out", dev, (B, hq, D))
    if out_lse is None:
        out_lse = torch.empty(B, hq, dtype=torch.float32, device=dev)
    _need(out_lse, torch.float32, "out_lse", dev, (B, hq))
    if ws is None:
        ws = decode_workspace(cache, q, block_tables, partition_blocks)
    _need(ws, None, "ws", dev)
    _check(load().pkv_paged_attn_decode_step(*head, _p(out), _p(out_lse), _p(ws),
                                             ws.numel() * ws.element_size(), _stream(dev)),
           "paged_attn_decode_step")
    return out, out_lse


def decode_partitions(cache, q_dtype, B, hq, max_blocks, partition_blocks=0):
    out = c_int32()
    d = cache.desc()
    code = _DTYPE_CODE[q_dtype] if isinstance(q_dtype, torch.dtype) else q_dtype
    _check(load().pkv_decode_partitions(ctypes.byref(d), code, B, hq, max_blocks,
                                        partition_blocks, ctypes.byref(out)), "decode_partitions")
    return out.value


def paged_attn_decode_partial(cache: PagedCache, q, block_tables, seq_lens, scale=0.0,
                              partition_blocks=0, part=None):
    """Partial form: returns (part_o [P,B,Hq,d], part_m [P,B,Hq], part_l [P,B,Hq])."""
    dev = cache.device
    B, hq, D = _need_q(q, cache)
    qc = _DTYPE_CODE.get(q.dtype)
    if qc is None:
        raise TypeError("q must be float32 or bfloat16")
    _need(block_tables, torch.int32, "block_tables", dev)
    _need(seq_lens, torch.int32, "seq_lens", dev, (B,))
    P = decode_partitions(cache, q.dtype, B, hq, block_tables.shape[1], partition_blocks)
    if part is None:
        part = (torch.empty(P, B, hq, D, dtype=torch.float32, device=dev),
                torch.empty(P, B, hq, dtype=torch.float32, device=dev),
                torch.empty(P, B, hq, dtype=torch.float32, device=dev))
    po, pm, pl = part
    _need(po, torch.float32, "part_o", dev, (P, B, hq, D))
    _need(pm, torch.float32, "part_m", dev, (P, B, hq))
    _need(pl, torch.float32, "part_l", dev, (P, B, hq))
    d = cache.desc()
    _check(load().pkv_paged_attn_decode_partial(ctypes.byref(d), _p(q), qc, B, hq,
                                                _p(block_tables), block_tables.shape[1],
                                                _p(seq_lens), float(scale), int(partition_blocks),
                                                _p(po), _p(pm), _p(pl), _stream(dev)),
           "paged_attn_decode_partial")
    return part


def paged_attn_prefill(cache: PagedCache, q, q_pos0, block_table, kv_begin, kv_end, causal=True,
                       scale=0.0, partial=False, out=None, out_lse=None, part=None):
    dev = cache.device
    T, hq, D = _need_q(q, cache, torch.bfloat16)
    _need(block_table, torch.int32, "block_table", dev)
    if block_table.dim() != 1:
        raise ValueError("block_table must be one sequence's table (1-D)")
    if partial:
        if part is None:
            part = (torch.empty(T, hq, D, dtype=torch.float32, device=dev),
                    torch.empty(T, hq, dtype=torch.float32, device=dev),
                    torch.empty(T, hq, dtype=torch.float32, device=dev))
        po, pm, pl = part
        _need(po, torch.float32, "part_o", dev, (T, hq, D))
        _need(pm, torch.float32, "part_m", dev, (T, hq))
        _need(pl, torch.float32, "part_l", dev, (T, hq))
        args = (None, None, _p(po), _p(pm), _p(pl))
    else:
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, "out", dev, (T, hq, D))
        if out_lse is None:
            out_lse = torch.empty(T, hq, dtype=torch.float32, device=dev)
        _need(out_lse, torch.float32, "out_lse", dev, (T, hq))
        args = (_p(out), _p(out_lse), None, None, None)
    d = cache.desc()
    _check(load().pkv_paged_attn_prefill(ctypes.byref(d), _p(q), PKV_BF16, T, hq, int(q_pos0),
                                         _p(block_table), block_table.numel(), int(kv_begin),
                                         int(kv_end), int(bool(causal)), float(scale), *args,
                                         _stream(dev)), "paged_attn_prefill")
    return part if partial else (out, out_lse)


def attn_lse_merge(part_o, part_m, part_l, out_dtype=torch.bfloat16, out=None, with_state=True,
                   out_lse=None):
    """part_o [S, rows..., d] fp32, part_m/part_l [S, rows...]; returns
    (O [rows..., d], M, L, lse)."""
    dev = part_o.device
    _need(part_o, torch.float32, "part_o", dev)
    if part_o.dim() < 3:
        raise ValueError("part_o must be [S, rows..., head_dim]")
    S = part_o.shape[0]
    D = part_o.shape[-1]
    rows_shape = tuple(part_o.shape[1:-1])
    rows = math.prod(rows_shape)
    _need(part_m, torch.float32, "part_m", dev, (S,) + rows_shape)
    _need(part_l, torch.float32, "part_l", dev, (S,) + rows_shape)
    if out is None:
        out = torch.empty(rows_shape + (D,), dtype=out_dtype, device=dev)
    if out.dtype not in _DTYPE_CODE:
        raise TypeError("out must be float32 or bfloat16")
    _need(out, None, "out", dev, rows_shape + (D,))
    m = l = None
    lse = out_lse
    if with_state:
        m = torch.empty(rows_shape, dtype=torch.float32, device=dev)
        l = torch.empty_like(m)
        lse = torch.empty_like(m) if lse is None else lse
    if lse is not None:
        _need(lse, torch.float32, "out_lse", dev, rows_shape)
    _check(load().pkv_attn_lse_merge(S, rows, D, _p(part_o), _p(part_m), _p(part_l), _p(out),
                                     _DTYPE_CODE[out.dtype], _p(m), _p(l), _p(lse), _stream(dev)),
           "attn_lse_merge")
    return out, m, l, lse


def copy_blocks(src: PagedCache, dst: PagedCache, src_ids, dst_ids, stream=None):
    """pkv_copy_blocks: block src_ids[i] of src -> block dst_ids[i] of dst
    (int32 id tensors on the GPU).  `stream` is a torch.cuda.Stream or None
    for the current stream of the ids' device."""
    _need(src_ids, torch.int32, "src_ids")
    _need(dst_ids, torch.int32, "dst_ids", src_ids.device, tuple(src_ids.shape))
    if not src_ids.is_cuda:
        raise ValueError("src_ids / dst_ids must be on the GPU")
    s = c_void_p(stream.cuda_stream) if stream is not None else _stream(src_ids.device)
    ds, dd = src.desc(), dst.desc()
    _check(load().pkv_copy_blocks(ctypes.byref(ds), ctypes.byref(dd), _p(src_ids), _p(dst_ids),
                                  src_ids.numel(), s), "copy_blocks")


def validate_tables(block_tables, seq_lens, num_blocks):
    first_bad = c_int64()
    st = load().pkv_validate_tables(_p(block_tables), _p(seq_lens), block_tables.shape[0],
                                    block_tables.shape[1], num_blocks, ctypes.byref(first_bad),
                                    _stream(block_tables.device))
    if st not in (PKV_OK, PKV_ERR_BAD_TABLE):
        _check(st, "validate_tables")
    return first_bad.value
