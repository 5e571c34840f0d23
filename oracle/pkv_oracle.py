"""CPU oracle for exact softmax attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP library and never imports it.

Plain, slow and obviously correct: numpy, float64 for every floating-point
step, the block table walked block by block, and a two-pass softmax (exact max
first, then exponentials) that deliberately does NOT use the online recurrence,
so the kernels' online softmax and log-sum-exp merge are checked against it
rather than assumed by it.

Pages followed (cited by title and section):

* [P1] "Long-context inference engineering truths 2026: PagedAttention, Ring
  Attention and KV-cache offload from 128K to 1M context" (blog.lonae.com),
  section 2.1 (block_size 16, waste bound), section 2.2 (block-table
  pseudocode: block id = t // block_size, offset = t % block_size, a new block
  is allocated when a token opens one), section 3.1 (online softmax state
  m, l, O and its update).
* [P2] "Unlocking long context: engineering practice and optimisation of
  million-token LLM inference" (www.ybb.press/ai-applications/14576),
  section 3.1 (fixed-size blocks, per-sequence logical block table), section
  3.2 (E4M3 FP8 KV, block-wise scaling of one scale per 64-128 tokens),
  section 4.1 (naive attention: scores q k^T / sqrt(d), softmax, times V),
  section 5.2 (chunked prefill).
* [P3] article at www.mhpn.cn/news/2466452, section 1.1 (attention =
  softmax(Q K^T / sqrt(d)) V), section 1.2 (FlashAttention keeps the flops,
  only avoids writing the n x n matrix), section 3.2 (GQA: several query heads
  share one key/value head).
* [P4] "Sequence-parallel engineering for long-context LLM inference: Ring
  Attention and distributed KV cache" (www.ybb.press/ai-applications/14023),
  section "numerically stable incremental softmax" (per-shard results are
  combined by a max-based log-sum-exp correction).

Readings where the pages are silent or garbled (each one listed in the design doc):

* scale defaults to 1/sqrt(d); scores are S = q K^T with a per-row max;
* partial state = (unnormalised O~, m, l) per query row and head; merge rescales
  by exp(m_i - M) and tracks l (the P4 correction written out with l);
* an allocation happens iff the token's logical block index equals the current
  table length (P1's membership test compares a logical index with physical ids);
* query head h uses kv head h // (Hq / Hkv);
* causal: key t is visible to a query at absolute position p iff t <= p;
* an empty visible set gives O = 0, m = -inf, l = 0, lse = -inf;
* FP8 is OCP E4M3FN (bias 7, max 448, no infinities, S.1111.111 = NaN), encoded
  round-to-nearest-even with saturation at +-448; one fp32 scale per 64-token
  group per kv head, scale = f32(amax / 448) (1 when that is 0 or subnormal),
  stored in every block slot of the group; quantise f32(x) * f32(1 / scale).

Pool layout (one layer): K pool [num_blocks, Hkv, 16, d] (token-major pages),
V pool [num_blocks, Hkv, d, 16] (dimension-major pages).  bf16 pools hold raw
uint16 bit patterns, E4M3 pools raw uint8 codes.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

BLOCK = 16          # tokens per physical block [P1 section 2.1, P2 section 3.1]
FP8_MAX = 448.0     # largest finite OCP E4M3FN magnitude
SCALE_GROUP = 64    # tokens per FP8 scale [P2 section 3.2, lower end of 64-128]


# --------------------------------------------------------------------------
# a0: on-demand block allocation and block tables   [P1 sections 2.1-2.2]
# --------------------------------------------------------------------------
class OutOfBlocks(RuntimeError):
    pass


class SharedBlock(RuntimeError):
    """A growth would write into a partly filled block another table holds."""


class Offloaded(RuntimeError):
    """The block named lives in host memory (it must be paged in first)."""


OFFLOADED = -2      # table entry of a block held in a host slot


class Allocator:
    """Free list of physical blocks handed out on demand.

    Blocks leave the free list from the front, in the given order; released
    blocks return to the back in table order.  A sequence's table grows by one
    block exactly when a token opens a new logical block.

    Prefix sharing [P2 section 3.1: shared-prefix blocks are reused, with
    copy-on-write; P1 section 5: prefix cache]: each block counts the tables
    that hold it and is free again only when none does.  fork() gives a new
    sequence every block of another; publish_prefix() / match_prefix() let a
    new sequence take over the full blocks of an earlier one whose prefix
    hashes (computed by the caller) agree.  A growth that writes into a partly
    filled last block held by another table is refused by reserve(); with
    reserve_cow() the sequence first moves onto a fresh block (taken before the
    growth's own blocks) and the (shared, fresh) pair to copy is returned.

    KV offload [P3 section 4.2: a page table recording, for every block, the
    device it is stored on, whether it is swapped out, and when it was last
    read; pages are brought back ahead of use (prefetch); P1 section 4:
    blocks not needed for a while move to CPU memory]: with host slots set,
    offload() moves a sequence's resident blocks to free host slots (their
    device blocks are freed) and page_in() moves them back to free device
    blocks; both return the (from, to) copy pairs.  Table entries of
    offloaded blocks read OFFLOADED.  The readings: only blocks held by a
    single table move (a shared block is refused); a growth that writes into
    an offloaded last block, and a fork of a sequence with offloaded blocks,
    are refused; offloaded blocks are never published; release returns host
    slots; slots leave from the front of the host free list and return to its
    back, as device blocks do."""

    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.block_size = block_size
        self.free = list(order)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.refs = [0] * num_blocks
        self.by_hash: dict[int, int] = {}
        self.hash_of: dict[int, int] = {}
        self.host_free: list[int] = []
        self.host_slots_set = False
        self.slot_of: dict[int, list[int]] = {}      # per sequence: host slot per block, -1
        self.last: dict[int, list[int]] = {}         # per sequence: last step read, -1

    def _grow(self, seq, new_len, cow):
        table = list(self.tables.get(seq, []))
        old_len = self.lens.get(seq, 0)
        if new_len < old_len:
            raise ValueError("a sequence never shrinks")
        free = list(self.free)
        refs = list(self.refs)
        pair = None
        writes_tail = new_len > old_len and old_len % self.block_size != 0
        if writes_tail and table[-1] == OFFLOADED:
            raise Offloaded(f"sequence {seq} would write into an offloaded block")
        if writes_tail and refs[table[-1]] > 1:
            if not cow:
                raise SharedBlock(f"sequence {seq} would write into shared block {table[-1]}")
            if not free:
                raise OutOfBlocks(f"no free block to copy block {table[-1]} into")
            fresh = free.pop(0)
            refs[fresh] = 1
            refs[table[-1]] -= 1
            pair = (table[-1], fresh)
            table[-1] = fresh
        for t in range(old_len, new_len):
            block_id = t // self.block_size
            if block_id == len(table):           # token t opens a new logical block
                if not free:                     # all-or-nothing: nothing changes
                    raise OutOfBlocks(f"no free block for sequence {seq} token {t}")
                b = free.pop(0)
                refs[b] = 1
                table.append(b)
        self.free, self.refs = free, refs
        added = len(table) - len(self.tables.get(seq, []))
        self.slot_of[seq] = self.slot_of.get(seq, []) + [-1] * added
        self.last[seq] = self.last.get(seq, []) + [-1] * added
        self.tables[seq] = table
        self.lens[seq] = new_len
        return list(table), pair

    def reserve(self, seq: int, new_len: int) -> list[int]:
        return self._grow(seq, new_len, cow=False)[0]

    def reserve_cow(self, seq: int, new_len: int):
        """(table, (shared block, fresh block) to copy, or None)."""
        return self._grow(seq, new_len, cow=True)

    def fork(self, src: int, dst: int) -> None:
        if src == dst or src not in self.tables or dst in self.tables:
            raise ValueError("fork needs an existing source and a new destination")
        if OFFLOADED in self.tables[src]:
            raise Offloaded("host slots are not shared")
        self.tables[dst] = list(self.tables[src])
        self.slot_of[dst] = [-1] * len(self.tables[src])
        self.last[dst] = [-1] * len(self.tables[src])
        self.lens[dst] = self.lens[src]
        for b in self.tables[dst]:
            self.refs[b] += 1

    def publish_prefix(self, seq: int, block_hashes) -> None:
        if seq not in self.tables:
            if len(block_hashes):
                raise ValueError("unknown sequence")
            return
        if len(block_hashes) * self.block_size > self.lens[seq]:
            raise ValueError("only full blocks can be published")
        for j, h in enumerate(block_hashes):
            b = self.tables[seq][j]
            if b == OFFLOADED:
                continue                          # in host memory: not shareable
            if int(h) in self.by_hash or b in self.hash_of:
                continue                          # the first entry stays
            self.by_hash[int(h)] = b
            self.hash_of[b] = int(h)

    def match_prefix(self, seq: int, block_hashes) -> int:
        if seq in self.tables and (self.lens[seq] or self.tables[seq]):
            raise ValueError("prefix matching needs a new sequence")
        table = []
        for h in block_hashes:
            b = self.by_hash.get(int(h))
            if b is None:
                break
            self.refs[b] += 1
            table.append(b)
        self.tables[seq] = table
        self.slot_of[seq] = [-1] * len(table)
        self.last[seq] = [-1] * len(table)
        self.lens[seq] = len(table) * self.block_size
        return len(table)

    def refcount(self, block: int) -> int:
        return self.refs[block]

    def release(self, seq: int) -> None:
        slots = self.slot_of.pop(seq, [])
        self.last.pop(seq, None)
        for j, b in enumerate(self.tables.pop(seq, [])):
            if b == OFFLOADED:
                self.host_free.append(slots[j])
                continue
            self.refs[b] -= 1
            if self.refs[b] == 0:
                h = self.hash_of.pop(b, None)
                if h is not None:
                    del self.by_hash[h]
                self.free.append(b)
        self.lens.pop(seq, None)

    def waste_slots(self, seq: int) -> int:
        return len(self.tables.get(seq, [])) * self.block_size - self.lens.get(seq, 0)

    def free_count(self) -> int:
        return len(self.free)

    # ---- host tier ---------------------------------------------------------
    def set_host_slots(self, n: int) -> None:
        if self.host_slots_set or n < 0:
            raise ValueError("host slots are set once")
        self.host_slots_set = True
        self.host_free = list(range(n))

    def _range(self, seq, first, count):
        if seq not in self.tables or first < 0 or count < 0:
            raise ValueError("unknown sequence or bad range")
        n = len(self.tables[seq])
        return range(min(first, n), min(first + count, n))

    def offload(self, seq: int, first: int, count: int):
        """Move the resident blocks among [first, first + count) to host
        slots; returns [(device block, host slot)] in block order."""
        table = self.tables[seq] if seq in self.tables else None
        js = [j for j in self._range(seq, first, count) if table[j] != OFFLOADED]
        if any(self.refs[table[j]] > 1 for j in js):
            raise SharedBlock("a shared block stays on the device")
        if len(js) > len(self.host_free):
            raise OutOfBlocks("not enough free host slots")
        pairs = []
        for j in js:
            slot = self.host_free.pop(0)
            b = table[j]
            pairs.append((b, slot))
            self.refs[b] -= 1                    # held by this table only: now free
            h = self.hash_of.pop(b, None)
            if h is not None:
                del self.by_hash[h]
            self.free.append(b)
            table[j] = OFFLOADED
            self.slot_of[seq][j] = slot
        return pairs

    def page_in(self, seq: int, first: int, count: int):
        """Bring the offloaded blocks among [first, first + count) back to
        free device blocks; returns [(host slot, device block)]."""
        js = [j for j in self._range(seq, first, count) if self.tables[seq][j] == OFFLOADED]
        if len(js) > len(self.free):
            raise OutOfBlocks("not enough free device blocks")
        pairs = []
        for j in js:
            b = self.free.pop(0)
            self.refs[b] = 1
            slot = self.slot_of[seq][j]
            pairs.append((slot, b))
            self.host_free.append(slot)
            self.tables[seq][j] = b
            self.slot_of[seq][j] = -1
        return pairs

    def touch(self, seq: int, first: int, count: int, step: int) -> None:
        for j in self._range(seq, first, count):
            self.last[seq][j] = int(step)

    def block_state(self, seq: int, j: int):
        """(device block or OFFLOADED, host slot or -1, last step read or -1)."""
        return self.tables[seq][j], self.slot_of[seq][j], self.last[seq][j]

    def table(self, seq: int) -> list[int]:
        return list(self.tables.get(seq, []))

    def host_free_count(self) -> int:
        return len(self.host_free)

    def coldest(self, max_n: int):
        """Offload candidates, least recently read first (ties by sequence,
        then block): resident full blocks held by one table only."""
        cand = []
        for seq, table in self.tables.items():
            for j in range(min(self.lens[seq] // self.block_size, len(table))):
                b = table[j]
                if b != OFFLOADED and self.refs[b] == 1:
                    cand.append((self.last[seq][j], seq, j))
        cand.sort()
        return [(seq, j) for _, seq, j in cand[:max_n]]


def build_tables(seq_lens, num_blocks, free_order=None, max_blocks=None):
    """Reserve every sequence in order; return (tables int32 [B, maxb] padded
    with -1, waste slots per sequence)."""
    alloc = Allocator(num_blocks, free_order)
    rows = [alloc.reserve(b, int(n)) for b, n in enumerate(seq_lens)]
    maxb = max([len(r) for r in rows] + [0]) if max_blocks is None else max_blocks
    tables = np.full((len(seq_lens), max(maxb, 1)), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        tables[b, :len(r)] = r
    return tables, [alloc.waste_slots(b) for b in range(len(seq_lens))]


# --------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN code: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no inf."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# non-negative finite grid: codes 0x00..0x7E, increasing in value
_POS_GRID = E4M3_TABLE[:0x7F]


def e4m3_encode(x) -> np.ndarray:
    """float32 -> E4M3 code, round to nearest with ties to the even code
    (even mantissa), magnitudes beyond 448 saturate to 448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a_sat = np.minimum(a, FP8_MAX)
    hi = np.searchsorted(_POS_GRID, a_sat, side="left")        # first grid value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - _POS_GRID[lo]
    d_hi = _POS_GRID[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a_sat == _POS_GRID[hi], hi, code).astype(np.uint8)   # exact hit
    code = code | sign
    code = np.where(np.isnan(a), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


# --------------------------------------------------------------------------
# FP8 block-wise scales   [P2 section 3.2]
# --------------------------------------------------------------------------
def group_scale(amax) -> np.ndarray:
    """fp32 scale for a group whose largest magnitude is ``amax``."""
    amax = f32(amax)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = f32(amax / np.float32(FP8_MAX))
    tiny = np.finfo(np.float32).tiny
    return np.where(s >= tiny, s, np.float32(1.0)).astype(np.float32)


def fp8_group_scales(src, pos0: int, table_row, scale_pool, group: int = SCALE_GROUP):
    """Scales for one sequence's tokens [pos0, pos0 + n), src [n, Hkv, d]
    (float32 values).  Groups are aligned to token 0; a group's scale comes from
    the given tokens of it, and every block of the group's whole span that the
    table names (entries at or past its end, and entries -1, are skipped)
    receives it in scale_pool[block, kv_head].  So a partial group of a
    decode stream fixes the scale of blocks the table does not hold yet only
    when they are named (the streaming reading)."""
    src = f32(src)
    n, hkv, _ = src.shape
    if pos0 % group:
        raise ValueError("pos0 must start a scale group")
    table_row = np.asarray(table_row)
    for g0 in range(0, n, group):
        rows = src[g0:g0 + group]
        amax = np.abs(rows).max(axis=(0, 2))                  # per kv head
        s = group_scale(amax)
        first_tok = pos0 + g0
        for j in range(first_tok // BLOCK, (first_tok + group - 1) // BLOCK + 1):
            if j < len(table_row) and 0 <= int(table_row[j]) < scale_pool.shape[0]:
                scale_pool[int(table_row[j]), :] = s
    return scale_pool


# --------------------------------------------------------------------------
# a1: append into pool slots through the block table   [P1 section 2.2]
# --------------------------------------------------------------------------
@dataclass
class Cache:
    k: np.ndarray            # [num_blocks, Hkv, 16, d]  (f32 | uint16 bf16 bits | uint8 e4m3)
    v: np.ndarray            # [num_blocks, Hkv, d, 16]
    fmt: str                 # "f32" | "bf16" | "e4m3"
    k_scale: np.ndarray | None = None   # [num_blocks, Hkv] float32 (e4m3)
    v_scale: np.ndarray | None = None

    @property
    def num_blocks(self):
        return self.k.shape[0]

    @property
    def hkv(self):
        return self.k.shape[1]

    @property
    def head_dim(self):
        return self.k.shape[3]


def new_cache(num_blocks, hkv, d, fmt, fill=None) -> Cache:
    dt = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[fmt]
    k = np.zeros((num_blocks, hkv, BLOCK, d), dtype=dt)
    v = np.zeros((num_blocks, hkv, d, BLOCK), dtype=dt)
    if fill is not None:
        k[...] = fill
        v[...] = fill
    ks = vs = None
    if fmt == "e4m3":
        ks = np.ones((num_blocks, hkv), dtype=np.float32)
        vs = np.ones((num_blocks, hkv), dtype=np.float32)
    return Cache(k, v, fmt, ks, vs)


def append(cache: Cache, k_new, v_new, seq_idx, pos, tables) -> Cache:
    """Write token i's K/V ([T, Hkv, d]) into slot pos[i] % 16 of physical block
    tables[seq_idx[i]][pos[i] // 16].

    f32 / bf16 caches: a plain copy of the given elements (bf16 passed as uint16
    bits).  E4M3 cache: k_new / v_new are the float32 source values and each is
    encoded as E4M3(f32(x) * f32(1 / scale)) with the scale of its block."""
    for i in range(len(seq_idx)):
        b, p = int(seq_idx[i]), int(pos[i])
        blk = int(tables[b][p // BLOCK])
        off = p % BLOCK
        if blk < 0:
            raise IndexError(f"token {i} has no block")
        if cache.fmt == "e4m3":
            inv_k = f32(np.float32(1.0) / cache.k_scale[blk])      # [Hkv]
            inv_v = f32(np.float32(1.0) / cache.v_scale[blk])
            cache.k[blk, :, off, :] = e4m3_encode(f32(f32(k_new[i]) * inv_k[:, None]))
            cache.v[blk, :, :, off] = e4m3_encode(f32(f32(v_new[i]) * inv_v[:, None]))
        else:
            cache.k[blk, :, off, :] = k_new[i]
            cache.v[blk, :, :, off] = v_new[i]
    return cache


def append_sequence(cache: Cache, k_seq, v_seq, table_row, pos0: int = 0, heads=None,
                    chunk: int = 4096) -> Cache:
    """Write one sequence's contiguous tokens [pos0, pos0 + n) (k_seq, v_seq
    [n, Hkv, d], element bits for f32 / bf16 caches, float32 values for E4M3)
    block by block.  Same result as append() token by token; ``heads``
    restricts the kv heads written."""
    n = k_seq.shape[0]
    heads = range(cache.hkv) if heads is None else list(heads)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        toks = pos0 + np.arange(c0, c1)
        blocks = np.asarray(table_row)[toks // BLOCK]
        for h in heads:
            kx = np.asarray(k_seq[c0:c1, h, :])
            vx = np.asarray(v_seq[c0:c1, h, :])
            if cache.fmt == "e4m3":
                inv_k = f32(np.float32(1.0) / cache.k_scale[blocks, h])
                inv_v = f32(np.float32(1.0) / cache.v_scale[blocks, h])
                kx = e4m3_encode(f32(f32(kx) * inv_k[:, None]))
                vx = e4m3_encode(f32(f32(vx) * inv_v[:, None]))
            i = 0
            while i < c1 - c0:
                t = int(toks[i])
                off = t % BLOCK
                cnt = min(BLOCK - off, c1 - c0 - i)
                blk = int(blocks[i])
                cache.k[blk, h, off:off + cnt, :] = kx[i:i + cnt]
                cache.v[blk, h, :, off:off + cnt] = vx[i:i + cnt].T
                i += cnt
    return cache


def copy_blocks(src: Cache, dst: Cache, src_ids, dst_ids) -> Cache:
    """Block dst_ids[i] of dst takes every page of block src_ids[i] of src (and
    its E4M3 scales): the copy of copy-on-write [P2 section 3.1] and of moving
    blocks between memory tiers [P1 section 4].  Pairs naming a block outside
    its pool are skipped.  Pages are copied whole, whatever their inner order."""
    for sb, db in zip(np.asarray(src_ids).tolist(), np.asarray(dst_ids).tolist()):
        if not (0 <= sb < src.num_blocks and 0 <= db < dst.num_blocks):
            continue
        dst.k[db] = src.k[sb]
        dst.v[db] = src.v[sb]
        if src.fmt == "e4m3":
            dst.k_scale[db] = src.k_scale[sb]
            dst.v_scale[db] = src.v_scale[sb]
    return dst


# --------------------------------------------------------------------------
# a2: walk the block table; dequantise   [P1 2.2, P2 3.1, P2 3.2]
# --------------------------------------------------------------------------
def _elements_to_f64(x, fmt):
    if fmt == "f32":
        return np.asarray(x, dtype=np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(x)
    return e4m3_decode(x)


def gather_kv(cache: Cache, table_row, n_tokens: int, kv_head: int):
    """Logical K, V [n_tokens, d] in float64 for one sequence and kv head,
    read one block at a time through the table."""
    d = cache.head_dim
    K = np.zeros((n_tokens, d), dtype=np.float64)
    V = np.zeros((n_tokens, d), dtype=np.float64)
    for j in range(-(-n_tokens // BLOCK)):
        blk = int(table_row[j])
        t0 = j * BLOCK
        cnt = min(BLOCK, n_tokens - t0)
        kb = _elements_to_f64(cache.k[blk, kv_head, :cnt, :], cache.fmt)
        vb = _elements_to_f64(cache.v[blk, kv_head, :, :cnt], cache.fmt).T
        if cache.fmt == "e4m3":
            kb = kb * float(cache.k_scale[blk, kv_head])
            vb = vb * float(cache.v_scale[blk, kv_head])
        K[t0:t0 + cnt] = kb
        V[t0:t0 + cnt] = vb
    return K, V


# --------------------------------------------------------------------------
# a3-a6: exact attention, two-pass softmax   [P2 4.1, P3 1.1, P3 3.2]
# --------------------------------------------------------------------------
def attend(q_rows, K, V, visible, scale):
    """q_rows [R, d], K/V [n, d], visible bool [R, n].

    Returns O [R, d] (normalised), O~ [R, d] (unnormalised), m, l, lse [R]."""
    R = q_rows.shape[0]
    d = V.shape[1]
    s = scale * (q_rows @ K.T)                                   # [R, n]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(R, -np.inf)
    empty = ~np.isfinite(m)
    w = np.where(visible, np.exp(s - np.where(empty, 0.0, m)[:, None]), 0.0)
    l = w.sum(axis=1)
    O_un = w @ V if s.shape[1] else np.zeros((R, d))
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(empty[:, None], 0.0, O_un / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    m = np.where(empty, -np.inf, m)
    l = np.where(empty, 0.0, l)
    return O, np.where(empty[:, None], 0.0, O_un), m, l, lse


def _q_f64(q, fmt):
    return bf16_bits_to_f64(q) if fmt == "bf16" else np.asarray(q, dtype=np.float64)


def decode(cache: Cache, q, q_fmt, tables, seq_lens, scale=None, kv_heads=None):
    """One query per sequence (the newest token, already appended) attends to
    all seq_lens[b] keys.  q [B, Hq, d].  Returns dict of float64 arrays
    o [B,Hq,d], o_un, m, l, lse [B,Hq]; ``kv_heads`` restricts the work to the
    query heads of those kv heads (the other rows stay 0)."""
    q = _q_f64(q, q_fmt)
    B, Hq, d = q.shape
    G = Hq // cache.hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = {k: np.zeros((B, Hq, d)) for k in ("o", "o_un")}
    out.update({k: np.zeros((B, Hq)) for k in ("m", "l", "lse")})
    for b in range(B):
        n = int(seq_lens[b])
        for g in (range(cache.hkv) if kv_heads is None else kv_heads):
            K, V = gather_kv(cache, tables[b], n, g)
            heads = slice(g * G, (g + 1) * G)
            vis = np.ones((G, n), dtype=bool)
            O, Ou, m, l, lse = attend(q[b, heads], K, V, vis, scale)
            out["o"][b, heads], out["o_un"][b, heads] = O, Ou
            out["m"][b, heads], out["l"][b, heads], out["lse"][b, heads] = m, l, lse
    return out


def prefill(cache: Cache, q, q_fmt, q_pos0, table_row, kv_begin, kv_end, causal=True,
            scale=None, rows=None):
    """Queries q [T, Hq, d] of one sequence at absolute positions q_pos0 + r
    attend to keys in [kv_begin, kv_end) (and t <= position when causal).
    ``rows`` optionally restricts to a subset of query rows.  Returns dict of
    float64 arrays o [R,Hq,d], o_un, m, l, lse [R,Hq]."""
    q = _q_f64(q, q_fmt)
    T, Hq, d = q.shape
    G = Hq // cache.hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    R = len(rows)
    qpos = q_pos0 + rows
    n = max(int(kv_end), 0)
    out = {k: np.zeros((R, Hq, d)) for k in ("o", "o_un")}
    out.update({k: np.zeros((R, Hq)) for k in ("m", "l", "lse")})
    t = np.arange(n)
    vis = (t[None, :] >= kv_begin) & (t[None, :] < kv_end)
    if causal:
        vis = vis & (t[None, :] <= qpos[:, None])
    vis = np.broadcast_to(vis, (R, n))
    for g in range(cache.hkv):
        K, V = gather_kv(cache, table_row, n, g)
        for h in range(g * G, (g + 1) * G):
            O, Ou, m, l, lse = attend(q[rows, h], K, V, vis, scale)
            out["o"][:, h], out["o_un"][:, h] = O, Ou
            out["m"][:, h], out["l"][:, h], out["lse"][:, h] = m, l, lse
    return out


# --------------------------------------------------------------------------
# a5 / a7: exact merge of KV-shard partials   [P4 incremental softmax, P1 3.1]
# --------------------------------------------------------------------------
def lse_merge(parts):
    """parts: list of (O~ [..., d], m [...], l [...]) float64 partial states
    over disjoint key sets.  Returns (O normalised, M, L) for the union; a
    part with l == 0 (no visible keys) contributes nothing."""
    def live(m, l):          # a part that saw at least one key
        return np.isfinite(m) & (l > 0)

    ms = np.stack([np.where(live(np.asarray(p[1], np.float64), np.asarray(p[2], np.float64)),
                            np.asarray(p[1], np.float64), -np.inf) for p in parts])
    M = ms.max(axis=0)
    empty = ~np.isfinite(M)
    Msafe = np.where(empty, 0.0, M)
    L = np.zeros_like(M)
    Osum = np.zeros_like(np.asarray(parts[0][0], dtype=np.float64))
    for Ou, m, l in parts:
        m = np.asarray(m, dtype=np.float64)
        l = np.asarray(l, dtype=np.float64)
        ok = live(m, l)
        alpha = np.where(ok, np.exp(np.where(ok, m, 0.0) - Msafe), 0.0)
        L = L + alpha * np.where(ok, l, 0.0)
        # select, never multiply: an empty part's O~ may hold anything
        Osum = Osum + np.where(ok[..., None], alpha[..., None] * np.asarray(Ou, np.float64), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where((L > 0)[..., None], Osum / np.where(L > 0, L, 1.0)[..., None], 0.0)
    return O, np.where(empty, -np.inf, M), L


def lse_of(m, l):
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
