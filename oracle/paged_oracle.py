"""Plain fp64 CPU oracle of paged KV attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and never imports it.  Everything here is written for clarity, not speed: it
follows the definitions the pages give, step by step, in float64.

Sources (page title, section):
  * Inside vLLM: Anatomy of a High-Throughput LLM Inference System
    (Gordic; Chinese translation), sections "Engine construction" (per-block
    byte formula), "Scheduler" (allocate_slots, ceil(n/16) blocks) and
    "Forward pass" (slot_mapping; one flattened super-sequence with positions
    and a mask so each sequence sees only its own tokens).
  * vLLM 技术内幕 (openeuler), section 2.1 (16-token blocks, block table as a
    page table, blockwise q.k then blockwise value accumulation) and 2.2
    (ref_cnt and copy-on-write of a shared block on write).
  * Continuous batching + PagedAttention (juhe.plus), section 3.3 (logical
    token -> block index and offset -> physical block), 3.6 (the kernel loop
    over the block table), 3.8 (COW walk-through), 4.2 (chunked prefill).
  * vLLM 源码精读, sections 2.1-2.4 (block_table, slot_mapping, copy-on-write)
    and 5.1 (prepare_attn builds slot_mapping; kernels scatter new K/V and
    gather old K/V through the table).

Readings where the pages are silent (each also listed in the design notes):
  * slot = physical_block * block_size + offset (implied by the 3.3 example).
  * a negative slot means "skip this token" (padding).
  * a sequence's length L counts the tokens written in the current step; the
    step's K/V are written before attention reads them (3.3 order).
  * GQA: query head h reads kv head h // (Hq / Hkv).
  * query i of a sequence with q_len new tokens sits at position
    L - q_len + i and sees keys 0..position (causal).
  * a freed block returns to the head of the free list; a request's blocks are
    returned last-to-first (vLLM 技术内幕 3.1 and 4: tail-to-head return,
    unhashed blocks reused first).

Pool layout (this library's documented ABI; the oracle implements it with
its own index arithmetic):
  pool[num_blocks][num_kv_heads][2 (K, V)][tile], tile = block_size*head_size
  elements.  With E = 16 / dtype_bytes elements per 16-byte granule:
    K tile: element (t, d) at ((d // E) * block_size + t) * E + d % E
    V tile: element (t, d) at ((t // E) * head_size + d) * E + t % E
"""
from __future__ import annotations

import math
from collections import deque

import numpy as np

BLOCK_SIZE = 16

# ----------------------------------------------------------------------------
# element types: codes are the raw stored bit patterns
# ----------------------------------------------------------------------------
_CODE = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}
_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def code_dtype(dtype: str):
    return _CODE[dtype]


def dtype_bytes(dtype: str) -> int:
    return _BYTES[dtype]


def decode(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of stored codes, as float64 (bf16 is the top half of an
    IEEE binary32, so widening is exact)."""
    if dtype == "bf16":
        return (codes.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.ascontiguousarray(codes).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# FP8 KV cache (the pages list an FP8 KV cache that halves its memory at
# nearly no accuracy cost: vLLM 技术内幕 section 7.2; Continuous batching +
# PagedAttention Q&A).  Reading taken here: codes are OCP FP8 E4M3 (1 sign
# bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, exponent
# and mantissa all ones = NaN, largest finite 448); each cache has one K scale
# and one V scale; a stored code c stands for e4m3(c) * scale; a written value
# x becomes the code nearest to x * (1 / scale) (both products in float32,
# ties to the even code), saturated to +-448.
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The number an E4M3 code stands for (NaN for 0x7F and 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:                              # subnormal: man * 2^-3 * 2^(1-7)
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float values -> E4M3 codes: the nearest representable magnitude, ties
    to the even code, magnitudes above 448 saturated to 448, NaN to 0x7F
    (with its sign bit); the sign of zero is kept."""
    y = np.asarray(y, dtype=np.float64)
    mags = e4m3_table()[:0x7F]                # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)  # first >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(mags[hi] == a, hi, pick)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    codes = (pick.astype(np.uint8) | sign)
    return np.where(np.isnan(y), np.uint8(0x7F) | sign, codes).astype(np.uint8)


def fp8_quantize(codes_bf16: np.ndarray, scale: float) -> np.ndarray:
    """bf16 codes -> E4M3 codes of x * (1 / scale), both steps in float32."""
    inv = np.float32(1.0) / np.float32(scale)
    x = (np.asarray(codes_bf16, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    return e4m3_encode((x * inv).astype(np.float32))


# ----------------------------------------------------------------------------
# sizes (Inside vLLM, "Engine construction": 2 * block_size * num_kv_heads *
# head_size * dtype_bytes per block and layer)
# ----------------------------------------------------------------------------
def block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_nbytes: int) -> int:
    return 2 * block_size * num_kv_heads * head_size * dtype_nbytes


def blocks_for_tokens(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Inside vLLM, "Scheduler": n tokens need ceil(n / block_size) blocks."""
    return -(-n_tokens // block_size)


# ----------------------------------------------------------------------------
# pool layout
# ----------------------------------------------------------------------------
def _granule(dtype: str) -> int:
    return 16 // dtype_bytes(dtype)


def k_tile_index(head_size: int, dtype: str, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """[block_size][head_size] -> flat position inside a K tile."""
    E = _granule(dtype)
    t = np.arange(block_size)[:, None]
    d = np.arange(head_size)[None, :]
    return ((d // E) * block_size + t) * E + (d % E)


def v_tile_index(head_size: int, dtype: str, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """[block_size][head_size] -> flat position inside a V tile."""
    E = _granule(dtype)
    t = np.arange(block_size)[:, None]
    d = np.arange(head_size)[None, :]
    return ((t // E) * head_size + d) * E + (t % E)


def new_pool(num_blocks: int, num_kv_heads: int, head_size: int, dtype: str,
             fill_code: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """A pool of codes, every element set to ``fill_code``."""
    return np.full((num_blocks, num_kv_heads, 2, block_size * head_size), fill_code,
                   dtype=code_dtype(dtype))


# ----------------------------------------------------------------------------
# address translation (juhe.plus 3.3: token -> (pos // bs, pos % bs) -> physical)
# ----------------------------------------------------------------------------
def slot_of(table_row, pos: int, block_size: int = BLOCK_SIZE) -> int:
    logical_block, offset = divmod(int(pos), block_size)
    return int(table_row[logical_block]) * block_size + offset


def slot_mapping(block_tables: np.ndarray, query_start_loc: np.ndarray,
                 seq_lens: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Slots of the step's new tokens, in flattened token order (vLLM 源码精读
    5.1: prepare_attn maps every new token's logical position to its slot)."""
    out = []
    for s in range(len(seq_lens)):
        q_len = int(query_start_loc[s + 1] - query_start_loc[s])
        L = int(seq_lens[s])
        for i in range(q_len):
            out.append(slot_of(block_tables[s], L - q_len + i, block_size))
    return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# block allocator with reference counts and copy-on-write
# (Inside vLLM "Scheduler": allocate_slots pops the first n free blocks;
#  vLLM 技术内幕 2.2 and juhe.plus 3.8: writing into a block whose ref_cnt > 1
#  allocates a new block, copies, and drops one reference of the old one)
# ----------------------------------------------------------------------------
class CowPool:
    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK_SIZE):
        self.block_size = block_size
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        self.free = deque(order)
        self.ref = [0] * num_blocks

    def num_free(self) -> int:
        return len(self.free)

    def _pop(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def append(self, table: list, cur_len: int, n_new: int):
        """Make room for n_new tokens after cur_len cached ones.

        ``table`` (a Python list of physical ids, one per logical block) is
        updated in place.  Returns (slots of the new tokens, cow pair or None).
        """
        bs = self.block_size
        have = blocks_for_tokens(cur_len, bs)
        need = blocks_for_tokens(cur_len + n_new, bs)
        assert len(table) == have
        cow = None
        partial = (cur_len % bs) != 0 and n_new > 0
        extra = need - have + (1 if partial and self.ref[table[-1]] > 1 else 0)
        if extra > len(self.free):
            raise MemoryError("pool exhausted")
        if partial and self.ref[table[-1]] > 1:
            old = table[-1]
            new = self._pop()
            self.ref[old] -= 1
            table[-1] = new
            cow = (old, new)
        for _ in range(need - have):
            table.append(self._pop())
        slots = [slot_of(table, cur_len + i, bs) for i in range(n_new)]
        return slots, cow

    def fork(self, table: list) -> list:
        """Another holder of the same blocks (parallel sampling, juhe.plus 3.5)."""
        for b in table:
            self.ref[b] += 1
        return list(table)

    def release(self, table: list) -> None:
        """Drop one reference of each block, last block first; a block whose
        count reaches zero goes to the head of the free list."""
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.appendleft(b)
        table.clear()


# ----------------------------------------------------------------------------
# prefix caching (Inside vLLM "Prefix caching"; vLLM 技术内幕 section 4):
# every full block gets a chained hash of its parent's hash and its token
# ids; a new request walks its full blocks from the first and reuses every
# cached block until the first miss; blocks registered after their KV are
# written; released blocks that still carry a hash go to the tail of the free
# queue (evicted last), others to the head; a hashed block loses its hash when
# it is taken from the head for a new use.  The hash is 64-bit FNV-1a (a
# published function) over the parent hash (8 bytes, little-endian) and the
# block's token ids (4 bytes each, little-endian); a hit also compares the
# stored parent hash and token ids.
# ----------------------------------------------------------------------------
FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_hash(parent: int, tokens) -> int:
    data = int(parent).to_bytes(8, "little") + b"".join(
        int(t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


def prefix_hashes(tokens, block_size: int = BLOCK_SIZE):
    """Chained hashes of the full blocks of a token-id list (parent of the
    first block: 0)."""
    out, parent = [], 0
    for i in range(len(tokens) // block_size):
        parent = block_hash(parent, tokens[i * block_size:(i + 1) * block_size])
        out.append(parent)
    return out


class PrefixCachePool(CowPool):
    """CowPool plus the prefix cache.  The free queue is a list (head first)."""

    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK_SIZE):
        super().__init__(num_blocks, free_order, block_size)
        self.free = list(self.free)
        self.key = [None] * num_blocks      # (hash, parent, tokens) of a cached block
        self.by_hash = {}                   # hash -> block

    def _pop(self) -> int:
        b = self.free.pop(0)
        if self.key[b] is not None:         # evicted from the cache on reuse
            h = self.key[b][0]
            if self.by_hash.get(h) == b:
                del self.by_hash[h]
            self.key[b] = None
        self.ref[b] = 1
        return b

    def release(self, table: list) -> None:
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.key[b] is not None:
                    self.free.append(b)
                else:
                    self.free.insert(0, b)
        table.clear()

    def match_prefix(self, tokens) -> list:
        """Longest run of cached full blocks from the start; each hit gains a
        reference (leaving the free queue if it was there)."""
        bs = self.block_size
        hits, parent = [], 0
        for i in range(len(tokens) // bs):
            blk = [int(t) for t in tokens[i * bs:(i + 1) * bs]]
            h = block_hash(parent, blk)
            b = self.by_hash.get(h)
            if b is None or self.key[b] != (h, parent, tuple(blk)):
                break
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            hits.append(b)
            parent = h
        return hits

    def cache_blocks(self, tokens, table, num_full: int) -> None:
        """Register the first num_full blocks of a sequence (their KV is
        written); a block already cached, or a hash another block holds, is
        left as it is."""
        bs = self.block_size
        parent = 0
        for i in range(num_full):
            blk = tuple(int(t) for t in tokens[i * bs:(i + 1) * bs])
            h = block_hash(parent, blk)
            b = int(table[i])
            if self.key[b] is None and h not in self.by_hash:
                self.key[b] = (h, parent, blk)
                self.by_hash[h] = b
            parent = h


# ----------------------------------------------------------------------------
# the two data movements
# ----------------------------------------------------------------------------
def kv_write(pool: np.ndarray, dtype: str, k_new: np.ndarray, v_new: np.ndarray,
             slots, block_size: int = BLOCK_SIZE, k_scale: float = 1.0,
             v_scale: float = 1.0) -> None:
    """Scatter each new token's K and V rows (all kv heads) to its slot, in
    place (vLLM 技术内幕 2.1: write_to_paged_cache / reshape_and_cache).
    k_new, v_new: codes [T][Hkv][D] of the cache's type, or bf16 codes for an
    FP8 cache, which stores them quantized.  A negative slot is skipped."""
    if dtype == "fp8":
        k_new = fp8_quantize(k_new, k_scale)
        v_new = fp8_quantize(v_new, v_scale)
    D = k_new.shape[2]
    kidx = k_tile_index(D, dtype, block_size)
    vidx = v_tile_index(D, dtype, block_size)
    for t, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        pool[blk, :, 0, kidx[off]] = k_new[t].T   # fancy index is [D][Hkv]
        pool[blk, :, 1, vidx[off]] = v_new[t].T


def block_copy(pool: np.ndarray, pairs) -> None:
    """For every (src, dst): block dst becomes a copy of block src as it was
    before the call (juhe.plus 3.8: copy block 2 into the new block 7)."""
    snapshot = {int(s): pool[int(s)].copy() for s, _ in pairs}
    for s, d in pairs:
        pool[int(d)] = snapshot[int(s)]


def block_swap(dev_pool: np.ndarray, host_pool: np.ndarray, pairs, to_host: bool) -> None:
    """Swap preemption's data move (juhe.plus 3.9; vLLM 源码精读 on swap out
    to CPU memory and back): every (src, dst) pair copies a whole block from
    the device pool to the host pool (to_host) or back.  Reads see the
    contents before the call."""
    src_pool, dst_pool = (dev_pool, host_pool) if to_host else (host_pool, dev_pool)
    snapshot = {int(s): src_pool[int(s)].copy() for s, _ in pairs}
    for s, d in pairs:
        dst_pool[int(d)] = snapshot[int(s)]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def gather_kv(pool: np.ndarray, dtype: str, table_row, L: int, head_size: int,
              block_size: int = BLOCK_SIZE):
    """Codes K, V [L][Hkv][D] of one sequence, walking its block table in
    logical order (juhe.plus 3.6: look up the physical block, read its K/V)."""
    kidx = k_tile_index(head_size, dtype, block_size)
    vidx = v_tile_index(head_size, dtype, block_size)
    Hkv = pool.shape[1]
    K = np.empty((L, Hkv, head_size), dtype=pool.dtype)
    V = np.empty((L, Hkv, head_size), dtype=pool.dtype)
    for j in range(L):
        blk = int(table_row[j // block_size])
        off = j % block_size
        K[j] = pool[blk, :, 0, kidx[off]].T
        V[j] = pool[blk, :, 1, vidx[off]].T
    return K, V


def attention_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale: float) -> np.ndarray:
    """Textbook softmax attention of query rows over one sequence's history.

    q: float64 [n][Hq][D]; K, V: float64 [L][Hkv][D]; positions[i] is the
    absolute position of query row i, which sees keys 0..positions[i].
    Returns float64 [n][Hq][D].
    """
    n, Hq, D = q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    out = np.zeros((n, Hq, D), dtype=np.float64)
    for i in range(n):
        p = int(positions[i])
        for h in range(Hq):
            g = h // group
            x = scale * (K[: p + 1, g, :] @ q[i, h, :])
            w = np.exp(x - x.max())
            out[i, h, :] = (w @ V[: p + 1, g, :]) / w.sum()
    return out


def paged_attention(pool: np.ndarray, dtype: str, q_codes: np.ndarray, block_tables,
                    seq_lens, query_start_loc, scale: float,
                    block_size: int = BLOCK_SIZE, k_scale: float = 1.0,
                    v_scale: float = 1.0) -> np.ndarray:
    """Attention of a flattened batch of query rows over the paged cache.

    q_codes: codes [T][Hq][D] (bf16 for an FP8 cache, whose stored codes
    stand for e4m3 value * k_scale or * v_scale); sequence s owns rows
    query_start_loc[s] .. query_start_loc[s+1]-1 (Inside vLLM "Forward pass":
    one super-sequence, each sequence attending only to its own tokens).
    A sequence of length 0 yields zeros.  Returns float64 [T][Hq][D].
    """
    T, Hq, D = q_codes.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    q = decode(q_codes, "bf16" if dtype == "fp8" else dtype)
    ks, vs = (float(k_scale), float(v_scale)) if dtype == "fp8" else (1.0, 1.0)
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        r0, r1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        if L == 0 or r1 == r0:
            continue
        K, V = gather_kv(pool, dtype, block_tables[s], L, D, block_size)
        positions = [L - (r1 - r0) + i for i in range(r1 - r0)]
        out[r0:r1] = attention_rows(q[r0:r1], decode(K, dtype) * ks, decode(V, dtype) * vs,
                                    positions, scale)
    return out
