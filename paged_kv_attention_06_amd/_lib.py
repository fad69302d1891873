"""ctypes binding of libpkv.so: argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/pkv.h) and converts torch tensors / numpy arrays to pointers.  All
computation happens in the library's HIP kernels or its C++ host code; if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2
STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_DIM", 3: "PKV_ERR_DTYPE",
          4: "PKV_ERR_WORKSPACE", 5: "PKV_ERR_HIP", 6: "PKV_ERR_NOMEM", 7: "PKV_ERR_RANGE"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
_lib = ctypes.CDLL(LIB_PATH)

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class PkvCache(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c = {}
_c["pkv_status_string"] = _sig("pkv_status_string", ctypes.c_char_p, [ctypes.c_int])
_c["pkv_last_error"] = _sig("pkv_last_error", ctypes.c_char_p, [])
_c["pkv_version"] = _sig("pkv_version", ctypes.c_int, [])
_c["pkv_block_bytes"] = _sig("pkv_block_bytes", ctypes.c_size_t, [ctypes.POINTER(PkvCache)])
_c["pkv_build_slot_mapping"] = _sig("pkv_build_slot_mapping", ctypes.c_int,
                                    [_i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
                                     ctypes.c_int32, _i64p])
_c["paged_kv_write"] = _sig("paged_kv_write", ctypes.c_int,
                            [ctypes.POINTER(PkvCache), _vp, _vp, _vp, ctypes.c_int64, _vp])
_c["block_copy"] = _sig("block_copy", ctypes.c_int,
                        [ctypes.POINTER(PkvCache), _vp, ctypes.c_int64, _vp])
_c["block_swap"] = _sig("block_swap", ctypes.c_int,
                        [ctypes.POINTER(PkvCache), _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                         ctypes.c_int32, _vp])
_c["pkv_attention_workspace_bytes"] = _sig("pkv_attention_workspace_bytes", ctypes.c_size_t,
                                           [ctypes.POINTER(PkvCache), ctypes.c_int32, _i32p,
                                            _i32p, ctypes.c_int32])
_c["paged_attention_decode"] = _sig("paged_attention_decode", ctypes.c_int,
                                    [ctypes.POINTER(PkvCache), _vp, _vp, ctypes.c_int32, _vp,
                                     ctypes.c_int32, _vp, _i32p, ctypes.c_int32, ctypes.c_float,
                                     _vp, ctypes.c_size_t, _vp])
_c["paged_attention_mixed"] = _sig("paged_attention_mixed", ctypes.c_int,
                                   [ctypes.POINTER(PkvCache), _vp, _vp, ctypes.c_int32, _vp, _vp,
                                    _i32p, _i32p, _vp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int64, ctypes.c_float, _vp, ctypes.c_size_t, _vp])
_c["pkv_pool_create"] = _sig("pkv_pool_create", _vp, [ctypes.c_int64, _i32p, ctypes.c_int32])
_c["pkv_pool_destroy"] = _sig("pkv_pool_destroy", None, [_vp])
_c["pkv_pool_num_free"] = _sig("pkv_pool_num_free", ctypes.c_int64, [_vp])
_c["pkv_pool_refcnt"] = _sig("pkv_pool_refcnt", ctypes.c_int32, [_vp, ctypes.c_int32])
_c["pkv_pool_append"] = _sig("pkv_pool_append", ctypes.c_int,
                             [_vp, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i64p, _i64p])
_c["pkv_pool_fork"] = _sig("pkv_pool_fork", ctypes.c_int, [_vp, _i32p, ctypes.c_int32, _i32p])
_c["pkv_pool_release"] = _sig("pkv_pool_release", ctypes.c_int, [_vp, _i32p, ctypes.c_int32])
_c["pkv_block_hash"] = _sig("pkv_block_hash", ctypes.c_uint64, [ctypes.c_uint64, _i32p, ctypes.c_int32])
_c["pkv_pool_match_prefix"] = _sig("pkv_pool_match_prefix", ctypes.c_int,
                                   [_vp, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p])
_c["pkv_pool_cache_blocks"] = _sig("pkv_pool_cache_blocks", ctypes.c_int,
                                   [_vp, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32])

_c["paged_attention_decode_noalloc"] = _sig("paged_attention_decode_noalloc", ctypes.c_int,
                                            [ctypes.POINTER(PkvCache), _vp, _vp, ctypes.c_int32,
                                             _vp, ctypes.c_int32, _vp, _i32p, ctypes.c_int32,
                                             ctypes.c_float, _vp])
_c["pkv_read_slices"] = _sig("pkv_read_slices", ctypes.c_int,
                             [ctypes.POINTER(PkvCache), _vp, ctypes.c_int64, ctypes.c_int32, _vp,
                              _vp])
_c["pkv_layout"] = _sig("pkv_layout", ctypes.c_int, [])
_c["pkv_validate_slots"] = _sig("pkv_validate_slots", ctypes.c_int,
                                [ctypes.POINTER(PkvCache), _i64p, ctypes.c_int64])
_c["pkv_validate_block_pairs"] = _sig("pkv_validate_block_pairs", ctypes.c_int,
                                      [_i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int32])
_c["pkv_validate_attention"] = _sig("pkv_validate_attention", ctypes.c_int,
                                    [ctypes.POINTER(PkvCache), _i32p, ctypes.c_int32, _i32p,
                                     _i32p, _i32p, _i32p, ctypes.c_int32])

EXPORTED = tuple(_c)
PKV_LAYOUT_HEAD_KV_GRANULE16 = 1


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _c["pkv_last_error"]().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PkvError(status, where)


# ----------------------------------------------------------------- helpers
def _host_i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


def _ptr_i64(a: np.ndarray):
    return a.ctypes.data_as(_i64p)


def _dev(t, what: str):
    """Device pointer of a contiguous CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def version() -> int:
    return _c["pkv_version"]()


def pkv_layout() -> int:
    return _c["pkv_layout"]()


def _opt_i32(a):
    return None if a is None else _ptr_i32(a)


def pkv_validate_slots(desc: PkvCache, slots) -> None:
    """Raises PkvError unless the host slots meet paged_kv_write's preconditions."""
    s = np.ascontiguousarray(slots, dtype=np.int64)
    _check(_c["pkv_validate_slots"](ctypes.byref(desc), _ptr_i64(s), s.shape[0]),
           "pkv_validate_slots")


def pkv_validate_block_pairs(pairs, num_src_blocks: int, num_dst_blocks: int,
                             same_pool: bool) -> None:
    p = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    _check(_c["pkv_validate_block_pairs"](_ptr_i64(p), p.shape[0], num_src_blocks,
                                          num_dst_blocks, int(same_pool)),
           "pkv_validate_block_pairs")


def pkv_validate_attention(desc: PkvCache, block_tables, seq_lens, h_seq_lens=None,
                           query_start_loc=None, h_query_start_loc=None) -> None:
    bt = _host_i32(block_tables)
    sl = _host_i32(seq_lens)
    hsl = None if h_seq_lens is None else _host_i32(h_seq_lens)
    qsl = None if query_start_loc is None else _host_i32(query_start_loc)
    hqsl = None if h_query_start_loc is None else _host_i32(h_query_start_loc)
    _check(_c["pkv_validate_attention"](ctypes.byref(desc), _ptr_i32(bt),
                                        bt.shape[1] if bt.ndim == 2 else 0, _ptr_i32(sl),
                                        _opt_i32(hsl), _opt_i32(qsl), _opt_i32(hqsl),
                                        sl.shape[0]), "pkv_validate_attention")


def status_string(status: int) -> str:
    return _c["pkv_status_string"](status).decode()


# ----------------------------------------------------------------- the cache
class Cache:
    """Descriptor of a KV pool living in a torch tensor of raw bytes."""

    def __init__(self, kv, num_blocks: int, num_kv_heads: int, head_size: int, dtype: int,
                 block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0):
        self.kv = kv
        self.desc = PkvCache(kv.data_ptr() if kv is not None else 0, num_blocks, block_size,
                             num_kv_heads, head_size, dtype, k_scale, v_scale)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def descriptor(num_blocks, num_kv_heads, head_size, dtype, block_size=16, kv_ptr=0,
               k_scale=1.0, v_scale=1.0) -> PkvCache:
    return PkvCache(kv_ptr, num_blocks, block_size, num_kv_heads, head_size, dtype, k_scale,
                    v_scale)


def pkv_block_bytes(desc: PkvCache) -> int:
    return _c["pkv_block_bytes"](ctypes.byref(desc))


def pkv_build_slot_mapping(block_tables, query_start_loc, seq_lens) -> np.ndarray:
    bt = _host_i32(block_tables)
    qsl = _host_i32(query_start_loc)
    sl = _host_i32(seq_lens)
    n = int(qsl[-1]) if qsl.size else 0
    out = np.empty(n, np.int64)
    _check(_c["pkv_build_slot_mapping"](_ptr_i32(bt), bt.shape[1] if bt.ndim == 2 else 0,
                                         _ptr_i32(qsl), _ptr_i32(sl), sl.shape[0], 16,
                                         _ptr_i64(out)), "pkv_build_slot_mapping")
    return out


def paged_kv_write(cache: Cache, k_new, v_new, slot_mapping, stream=None) -> None:
    T = int(slot_mapping.shape[0])
    _check(_c["paged_kv_write"](cache.ref, _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev(slot_mapping, "slot_mapping"), T, _stream(stream)),
           "paged_kv_write")


def block_copy(cache: Cache, pairs, stream=None) -> None:
    n = int(pairs.shape[0])
    _check(_c["block_copy"](cache.ref, _dev(pairs, "pairs"), n, _stream(stream)), "block_copy")


PKV_SWAP_OUT = 0
PKV_SWAP_IN = 1


def block_swap(cache: Cache, host_kv, pairs, to_host: bool, stream=None) -> None:
    """host_kv: a pinned CPU torch tensor of whole blocks (uint8)."""
    n = int(pairs.shape[0])
    nb = host_kv.numel() * host_kv.element_size() // pkv_block_bytes(cache.desc)
    _check(_c["block_swap"](cache.ref, ctypes.c_void_p(host_kv.data_ptr()), nb,
                            _dev(pairs, "pairs"), n, PKV_SWAP_OUT if to_host else PKV_SWAP_IN,
                            _stream(stream)), "block_swap")


def pkv_attention_workspace_bytes(cache: Cache, num_q_heads: int, h_seq_lens,
                                  h_query_start_loc=None) -> int:
    sl = _host_i32(h_seq_lens)
    qsl = None if h_query_start_loc is None else _host_i32(h_query_start_loc)
    return _c["pkv_attention_workspace_bytes"](cache.ref, num_q_heads,
                                               None if qsl is None else _ptr_i32(qsl),
                                               _ptr_i32(sl), sl.shape[0])


def paged_attention_decode(cache: Cache, out, q, block_tables, seq_lens, h_seq_lens, scale: float,
                           workspace, stream=None) -> None:
    hsl = _host_i32(h_seq_lens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_c["paged_attention_decode"](cache.ref, _dev(out, "out"), _dev(q, "q"), int(q.shape[1]),
                                        _dev(block_tables, "block_tables"),
                                        int(block_tables.shape[1]), _dev(seq_lens, "seq_lens"),
                                        _ptr_i32(hsl), hsl.shape[0], float(scale),
                                        _dev(workspace, "workspace"), ws_bytes, _stream(stream)),
           "paged_attention_decode")


def pkv_read_slices(cache: Cache, slices, waves: int, sink, stream=None) -> None:
    """slices: int64 GPU tensor of block * num_kv_heads + kv head; sink: int32
    GPU tensor of `waves` entries (the XOR of each wave's words)."""
    _check(_c["pkv_read_slices"](cache.ref, _dev(slices, "slices"), int(slices.shape[0]),
                                 int(waves), _dev(sink, "sink"), _stream(stream)),
           "pkv_read_slices")


def paged_attention_decode_noalloc(cache: Cache, out, q, block_tables, seq_lens, h_seq_lens,
                                   scale: float, stream=None) -> None:
    hsl = _host_i32(h_seq_lens)
    _check(_c["paged_attention_decode_noalloc"](cache.ref, _dev(out, "out"), _dev(q, "q"),
                                                int(q.shape[1]),
                                                _dev(block_tables, "block_tables"),
                                                int(block_tables.shape[1]),
                                                _dev(seq_lens, "seq_lens"), _ptr_i32(hsl),
                                                hsl.shape[0], float(scale), _stream(stream)),
           "paged_attention_decode_noalloc")


def paged_attention_mixed(cache: Cache, out, q, query_start_loc, seq_lens, h_query_start_loc,
                          h_seq_lens, block_tables, scale: float, workspace, stream=None) -> None:
    hsl = _host_i32(h_seq_lens)
    hqsl = _host_i32(h_query_start_loc)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_c["paged_attention_mixed"](cache.ref, _dev(out, "out"), _dev(q, "q"), int(q.shape[1]),
                                       _dev(query_start_loc, "query_start_loc"),
                                       _dev(seq_lens, "seq_lens"), _ptr_i32(hqsl), _ptr_i32(hsl),
                                       _dev(block_tables, "block_tables"),
                                       int(block_tables.shape[1]), hsl.shape[0],
                                       int(q.shape[0]), float(scale),
                                       _dev(workspace, "workspace"), ws_bytes, _stream(stream)),
           "paged_attention_mixed")


# ----------------------------------------------------------------- allocator
class Pool:
    """Host block allocator (pkv_pool_*).  Tables are numpy int32 arrays."""

    def __init__(self, num_blocks: int, free_order=None, block_size: int = 16):
        order = None if free_order is None else _host_i32(free_order)
        self._keep = order
        h = _c["pkv_pool_create"](num_blocks, None if order is None else _ptr_i32(order), block_size)
        if not h:
            raise PkvError(2, "pkv_pool_create")
        self.h = ctypes.c_void_p(h)
        self.block_size = block_size

    def close(self):
        if self.h:
            _c["pkv_pool_destroy"](self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return _c["pkv_pool_num_free"](self.h)

    def refcnt(self, block: int) -> int:
        return _c["pkv_pool_refcnt"](self.h, block)

    def append(self, table: np.ndarray, cur_len: int, n_new: int):
        """table: int32 array with capacity; returns (slots int64[n_new], cow (src, dst) or None)."""
        assert table.dtype == np.int32 and table.flags.c_contiguous
        slots = np.empty(max(n_new, 0), np.int64)
        cow = np.empty(2, np.int64)
        _check(_c["pkv_pool_append"](self.h, _ptr_i32(table), table.shape[0], cur_len, n_new,
                                     _ptr_i64(slots), _ptr_i64(cow)), "pkv_pool_append")
        return slots, (None if cow[0] < 0 else (int(cow[0]), int(cow[1])))

    def fork(self, table: np.ndarray, n_blocks: int) -> np.ndarray:
        out = np.zeros_like(table)
        _check(_c["pkv_pool_fork"](self.h, _ptr_i32(table), n_blocks, _ptr_i32(out)), "pkv_pool_fork")
        return out

    def release(self, table: np.ndarray, n_blocks: int) -> None:
        _check(_c["pkv_pool_release"](self.h, _ptr_i32(table), n_blocks), "pkv_pool_release")

    def match_prefix(self, tokens, table: np.ndarray) -> int:
        """Cached full blocks from the start of `tokens` go to table[:n]; returns n."""
        t = _host_i32(tokens)
        assert table.dtype == np.int32 and table.flags.c_contiguous
        n = ctypes.c_int32(0)
        _check(_c["pkv_pool_match_prefix"](self.h, _ptr_i32(t), t.shape[0], _ptr_i32(table),
                                           table.shape[0], ctypes.byref(n)), "pkv_pool_match_prefix")
        return int(n.value)

    def cache_blocks(self, tokens, table: np.ndarray, num_full_blocks: int) -> None:
        t = _host_i32(tokens)
        _check(_c["pkv_pool_cache_blocks"](self.h, _ptr_i32(t), t.shape[0], _ptr_i32(table),
                                           num_full_blocks), "pkv_pool_cache_blocks")


def pkv_block_hash(parent: int, tokens) -> int:
    t = _host_i32(tokens)
    return int(_c["pkv_block_hash"](parent, _ptr_i32(t), t.shape[0]))
