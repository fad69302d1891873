"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and its host-side work (slot mapping, block allocator, argument checks,
sizing) agrees exactly with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads
from oracle import paged_oracle as po
from oracle import scenario

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = pytest.importorskip("paged_kv_attention_06_amd")
from paged_kv_attention_06_amd import _lib as L  # noqa: E402


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keywords = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in keywords})


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(L.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 17
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(L.EXPORTED)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_block_bytes_per_workload(cfg):
    w = workloads.small(cfg)
    d = P.descriptor(7, w.num_kv_heads, w.head_size, P.PKV_F32 if w.dtype == "f32" else P.PKV_BF16)
    assert P.pkv_block_bytes(d) == po.block_bytes(16, w.num_kv_heads, w.head_size, w.dtype_bytes)


def test_fp8_descriptor_bytes_and_scales():
    """An FP8 E4M3 cache has one byte per element; its scales must be finite
    and positive."""
    d = P.descriptor(7, 8, 128, P.PKV_FP8_E4M3, k_scale=0.5, v_scale=0.25)
    assert P.pkv_block_bytes(d) == po.block_bytes(16, 8, 128, 1) == 32768
    good = P.descriptor(16, 8, 128, P.PKV_FP8_E4M3, kv_ptr=0x1000, k_scale=0.5, v_scale=0.5)
    assert _call_decode(good, hq=32) == 4                       # gets to the workspace check
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (float("nan"), 1.0)):
        bad = P.descriptor(16, 8, 128, P.PKV_FP8_E4M3, kv_ptr=0x1000, k_scale=ks, v_scale=vs)
        assert _call_decode(bad, hq=32) == 7                    # PKV_ERR_RANGE


def test_fp8_cache_rejects_prefill_rows():
    """Rows with q_len > 1 need a bf16 cache."""
    d = P.descriptor(64, 8, 128, P.PKV_FP8_E4M3, kv_ptr=0x1000, k_scale=0.5, v_scale=0.5)
    qsl = np.array([0, 1, 5], np.int32)
    sl = np.array([3, 9], np.int32)
    st = L._c["paged_attention_mixed"](
        ctypes.byref(d), 1, 1, 32, 1, 1, qsl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 4, 2, 5, 0.1, 1, 1 << 30, None)
    assert st == 3                                              # PKV_ERR_DTYPE


def test_block_bytes_rejects_bad_descriptors():
    assert P.pkv_block_bytes(P.descriptor(7, 8, 96, P.PKV_BF16)) == 0     # head size
    assert P.pkv_block_bytes(P.descriptor(7, 8, 128, 9)) == 0             # dtype
    assert P.pkv_block_bytes(P.descriptor(7, 8, 128, P.PKV_BF16, block_size=32)) == 0
    assert P.pkv_block_bytes(P.descriptor(0, 8, 128, P.PKV_BF16)) == 0


def _gpu_side_tables(w):
    """Replays allocation with the library's pkv_pool (host only)."""
    pool = P.Pool(w.num_blocks, w.free_order)
    maxb = max(1, -(-int(w.seq_lens.max()) // 16))
    tables = np.zeros((w.batch, maxb), np.int32)
    prompts = []
    for p in range(len(w.prompt_len)):
        t = np.zeros(maxb, np.int32)
        pool.append(t, 0, int(w.prompt_len[p]))
        prompts.append(t)
    for s in range(w.batch):
        if w.fork_of[s] < 0:
            pool.append(tables[s], 0, int(w.hist_len[s]))
    for s in range(w.batch):
        if w.fork_of[s] >= 0:
            p = int(w.fork_of[s])
            nb = -(-int(w.prompt_len[p]) // 16)
            tables[s, :nb] = pool.fork(prompts[p], nb)[:nb]
    if not w.prompt_owner_keeps_ref:
        for p, t in enumerate(prompts):
            pool.release(t, -(-int(w.prompt_len[p]) // 16))
    slots, cows = [], []
    for s in range(w.batch):
        sl, c = pool.append(tables[s], int(w.hist_len[s]), int(w.q_len[s]))
        slots.append(sl)
        if c is not None:
            cows.append(c)
    return pool, tables, np.concatenate(slots), np.asarray(cows, np.int64).reshape(-1, 2), prompts


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_allocator_matches_oracle_small(cfg):
    w = workloads.small(cfg)
    pool, tables, slots, cows, prompts = _gpu_side_tables(w)
    st = scenario.build_tables(w, with_pool=False)
    for s in range(w.batch):
        n = len(st["tables"][s])
        assert tables[s, :n].tolist() == st["tables"][s]
    assert np.array_equal(slots, st["slots"])
    assert np.array_equal(cows, st["cow_pairs"])
    assert pool.num_free() == st["alloc"].num_free()
    for b in range(w.num_blocks):
        assert pool.refcnt(b) == st["alloc"].ref[b]


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_allocator_and_slots_match_oracle_full_size(cfg):
    w = workloads.make(cfg, values=False)
    pool, tables, slots, cows, _ = _gpu_side_tables(w)
    st = scenario.build_tables(w, with_pool=False)
    for s in range(w.batch):
        n = len(st["tables"][s])
        assert tables[s, :n].tolist() == st["tables"][s]
    assert np.array_equal(slots, st["slots"])
    assert np.array_equal(cows, st["cow_pairs"])
    # the library's slot builder agrees with the allocator's slots and the oracle's
    lib_slots = P.pkv_build_slot_mapping(tables, w.query_start_loc, w.seq_lens)
    assert np.array_equal(lib_slots, slots)
    bt = scenario.table_matrix(st["tables"], tables.shape[1])
    assert np.array_equal(po.slot_mapping(bt, w.query_start_loc, w.seq_lens), lib_slots)


def test_cow_walkthrough_through_library():
    pool = P.Pool(10, np.array([0, 1, 2, 7, 3, 4, 5, 6, 8, 9], np.int32))
    prompt = np.zeros(4, np.int32)
    pool.append(prompt, 0, 40)
    assert prompt[:3].tolist() == [0, 1, 2]
    samples = [prompt] + [pool.fork(prompt, 3) for _ in range(3)]
    assert [pool.refcnt(b) for b in (0, 1, 2)] == [4, 4, 4]
    slots, cow = pool.append(samples[0], 40, 1)
    assert cow == (2, 7) and samples[0][:3].tolist() == [0, 1, 7] and pool.refcnt(2) == 3
    assert slots.tolist() == [7 * 16 + 8]


def test_allocator_errors_leave_state_unchanged():
    pool = P.Pool(3)
    t = np.zeros(8, np.int32)
    with pytest.raises(P.PkvError) as e:
        pool.append(t, 0, 60)                       # 4 blocks > 3 free
    assert e.value.status == 6
    assert pool.num_free() == 3
    with pytest.raises(P.PkvError) as e:
        pool.append(np.zeros(2, np.int32), 0, 40)   # table capacity
    assert e.value.status == 7
    with pytest.raises(P.PkvError):
        P.Pool(3, np.array([0, 0, 1], np.int32))    # not a permutation


def test_slot_mapping_rejects_bad_lengths():
    bt = np.array([[3, 4]], np.int32)
    with pytest.raises(P.PkvError) as e:
        P.pkv_build_slot_mapping(bt, [0, 1], [33])  # longer than the table
    assert e.value.status == 7
    with pytest.raises(P.PkvError):
        P.pkv_build_slot_mapping(bt, [0, 3], [2])   # more rows than tokens
    assert P.pkv_build_slot_mapping(bt, [0, 2], [18]).tolist() == [4 * 16 + 0, 4 * 16 + 1]


def test_page_address_translation_through_library():
    bt = np.array([[17, 42, 99]], np.int32)
    assert P.pkv_build_slot_mapping(bt, [0, 1], [19]).tolist() == [42 * 16 + 2]


def test_workspace_sizing():
    d = P.descriptor(100, 8, 128, P.PKV_BF16)
    cache = P.Cache(None, 100, 8, 128, P.PKV_BF16)
    cache.desc = d
    lens = np.array([1, 256, 257, 0, 8192], np.int32)
    units = 1 + 1 + 2 + 0 + 32
    header = 256                                      # workspace header
    split_k = header + units * 32 * (128 + 2) * 4
    # a pure decode batch may instead run the stream kernel: one cost unit per
    # 32-token step plus one setup unit per (row, kv head); at most one wave
    # per 8 units, two partials (4 heads x (128 + 2) floats) per wave, then
    # (256-aligned) one 8-byte counter per (row, kv head)
    cost = 8 * sum(-(-int(x) // 32) + 1 for x in lens if x > 0)
    waves = min(4096, -(-cost // 8))
    ml_end = header + 2 * waves * 4 * 128 * 4 + 2 * waves * 4 * 2 * 4
    stream = -(-ml_end // 256) * 256 + 5 * 8 * 8
    assert P.pkv_attention_workspace_bytes(cache, 32, lens) == max(split_k, stream)
    qsl = np.array([0, 1, 2, 3, 3, 1000], np.int32)   # seq 4 is a prefill chunk
    # a prefill sequence of length L adds fp16 V tiles of its blocks, rounded
    # up to whole 64-key tiles, for every kv head, and one int32 exponent each
    vblocks = 4 * -(-8192 // 64)
    prefill = vblocks * 8 * (16 * 128 * 2 + 4)
    # the decode rows' region fits either decode path: fixed partitions, or
    # the stream kernel sized by the decode rows alone (rows 0..2)
    dec = header + 4 * 32 * 130 * 4
    cost_d = 8 * sum(-(-int(x) // 32) + 1 for x in lens[:3])
    waves_d = min(4096, -(-cost_d // 8))
    ml_end_d = header + 2 * waves_d * 4 * 128 * 4 + 2 * waves_d * 4 * 2 * 4
    stream_d = -(-ml_end_d // 256) * 256 + 5 * 8 * 8
    dec = max(dec, stream_d)
    assert P.pkv_attention_workspace_bytes(cache, 32, lens, qsl) == -(-dec // 256) * 256 + prefill
    only_prefill = np.array([0, 1000], np.int32)
    assert P.pkv_attention_workspace_bytes(cache, 32, lens[4:], only_prefill) == header + prefill
    assert P.pkv_attention_workspace_bytes(cache, 32, lens[3:4], np.array([0, 0], np.int32)) == 0


def _call_decode(cache_desc, out=1, q=1, bt=1, sl=1, h_sl=None, n=1, hq=32, ws=None, ws_bytes=0,
                 maxb=4):
    h_sl = np.array([5], np.int32) if h_sl is None else h_sl
    return L._c["paged_attention_decode"](
        ctypes.byref(cache_desc), out, q, hq, bt, maxb, sl,
        h_sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, 0.1, ws, ws_bytes, None)


def test_argument_checks_return_before_launch():
    good = P.descriptor(16, 8, 128, P.PKV_BF16, kv_ptr=0x1000)
    assert _call_decode(P.descriptor(16, 8, 128, P.PKV_BF16)) == 1          # NULL pool
    assert _call_decode(P.descriptor(16, 8, 96, P.PKV_BF16, kv_ptr=0x1000)) == 2
    assert _call_decode(P.descriptor(16, 8, 128, 7, kv_ptr=0x1000)) == 3
    assert _call_decode(good, hq=12) == 2                                   # 12 % 8 != 0
    assert _call_decode(good, hq=8 * 16) == 2                               # group of 16
    assert _call_decode(good, h_sl=np.array([65], np.int32)) == 7          # > 4 blocks
    assert _call_decode(good, out=None) == 1
    assert _call_decode(good, h_sl=np.array([300], np.int32), maxb=32) == 4  # needs workspace
    st = L._c["paged_kv_write"](ctypes.byref(good), None, None, None, 5, None)
    assert st == 1
    assert L._c["paged_kv_write"](ctypes.byref(good), None, None, None, 0, None) == 0
    assert L._c["block_copy"](ctypes.byref(good), None, -1, None) == 2


def test_block_swap_argument_checks():
    """Errors come back before anything is launched: bad direction or counts,
    NULL pointers, and host memory that is not pinned and device-mapped."""
    d = P.descriptor(16, 8, 128, P.PKV_BF16, kv_ptr=0x1000)
    host = np.zeros(65536 * 2, np.uint8)
    hp = host.ctypes.data_as(ctypes.c_void_p)
    f = L._c["block_swap"]
    assert f(ctypes.byref(d), hp, 2, 1, 1, 5, None) == 7          # direction
    assert f(ctypes.byref(d), hp, 2, 1, -1, 0, None) == 2         # negative count
    assert f(ctypes.byref(d), hp, 2, 1, 0, 0, None) == 0          # nothing to do
    assert f(ctypes.byref(d), None, 2, 1, 1, 0, None) == 1        # NULL host pool
    assert f(ctypes.byref(d), hp, 2, None, 1, 1, None) == 1       # NULL pairs
    assert f(ctypes.byref(d), hp, 2, 1, 1, 0, None) == 7          # malloc'd, not pinned


def test_block_hash_matches_oracle():
    rng = np.random.default_rng(12)
    for _ in range(50):
        parent = int(rng.integers(0, 2**63))
        toks = rng.integers(-2**31, 2**31, size=16).astype(np.int32)
        assert P.pkv_block_hash(parent, toks) == po.block_hash(parent, toks.tolist())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefix_cache_replay_matches_oracle(seed):
    """Requests from a few shared-prefix families arrive, reuse their cached
    prefix, append the rest, register their full blocks and finish at random;
    the library's pool and the oracle's take identical decisions (hits,
    tables, reference counts, free counts), evictions included."""
    rng = np.random.default_rng(100 + seed)
    nb = 160
    order = rng.permutation(nb).astype(np.int32)
    lib = P.Pool(nb, order)
    ora = po.PrefixCachePool(nb, order)
    families = [rng.integers(0, 50000, size=int(n)).tolist() for n in (40, 96, 130, 16)]
    live = []
    total_hits = 0
    for step in range(300):
        if live and (rng.random() < 0.45 or lib.num_free() < 40):
            i = int(rng.integers(len(live)))
            toks, t_lib, t_ora = live.pop(i)
            n = -(-len(toks) // 16)
            lib.release(t_lib, n)
            ora.release(t_ora)
        else:
            fam = families[int(rng.integers(len(families)))]
            cut = int(rng.integers(len(fam) // 2, len(fam) + 1))
            toks = fam[:cut] + rng.integers(0, 50000, size=int(rng.integers(1, 40))).tolist()
            t_lib = np.zeros(32, np.int32)
            hits = lib.match_prefix(toks, t_lib)
            hits_o = ora.match_prefix(toks)
            assert t_lib[:hits].tolist() == hits_o
            total_hits += hits
            t_ora = list(hits_o)
            lib.append(t_lib, hits * 16, len(toks) - hits * 16)
            ora.append(t_ora, hits * 16, len(toks) - hits * 16)
            n = -(-len(toks) // 16)
            assert t_lib[:n].tolist() == t_ora
            lib.cache_blocks(toks, t_lib, len(toks) // 16)
            ora.cache_blocks(toks, t_ora, len(toks) // 16)
            live.append((toks, t_lib, t_ora))
        assert lib.num_free() == len(ora.free)
        assert [lib.refcnt(b) for b in range(nb)] == ora.ref
    assert total_hits > 50


# ----------------------------------------- debug checks of device-side preconditions
def _status(fn, *args, **kw):
    try:
        fn(*args, **kw)
        return 0, ""
    except L.PkvError as e:
        return e.status, str(e)


def test_layout_constant():
    """The pool layout is exported as a value callers can check."""
    assert P.pkv_layout() == P.PKV_LAYOUT_HEAD_KV_GRANULE16 == 1
    assert "PKV_LAYOUT_HEAD_KV_GRANULE16 = 1" in open(os.path.join(ROOT, "include", "pkv.h")).read()


def test_validate_slots_rejects_each_violation():
    """paged_kv_write's preconditions (vLLM 源码精读 5.1: every new token has a
    slot of its own): slots below num_blocks * 16, no slot written twice;
    negative slots are skipped."""
    d = P.descriptor(4, 2, 64, P.PKV_BF16)                # 64 slots
    assert _status(P.pkv_validate_slots, d, [0, 63, -1, 17, -5, 16]) == (0, "")
    assert _status(P.pkv_validate_slots, d, [])[0] == 0
    st, msg = _status(P.pkv_validate_slots, d, [3, 64])
    assert st == 7 and "slot_mapping[1] = 64" in msg
    st, msg = _status(P.pkv_validate_slots, d, [3, 5, -1, 3])
    assert st == 7 and "slot 3 is written by tokens 0 and 3" in msg
    assert _status(P.pkv_validate_slots, P.descriptor(4, 2, 96, P.PKV_BF16), [0])[0] == 2


def test_validate_block_pairs_rejects_each_violation():
    """block_copy's preconditions (juhe.plus 3.8: copy-on-write copies a
    shared block into a fresh one) and block_swap's (ids on both sides)."""
    ok = [[0, 5], [0, 6], [1, 7]]                          # a source may repeat
    assert _status(P.pkv_validate_block_pairs, ok, 8, 8, True)[0] == 0
    for pairs, what in (([[8, 1]], "source block 8"), ([[-1, 1]], "source block -1"),
                        ([[0, 8]], "destination block 8"), ([[0, 5], [1, 5]], "block 5 is the destination of pairs 0 and 1"),
                        ([[0, 5], [5, 6]], "block 5 is the destination of pair 0 and the source of pair 1")):
        st, msg = _status(P.pkv_validate_block_pairs, pairs, 8, 8, True)
        assert st == 7 and what in msg, (pairs, msg)
    # swap: two pools, so a block id may appear on both sides
    assert _status(P.pkv_validate_block_pairs, [[0, 5], [5, 6]], 8, 8, False)[0] == 0
    assert _status(P.pkv_validate_block_pairs, [[2, 9]], 3, 10, False)[0] == 0
    assert _status(P.pkv_validate_block_pairs, [[3, 0]], 3, 10, False)[0] == 7
    assert _status(P.pkv_validate_block_pairs, [[0, 10]], 3, 10, False)[0] == 7


def test_validate_attention_rejects_each_violation():
    """Attention's preconditions (juhe.plus 3.3 / 3.6: every position below
    the length translates through a valid table entry)."""
    d = P.descriptor(10, 2, 64, P.PKV_BF16)
    bt = np.array([[3, 9, 0], [1, -1, -1]], np.int32)      # unused entries may hold anything
    lens = np.array([33, 16], np.int32)
    assert _status(P.pkv_validate_attention, d, bt, lens, lens)[0] == 0
    assert _status(P.pkv_validate_attention, d, bt, lens, None, [0, 1, 2], [0, 1, 2])[0] == 0
    assert _status(P.pkv_validate_attention, d, bt, [0, 0], [0, 0])[0] == 0
    cases = [
        (dict(seq_lens=[49, 16], h_seq_lens=None), "seq_lens[0] = 49 outside"),
        (dict(seq_lens=[-1, 16], h_seq_lens=None), "seq_lens[0] = -1 outside"),
        (dict(block_tables=[[3, 10, 0], [1, 0, 0]]), "block_tables[0][1] = 10"),
        (dict(block_tables=[[3, 9, 0], [-1, 0, 0]]), "block_tables[1][0] = -1"),
        (dict(seq_lens=[33, 17], h_seq_lens=None), "block_tables[1][1] = -1"),
        (dict(h_seq_lens=[33, 15]), "seq_lens[1] = 16, but 15 in the host copy"),
        (dict(query_start_loc=[0, 2, 3], h_query_start_loc=[0, 1, 3]), "query_start_loc[1] = 2"),
        (dict(query_start_loc=[0, 34, 35], h_query_start_loc=None), "34 query rows and length 33"),
        (dict(query_start_loc=[1, 2, 3], h_query_start_loc=None), "query_start_loc[0] = 1"),
    ]
    for change, what in cases:
        kw = dict(block_tables=bt, seq_lens=lens, h_seq_lens=lens, query_start_loc=None,
                  h_query_start_loc=None)
        kw.update(change)
        st, msg = _status(P.pkv_validate_attention, d, **kw)
        assert st == 7 and what in msg, (change, msg)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_validators_accept_the_full_size_workloads(cfg):
    """The tables, lengths, slots and copy-on-write pairs the library's
    allocator builds for every full-size workload meet every precondition."""
    w = workloads.make(cfg, values=False)
    _, tables, slots, cows, _ = _gpu_side_tables(w)
    d = P.descriptor(w.num_blocks, w.num_kv_heads, w.head_size, P.PKV_BF16)
    P.pkv_validate_slots(d, slots)
    P.pkv_validate_block_pairs(cows, w.num_blocks, w.num_blocks, True)
    P.pkv_validate_attention(d, tables, w.seq_lens, w.seq_lens, w.query_start_loc,
                             w.query_start_loc)
