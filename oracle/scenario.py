"""Oracle-side replay of one workload step.  TEST INFRASTRUCTURE ONLY.

Builds the cache the way the pages describe and runs the step on the CPU:
  1. shared prompts, then every independent sequence's history, are appended
     through the block allocator and written to their slots;
  2. forks take another reference on their prompt's blocks (parallel
     sampling, juhe.plus 3.5); the prompt's owner keeps its own reference
     when the workload says so;
  3. the step appends each sequence's new tokens in batch order; appending
     into a partly filled block that is shared triggers copy-on-write
     (vLLM 技术内幕 2.2, juhe.plus 3.8);
  4. the copies are applied, the new tokens' K/V are written, and attention
     runs over the paged cache.
"""
from __future__ import annotations

import numpy as np

from . import paged_oracle as po


def build_tables(w, with_pool: bool = True):
    """Steps 1-3.  Returns a dict with the pool (or None), block tables
    (lists), the step's slots and COW pairs, and the allocator."""
    alloc = po.CowPool(w.num_blocks, w.free_order)
    kvd = w.kv_dtype
    wr = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    pool = po.new_pool(w.num_blocks, w.num_kv_heads, w.head_size, kvd, w.pool_fill) \
        if with_pool else None

    prompt_tables = []
    for p in range(len(w.prompt_len)):
        table = []
        slots, _ = alloc.append(table, 0, int(w.prompt_len[p]))
        if with_pool:
            a, b = int(w.prompt_start[p]), int(w.prompt_start[p + 1])
            po.kv_write(pool, kvd, w.prompt_k[a:b], w.prompt_v[a:b], slots, **wr)
        prompt_tables.append(table)

    tables = [None] * w.batch
    for s in range(w.batch):
        if w.fork_of[s] >= 0:
            continue
        table = []
        slots, _ = alloc.append(table, 0, int(w.hist_len[s]))
        if with_pool:
            a, b = int(w.hist_start[s]), int(w.hist_start[s + 1])
            po.kv_write(pool, kvd, w.hist_k[a:b], w.hist_v[a:b], slots, **wr)
        tables[s] = table
    for s in range(w.batch):
        if w.fork_of[s] >= 0:
            tables[s] = alloc.fork(prompt_tables[int(w.fork_of[s])])
    if not w.prompt_owner_keeps_ref:
        for t in prompt_tables:
            alloc.release(t)

    step_slots, cow_pairs = [], []
    for s in range(w.batch):
        slots, cow = alloc.append(tables[s], int(w.hist_len[s]), int(w.q_len[s]))
        step_slots.extend(slots)
        if cow is not None:
            cow_pairs.append(cow)
    return dict(pool=pool, tables=tables, slots=np.asarray(step_slots, np.int64),
                cow_pairs=np.asarray(cow_pairs, np.int64).reshape(-1, 2), alloc=alloc,
                prompt_tables=prompt_tables)


def table_matrix(tables, max_blocks: int | None = None) -> np.ndarray:
    """Block tables as a zero-padded int32 matrix [B][max_blocks]."""
    width = max_blocks or max(1, max(len(t) for t in tables))
    m = np.zeros((len(tables), width), np.int32)
    for s, t in enumerate(tables):
        m[s, : len(t)] = t
    return m


def run_step(w):
    """Steps 1-4 on a full oracle pool: returns the state dict with the
    final pool and the float64 attention output [T][Hq][D]."""
    st = build_tables(w, with_pool=True)
    po.block_copy(st["pool"], st["cow_pairs"])
    po.kv_write(st["pool"], w.kv_dtype, w.new_k, w.new_v, st["slots"], k_scale=w.k_scale,
                v_scale=w.v_scale)
    bt = table_matrix(st["tables"])
    st["block_tables"] = bt
    st["out"] = po.paged_attention(st["pool"], w.kv_dtype, w.q, bt, w.seq_lens,
                                   w.query_start_loc, w.scale, k_scale=w.k_scale,
                                   v_scale=w.v_scale)
    return st


def sequence_kv(w, s: int):
    """Codes K, V [L][Hkv][D] of sequence s in logical order, straight from
    the workload's draws (no pool): its history (or its prompt) followed by
    its new tokens.  Used for sampled checks at sizes where a full oracle
    pool does not fit."""
    qsl = w.query_start_loc
    new_k = w.new_k[qsl[s]:qsl[s + 1]]
    new_v = w.new_v[qsl[s]:qsl[s + 1]]
    if w.fork_of[s] >= 0:
        p = int(w.fork_of[s])
        a, b = int(w.prompt_start[p]), int(w.prompt_start[p + 1])
        hk, hv = w.prompt_k[a:b], w.prompt_v[a:b]
    else:
        a, b = int(w.hist_start[s]), int(w.hist_start[s + 1])
        hk, hv = w.hist_k[a:b], w.hist_v[a:b]
    return np.concatenate([hk, new_k]), np.concatenate([hv, new_v])


def sequence_attention(w, s: int, rows=None) -> np.ndarray:
    """float64 output rows of sequence s computed from its logical K/V
    (textbook attention, no paging).  ``rows`` selects query rows of s."""
    K, V = sequence_kv(w, s)
    qsl = w.query_start_loc
    q_len = int(qsl[s + 1] - qsl[s])
    L = int(w.seq_lens[s])
    rows = range(q_len) if rows is None else rows
    rows = list(rows)
    q = po.decode(w.q[qsl[s] + np.asarray(rows, np.int64)], w.dtype)
    positions = [L - q_len + i for i in rows]
    if w.kv_dtype == "fp8":       # what an FP8 cache holds: the quantized values
        Kf = po.decode(po.fp8_quantize(K, w.k_scale), "fp8") * w.k_scale
        Vf = po.decode(po.fp8_quantize(V, w.v_scale), "fp8") * w.v_scale
        return po.attention_rows(q, Kf, Vf, positions, w.scale)
    return po.attention_rows(q, po.decode(K, w.dtype), po.decode(V, w.dtype), positions, w.scale)
