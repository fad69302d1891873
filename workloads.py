"""Seeded synthetic workloads shaped like the pages' serving workloads.

This module only *draws* inputs: sequence lengths, the order in which the
pool hands out physical blocks, and K/V/Q values.  It holds none of the
method's arithmetic (no slot, table, copy or attention computation): the HIP
library and the CPU oracle each derive those from what is drawn here.

Five workloads, all with 16-token blocks:
  1 tiny decode      4 seqs, L = {5,16,17,40}, Hq = Hkv = 4, D = 64, fp32
                     U[-1,1], pool of 64 blocks handed out in a seeded random
                     order, scale 1/8.
  2 7B-shaped MHA    Hq = Hkv = 32, D = 128, bf16 N(0,1), B = 64,
                     L ~ U[128, 2048], pool = 1.25 x the blocks needed.
  3 8B-shaped GQA    Hq = 32, Hkv = 8, D = 128, bf16 N(0,1), B = 256,
                     L ~ lognormal(median 800, sigma 1) clipped to [16, 8192],
                     blocks scattered over a pool of 200,000.
  4 mixed step       8B GQA shape; 98 decode seqs (L ~ U[64, 4096]) followed
                     by one 1950-token prefill chunk on top of 1048 cached
                     tokens; 2048 new tokens in all.
  5 13B-shaped MHA   Hq = Hkv = 40, D = 128, bf16; 16 forks of one
                     1032-token prompt (the prompt's owner keeps a reference),
                     16 independent seqs with L ~ U[1, 16384], one at 16384.

Every sequence appends ``q_len`` new tokens in the step (1 for decode) on
top of ``hist_len`` cached ones, so its length is hist_len + q_len.

Random streams: numpy SeedSequence(workload_id + 1000 * seed).spawn(4) ->
(lengths, physical block order, values, spare).  Values are drawn in float32
and rounded to nearest-even bf16 where the workload is bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = 0x7FC0
F32_NAN = 0x7FC00000
FP8_NAN = 0x7F
# FP8 KV caches of the FP8 variants: one K and one V scale per cache.  Values
# are N(0,1); with scale 1/64 the largest E4M3 magnitude 448 stands for 7.
FP8_SCALE = 1.0 / 64.0


@dataclass
class Workload:
    workload_id: int
    name: str
    dtype: str                  # "f32" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    scale: float
    num_blocks: int             # pool size in blocks
    free_order: np.ndarray      # int32 [num_blocks]: order the pool hands out blocks
    hist_len: np.ndarray        # int32 [B]: tokens cached before the step
    q_len: np.ndarray           # int32 [B]: tokens appended (and queried) in the step
    fork_of: np.ndarray         # int32 [B]: -1, or index of the shared prompt it forks
    prompt_len: np.ndarray      # int32 [P]: lengths of shared prompts
    prompt_owner_keeps_ref: bool
    # codes (uint16 for bf16, uint32 for f32)
    hist_k: np.ndarray          # [sum hist of independent seqs][Hkv][D]
    hist_v: np.ndarray
    hist_start: np.ndarray      # int64 [B+1] offsets into hist_* (forks own none)
    prompt_k: np.ndarray        # [sum prompt_len][Hkv][D]
    prompt_v: np.ndarray
    prompt_start: np.ndarray    # int64 [P+1]
    new_k: np.ndarray           # [T][Hkv][D], T = sum q_len, flattened seq order
    new_v: np.ndarray
    q: np.ndarray               # [T][Hq][D]
    pool_fill: int              # code every pool element holds before use (NaN)
    extra: dict = field(default_factory=dict)
    cache_dtype: str = ""       # "" = dtype; "fp8" = E4M3 cache written from bf16 values
    k_scale: float = 1.0        # FP8 cache: a stored code stands for e4m3 value * scale
    v_scale: float = 1.0

    @property
    def kv_dtype(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def kv_dtype_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    @property
    def batch(self) -> int:
        return int(self.hist_len.shape[0])

    @property
    def seq_lens(self) -> np.ndarray:
        return (self.hist_len + self.q_len).astype(np.int32)

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_len)]).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(self.q_len.sum())

    @property
    def dtype_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _bf16_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 codes, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def _values(rng: np.random.Generator, shape, dtype: str, draw: bool = True) -> np.ndarray:
    if not draw:
        return np.zeros(shape, dtype=np.uint32 if dtype == "f32" else np.uint16)
    if dtype == "f32":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32).view(np.uint32)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = _bf16_codes(rng.standard_normal(n, dtype=np.float32))
    return out


def _pool_size(lengths, factor: float, extra_blocks: int = 0) -> int:
    need = int(sum((int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in lengths)) + extra_blocks
    return int(np.ceil(factor * need))


def _build(workload_id: int, name: str, dtype: str, Hq: int, Hkv: int, D: int, scale: float,
           hist_len, q_len, num_blocks: int, streams, fork_of=None, prompt_len=(),
           owner_ref=False, extra=None, values: bool = True, cache_dtype: str = "",
           kv_scale: float = 1.0) -> Workload:
    _, r_blocks, r_vals, _ = streams
    hist_len = np.asarray(hist_len, dtype=np.int32)
    q_len = np.asarray(q_len, dtype=np.int32)
    B = hist_len.shape[0]
    fork_of = np.full(B, -1, np.int32) if fork_of is None else np.asarray(fork_of, np.int32)
    prompt_len = np.asarray(prompt_len, dtype=np.int32)
    own_hist = np.where(fork_of < 0, hist_len, 0).astype(np.int64)
    hist_start = np.concatenate([[0], np.cumsum(own_hist)]).astype(np.int64)
    prompt_start = np.concatenate([[0], np.cumsum(prompt_len.astype(np.int64))]).astype(np.int64)
    free_order = r_blocks.permutation(num_blocks).astype(np.int32)
    T = int(q_len.sum())
    n_hist = int(hist_start[-1])
    n_prompt = int(prompt_start[-1])
    w = Workload(
        workload_id=workload_id, name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
        head_size=D, scale=scale, num_blocks=num_blocks, free_order=free_order,
        hist_len=hist_len, q_len=q_len, fork_of=fork_of, prompt_len=prompt_len,
        prompt_owner_keeps_ref=owner_ref,
        hist_k=_values(r_vals, (n_hist, Hkv, D), dtype, values),
        hist_v=_values(r_vals, (n_hist, Hkv, D), dtype, values),
        hist_start=hist_start,
        prompt_k=_values(r_vals, (n_prompt, Hkv, D), dtype, values),
        prompt_v=_values(r_vals, (n_prompt, Hkv, D), dtype, values),
        prompt_start=prompt_start,
        new_k=_values(r_vals, (T, Hkv, D), dtype, values),
        new_v=_values(r_vals, (T, Hkv, D), dtype, values),
        q=_values(r_vals, (T, Hq, D), dtype, values),
        pool_fill=FP8_NAN if cache_dtype == "fp8" else (F32_NAN if dtype == "f32" else BF16_NAN),
        extra=extra or {},
        cache_dtype=cache_dtype, k_scale=kv_scale, v_scale=kv_scale,
    )
    return w


def make_verify(k: int = 3, seed: int = 0, small_size: bool = False) -> Workload:
    """Speculative-decoding verify step on the 8B GQA decode batch: every
    sequence appends its last accepted token plus k draft tokens and queries
    all k + 1 positions (causal), as the pages' verify pass does (k = 3 in
    their n-gram example).  Lengths, pool and values are drawn like the 8B
    GQA decode workload (batch 256, or 12 short sequences with small_size)."""
    streams = [np.random.default_rng(x)
               for x in np.random.SeedSequence(20_000 + 1000 * seed + 10 * small_size).spawn(4)]
    r_len = streams[0]
    if small_size:
        B = 12
        L = np.clip(np.rint(r_len.lognormal(np.log(120.0), 1.0, size=B)), k + 1, 900).astype(np.int32)
        L[0], L[1], L[2] = k + 1, 16, 17
        pool = 4000
    else:
        B = 256
        L = np.clip(np.rint(r_len.lognormal(np.log(800.0), 1.0, size=B)), 16, 8192).astype(np.int32)
        pool = 200_000
    return _build(3, f"8B GQA verify (k={k})" + (" (small)" if small_size else ""), "bf16", 32, 8,
                  128, 128 ** -0.5, L - (k + 1), np.full(B, k + 1, np.int32), pool, streams)


def make_fp8(workload_id: int, seed: int = 0, small_size: bool = False) -> Workload:
    """A bf16 workload (2, 3 or 5, full or small) whose KV cache is
    FP8 E4M3 with K and V scales of 1/64: same lengths, blocks and drawn
    values; the cache stores them quantized."""
    w = small(workload_id, seed) if small_size else make(workload_id, seed)
    assert w.dtype == "bf16"
    w.name = w.name + " (fp8 KV)"
    w.cache_dtype = "fp8"
    w.k_scale = w.v_scale = FP8_SCALE
    w.pool_fill = FP8_NAN
    return w


def make(workload_id: int, seed: int = 0, batch: int | None = None, values: bool = True) -> Workload:
    """Workload ``workload_id`` of the list above.  ``batch`` (optional) keeps the
    shape and length distribution but draws fewer sequences, for quick runs.
    ``values=False`` skips drawing K/V/Q (zeros instead); lengths and block
    order are unchanged."""
    streams = np.random.SeedSequence(workload_id + 1000 * seed).spawn(4)
    streams = [np.random.default_rng(s) for s in streams]
    r_len = streams[0]

    if workload_id == 1:
        L = np.array([5, 16, 17, 40], np.int32)
        return _build(1, "tiny decode", "f32", 4, 4, 64, 1.0 / 8.0, L - 1, np.ones(4, np.int32),
                      64, streams, values=values)

    if workload_id == 2:
        B = batch or 64
        L = r_len.integers(128, 2048, size=B, endpoint=True).astype(np.int32)
        return _build(2, "7B MHA decode", "bf16", 32, 32, 128, 128 ** -0.5, L - 1,
                      np.ones(B, np.int32), _pool_size(L, 1.25), streams, values=values)

    if workload_id == 3:
        B = batch or 256
        L = np.rint(r_len.lognormal(np.log(800.0), 1.0, size=B))
        L = np.clip(L, 16, 8192).astype(np.int32)
        return _build(3, "8B GQA decode", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                      np.ones(B, np.int32), 200_000, streams, values=values)

    if workload_id == 4:
        n_dec = 98 if batch is None else max(batch - 1, 1)
        L_dec = r_len.integers(64, 4096, size=n_dec, endpoint=True).astype(np.int32)
        chunk, cached = 1950, 1048
        hist = np.concatenate([L_dec - 1, [cached]]).astype(np.int32)
        qlen = np.concatenate([np.ones(n_dec, np.int32), [chunk]]).astype(np.int32)
        return _build(4, "mixed chunked prefill + decode", "bf16", 32, 8, 128, 128 ** -0.5,
                      hist, qlen, _pool_size(hist + qlen, 1.25), streams, values=values)

    if workload_id == 5:
        n_fork = 16 if batch is None else max(batch // 2, 1)
        n_ind = 16 if batch is None else max(batch - n_fork, 1)
        prompt = 1032
        L_ind = r_len.integers(1, 16384, size=n_ind, endpoint=True).astype(np.int32)
        L_ind[0] = 16384
        hist = np.concatenate([np.full(n_fork, prompt, np.int32), L_ind - 1]).astype(np.int32)
        qlen = np.ones(n_fork + n_ind, np.int32)
        fork_of = np.concatenate([np.zeros(n_fork, np.int32), np.full(n_ind, -1, np.int32)])
        lengths = list(L_ind) + [prompt]
        return _build(5, "13B MHA prefix sharing + long context", "bf16", 40, 40, 128,
                      128 ** -0.5, hist, qlen, _pool_size(lengths, 1.25, extra_blocks=n_fork),
                      streams, fork_of=fork_of, prompt_len=[prompt], owner_ref=True, values=values)

    raise ValueError(f"unknown workload {workload_id}")


def small(workload_id: int, seed: int = 0) -> Workload:
    """A reduced workload of the same family that the oracle finishes in
    seconds: same head shapes and distributions, fewer and shorter seqs."""
    streams = [np.random.default_rng(s)
               for s in np.random.SeedSequence(10_000 + workload_id + 1000 * seed).spawn(4)]
    r_len = streams[0]
    if workload_id == 1:
        return make(1, seed)
    if workload_id == 2:
        L = r_len.integers(1, 300, size=6, endpoint=True).astype(np.int32)
        return _build(2, "7B MHA decode (small)", "bf16", 32, 32, 128, 128 ** -0.5, L - 1,
                      np.ones(6, np.int32), _pool_size(L, 1.25), streams)
    if workload_id == 3:
        L = np.clip(np.rint(r_len.lognormal(np.log(120.0), 1.0, size=12)), 1, 900).astype(np.int32)
        L[0] = 1
        L[1] = 16
        L[2] = 17
        L[3] = 513
        return _build(3, "8B GQA decode (small)", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                      np.ones(12, np.int32), 4000, streams)
    if workload_id == 4:
        L_dec = r_len.integers(1, 400, size=5, endpoint=True).astype(np.int32)
        hist = np.concatenate([L_dec - 1, [37]]).astype(np.int32)
        qlen = np.concatenate([np.ones(5, np.int32), [150]]).astype(np.int32)
        return _build(4, "mixed step (small)", "bf16", 32, 8, 128, 128 ** -0.5, hist, qlen,
                      _pool_size(hist + qlen, 1.25), streams)
    if workload_id == 5:
        prompt = 40
        L_ind = r_len.integers(1, 600, size=3, endpoint=True).astype(np.int32)
        hist = np.concatenate([np.full(3, prompt, np.int32), L_ind - 1]).astype(np.int32)
        fork_of = np.array([0, 0, 0, -1, -1, -1], np.int32)
        return _build(5, "13B MHA prefix sharing (small)", "bf16", 40, 40, 128, 128 ** -0.5,
                      hist, np.ones(6, np.int32), _pool_size(list(L_ind) + [prompt], 1.25, 3),
                      streams, fork_of=fork_of, prompt_len=[prompt], owner_ref=True)
    raise ValueError(workload_id)
