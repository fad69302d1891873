"""Benchmark of the paged KV attention hot path on one MI355X.

A step is one pass of the whole path over the 8B-shaped GQA decode batch
(32 query / 8 kv heads, head size 128, bf16, 256 sequences with lognormal
contexts, median 800, in a 200,000-block pool): block copies (none in this
workload), the KV write of the 256 new tokens, and decode attention (one launch of the
stream-split kernel, which also merges split rows).  Inputs are resident in
HBM before timing starts.

Prints one JSON line (rank 0, N = 1).  The roofline object describes the
attention call, the dominant cost of the step: algorithmic bytes (every
valid token's K and V once, plus q, out, tables and lengths) divided by its
average duration from HIP events on the launch stream.  Beside it, each with
its own roofline: `gather_ceiling` (the same batch's (block, kv head) slices
read once by pkv_read_slices, no arithmetic: the read rate this access
pattern allows), `mixed_step` (the 8B GQA chunked-prefill step: 98 decode
rows plus a 1950-row chunk, against the serialized HBM + MFMA bound) and
`prefill_chunk` (that chunk alone, against the bf16 MFMA peak).  The CPU
baseline (the oracle on every host core) runs first, before the GPU is
touched.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode attention tokens/s & achieved HBM GB/s (% of peak), 8B-GQA batch 256"
# HBM bytes per launch of the dominant kernel of each workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, each scaled by what the
# counter reads for a device copy of known size), with a digest of the kernel
# code they were taken on (profiles/traffic.json).  A figure is reported only
# while that code is unchanged; otherwise `traffic` is null until the counters
# are taken again.
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_attention_06_amd", "csrc", "pkv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_code_digest(path: str = KERNEL_SOURCE) -> str:
    """SHA-256 of the kernel source without its comments, blank lines and
    runs of blanks: edits of comments or layout keep the digest, any change
    of code changes it.  (A `//` inside a string literal would count as a
    comment; the kernel source has none.)"""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [" ".join(line.split()) for line in text.split("\n")]
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def measured_traffic(key: str):
    try:
        rec = json.load(open(TRAFFIC_FILE))[key]
        digest = kernel_code_digest()
    except (OSError, KeyError, ValueError):
        return None
    return int(rec["bytes_per_launch"]) if rec.get("kernel_code_sha256") == digest else None


def algorithmic_kv_bytes(w) -> int:
    """K and V of every valid token of every kv head, once per sequence."""
    return int(w.seq_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_size * w.kv_dtype_bytes


def algorithmic_bytes(w) -> int:
    """Bytes the decode step must move: K and V of every valid token of every
    kv head (at the cache's element size), the query rows read, the fp32
    outputs written, the block-table entries in use and the lengths."""
    L = w.seq_lens.astype(np.int64)
    kv = int(L.sum()) * 2 * w.num_kv_heads * w.head_size * w.kv_dtype_bytes
    q = w.num_tokens * w.num_q_heads * w.head_size * w.dtype_bytes
    out = w.num_tokens * w.num_q_heads * w.head_size * 4
    tables = int(((L + 15) // 16).sum()) * 4
    qsl = 4 * (w.batch + 1) if w.num_tokens != w.batch else 0
    return kv + q + out + tables + 4 * w.batch + qsl


def unique_kv_bytes(w, tables) -> int:
    """K/V bytes of the distinct physical blocks the batch reads (a block
    shared by several sequences counted once, with the most tokens any of
    them reads from it)."""
    used = {}
    for s in range(w.batch):
        L = int(w.seq_lens[s])
        for j in range(-(-L // 16)):
            b = int(tables[s][j])
            used[b] = max(used.get(b, 0), min(16, L - 16 * j))
    return sum(used.values()) * 2 * w.num_kv_heads * w.head_size * w.kv_dtype_bytes


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(rows, dtype, scale, seconds, ready, start, out):
    """Worker of the CPU baseline: its share of decode rows arrives with the
    process; after every worker is ready it computes the oracle's rows over
    and over with one BLAS thread for `seconds` and reports the rows done."""
    from threadpoolctl import threadpool_limits

    from oracle import paged_oracle as po
    done = 0
    with threadpool_limits(1):
        ready.put(1)
        start.wait()
        deadline = time.time() + seconds
        while time.time() < deadline:
            for q, K, V, L in rows:
                po.attention_rows(po.decode(q, dtype), po.decode(K, dtype), po.decode(V, dtype),
                                  [L - 1], scale)
                done += 1
                if time.time() >= deadline:
                    break
    out.put(done)


def cpu_baseline(w, seconds: float = 12.0):
    """The oracle (unchanged) on every host core, before the GPU is touched:
    one spawned worker process per core with one BLAS thread, each given its
    share of the batch's decode rows (query codes and the sequence's K/V
    codes in logical order, dealt round-robin in a seeded random order) and
    computing textbook fp64 attention of those rows, all heads, over and
    over for a fixed wall time that starts once every worker holds its data.
    The rate is rows per second over all workers."""
    import multiprocessing as mp

    from oracle import scenario
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    workers = max(1, min(cores, 32))
    order = np.random.default_rng(1).permutation(w.batch)
    qsl = w.query_start_loc
    shares = [[] for _ in range(workers)]
    for i, s in enumerate(order):
        K, V = scenario.sequence_kv(w, int(s))
        shares[i % workers].append((w.q[qsl[s]:qsl[s] + 1], K, V, int(w.seq_lens[s])))
    ctx = mp.get_context("spawn")
    ready, out, start = ctx.Queue(), ctx.Queue(), ctx.Event()
    procs = [ctx.Process(target=_oracle_worker,
                         args=(sh, w.dtype, w.scale, seconds, ready, start, out))
             for sh in shares]
    for pr in procs:
        pr.start()
    for _ in procs:
        ready.get(timeout=600)
    t0 = time.time()
    start.set()
    rows = sum(out.get(timeout=600 + seconds) for _ in procs)
    dt = time.time() - t0
    for pr in procs:
        pr.join()
    return {"value": rows / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cores": os.cpu_count(),
            "sample": f"{rows} decode rows of this batch (all {w.num_q_heads} heads each) in "
                      f"{dt:.1f} s on {workers} worker processes, fp64 NumPy, one BLAS thread "
                      f"each"}


def prefill_flops(w) -> float:
    """Multiply-adds of the chunk's unmasked (query, key) pairs, 2 flops
    each, for Q.K^T and P.V over all query heads."""
    total = 0.0
    for s in range(w.batch):
        ql = int(w.q_len[s])
        if ql <= 1:
            continue
        first = int(w.seq_lens[s]) - ql
        pairs = sum(first + i + 1 for i in range(ql))
        total += 4.0 * w.head_size * w.num_q_heads * pairs
    return total


def make_flush(mb: int):
    """A callable that reads `mb` MiB of scratch on the current stream (no-op for 0).

    Run before every timed step so that no step finds the previous step's data
    in the 256 MB Infinity Cache or its translations in the TLBs.  It reads
    rather than writes: a written flush leaves dirty lines whose write-back
    then lands inside the timed call (on the 8B GQA decode step that costs
    +33%, against +9% for the read, and 2 ms of idle time in between changes
    neither)."""
    import torch
    if mb <= 0:
        return lambda: None
    buf = torch.ones((mb << 20) // 4, dtype=torch.int32, device="cuda")
    return lambda: buf.sum()


def _timed(fn, steps, warmup, stream, flush=None):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush()
        a, b = ev[i]
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def copy_bandwidth(nbytes=1 << 30):
    """Device-to-device copy rate on this GPU (read + write bytes / time)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = _timed(lambda: dst.copy_(src), 10, 3, torch.cuda.current_stream())
    return 2 * nbytes / (float(np.median(ms)) * 1e-3) / 1e9


MFMA_PEAK_TFLOPS = 2500.0  # bf16 dense


def measure_mixed(steps: int, warmup: int, flush_mb: int):
    """The 8B GQA mixed step (98 decode rows + a 1950-row chunk on 1048 cached
    tokens): the whole mixed call, and the chunk's rows alone through the
    same entry point.  Returns (mixed_step, prefill_chunk) records."""
    import torch

    import workloads
    from paged_kv_attention_06_amd import _lib as L
    from paged_kv_attention_06_amd import step as gpu_step

    w = workloads.make(4)
    st = gpu_step.PagedStep(w, "cuda")
    st.build_history()
    st.prepare_step()
    st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    flush = make_flush(flush_mb)
    mixed_ms = _timed(st.attend, steps, warmup, stream, flush)
    # the chunk alone: same call restricted to the prefill sequence
    s = int(np.argmax(w.q_len))
    r0, r1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
    sub_qsl = np.array([0, r1 - r0], np.int32)
    sub_len = w.seq_lens[s:s + 1].astype(np.int32)
    d_qsl = torch.from_numpy(sub_qsl).cuda()
    d_len = torch.from_numpy(sub_len).cuda()
    d_bt = st.block_tables[s:s + 1].contiguous()
    q = st.q[r0:r1].contiguous()
    out = torch.empty((r1 - r0, w.num_q_heads, w.head_size), dtype=torch.float32, device="cuda")
    ws_bytes = L.pkv_attention_workspace_bytes(st.cache, w.num_q_heads, sub_len, sub_qsl)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def prefill():
        L.paged_attention_mixed(st.cache, out, q, d_qsl, d_len, sub_qsl, sub_len, d_bt, w.scale,
                                ws)

    pre_ms = _timed(prefill, steps, warmup, stream, flush)
    torch.cuda.synchronize()
    # The mixed call runs the chunk in 4-wave workgroups beside the decode
    # rows; alone it may split each q tile's keys over two groups, which
    # changes the summation order, not the result beyond rounding.
    alone_vs_mixed = float((out - st.out[r0:r1]).abs().max())
    assert alone_vs_mixed <= 5e-3, f"prefill-alone rows differ from the mixed call's: {alone_vs_mixed}"
    # k_prefill_split when every (q tile, kv head) item has a CU of its own
    items = -(-(r1 - r0) // (128 // (w.num_q_heads // w.num_kv_heads))) * w.num_kv_heads
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    forced = os.environ.get("PKV_PREFILL_SPLIT")
    split = forced == "1" or (forced != "0" and items <= cus)
    chunk_kernel = "k_prefill_split" if split else "k_prefill_tile"
    flops = prefill_flops(w)
    pre_mean = float(pre_ms.mean())
    tflops = flops / (pre_mean * 1e-3) / 1e12
    mixed_mean = float(mixed_ms.mean())
    # bytes the whole call must move (every sequence's K/V once, q, out,
    # tables, lengths, query_start_loc) and those of the decode rows alone
    all_bytes = algorithmic_bytes(w)
    dec = np.flatnonzero(w.q_len == 1)
    dec_bytes = (int(w.seq_lens[dec].astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_size * 2
                 + len(dec) * w.num_q_heads * w.head_size * (2 + 4)
                 + int(((w.seq_lens[dec].astype(np.int64) + 15) // 16).sum()) * 4 + 4 * len(dec))
    bound_ms = all_bytes / (HBM_PEAK_GBPS * 1e9) * 1e3 + flops / (MFMA_PEAK_TFLOPS * 1e12) * 1e3
    mixed_rec = {
        "ms": mixed_mean,
        "ms_median_p10_p90": [float(np.median(mixed_ms)), float(np.percentile(mixed_ms, 10)),
                              float(np.percentile(mixed_ms, 90))],
        "workload": "8B GQA mixed step: 98 decode rows (contexts U[64,4096]) + one 1950-token "
                    "prefill chunk on 1048 cached tokens, 2048 new tokens",
        "roofline": {"bound": "hbm+mfma (serialized)", "achieved_ms": mixed_mean,
                     "bound_ms": bound_ms, "frac": bound_ms / mixed_mean,
                     "algorithmic_bytes": all_bytes, "algorithmic_flops": flops,
                     "peaks": {"hbm_GBps": HBM_PEAK_GBPS, "mfma_TFLOPs": MFMA_PEAK_TFLOPS},
                     "traffic": None},
        "decode_rows_bytes": dec_bytes,
        "decode_rows_pct_hbm_peak_over_the_call": 100.0 * dec_bytes / (mixed_mean * 1e-3) / 1e9
        / HBM_PEAK_GBPS,
        "kernels": "k_v_fp16 + k_prefill_tile on the side stream beside k_decode_stream",
    }
    prefill_rec = {
        "ms": pre_mean,
        "ms_median_p10_p90": [float(np.median(pre_ms)), float(np.percentile(pre_ms, 10)),
                              float(np.percentile(pre_ms, 90))],
        "workload": "the mixed step's 1950-row chunk alone (1048 cached tokens, causal), 8B GQA",
        "gflop": flops / 1e9,
        "alone_vs_mixed_max_abs": alone_vs_mixed,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "k_v_fp16 + " + chunk_kernel,
                     "algorithmic_flops_per_launch": flops},
    }
    del st
    return mixed_rec, prefill_rec


def measure_gather(st, w, steps: int, warmup: int, flush_mb: int, decode_ms: float):
    """The read ceiling of the decode batch's access pattern: pkv_read_slices
    over the (block, kv head) slices the decode reads, in its order
    (sequence, kv head, block), with as many waves as the decode and the same
    1 GiB read before every call."""
    import torch

    from paged_kv_attention_06_amd import _lib as L
    ids = []
    for s in range(w.batch):
        nb = -(-int(w.seq_lens[s]) // 16)
        row = st.tables[s][:nb].astype(np.int64) * w.num_kv_heads
        for h in range(w.num_kv_heads):
            ids.append(row + h)
    ids = torch.from_numpy(np.concatenate(ids)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = 8 * cus
    sink = torch.empty(waves, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = _timed(lambda: L.pkv_read_slices(st.cache, ids, waves, sink), steps, warmup, stream,
                make_flush(flush_mb))
    ms_b2b = _timed(lambda: L.pkv_read_slices(st.cache, ids, waves, sink), steps, warmup, stream)
    slice_bytes = 2 * 16 * w.head_size * w.kv_dtype_bytes
    nbytes = int(ids.shape[0]) * slice_bytes
    mean = float(ms.mean())
    gbps = nbytes / (mean * 1e-3) / 1e9
    return {
        "ms": mean, "ms_back_to_back": float(ms_b2b.mean()),
        "bytes_read": nbytes, "slices": int(ids.shape[0]), "waves": waves,
        "gbps": gbps, "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "gbps_back_to_back": nbytes / (float(ms_b2b.mean()) * 1e-3) / 1e9,
        "decode_call_vs_probe_time": decode_ms / mean,
        "kernel": "pkv_read_slices (k_read_slices): the decode's slices read once, no arithmetic",
    }


def run_mixed(args):
    mixed, prefill = measure_mixed(args.steps, args.warmup, args.flush_mb)
    return {
        "metric": "mixed chunked-prefill step: attention ms and prefill-tile MFMA TFLOP/s",
        "value": mixed["ms"], "unit": "ms", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": mixed["ms"],
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": mixed["workload"],
                   "flush_mb_read_before_each_step": args.flush_mb},
        "mixed_step": mixed, "prefill_chunk": prefill,
        "roofline": prefill["roofline"],
    }


def run_prefill(args):
    """One prefill chunk alone in the 8B GQA shape (32 q / 8 kv heads, head
    128, bf16): `--chunk-rows` causal query rows on `--cached` cached
    tokens, through paged_attention_mixed."""
    import torch

    import workloads
    from paged_kv_attention_06_amd import step as gpu_step

    rows, cached = args.chunk_rows, args.cached
    if rows < 2 or cached < 0:
        raise SystemExit("--chunk-rows must be >= 2 and --cached >= 0")
    streams = [np.random.default_rng(x)
               for x in np.random.SeedSequence(4_000 + rows + 7 * cached).spawn(4)]
    blocks = -(-(cached + rows) // 16)
    w = workloads._build(4, f"8B GQA prefill chunk: {rows} rows on {cached} cached tokens", "bf16",
                         32, 8, 128, 128 ** -0.5, np.array([cached], np.int32),
                         np.array([rows], np.int32), blocks + blocks // 4 + 8, streams)
    st = gpu_step.PagedStep(w, "cuda")
    st.build_history()
    st.prepare_step()
    st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    flush = make_flush(args.flush_mb)
    ms = _timed(st.attend, args.steps, args.warmup, stream, flush)
    flops = prefill_flops(w)
    mean = float(ms.mean())
    tflops = flops / (mean * 1e-3) / 1e12
    # the kernel the library picks for this call (see the tuning switches)
    items = -(-rows // 32) * w.num_kv_heads
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    forced = os.environ.get("PKV_PREFILL_SPLIT")
    if rows <= 8 and os.environ.get("PKV_PREFILL_MQ") != "0":
        kernel = "k_prefill_mq"
    elif rows <= 64 and os.environ.get("PKV_PREFILL_V") != "fp16":
        kernel = "k_prefill_tile (bf16 V from the pool)"
    else:
        split = forced == "1" or (forced != "0" and items <= cus)
        kernel = "k_v_fp16 + " + ("k_prefill_split" if split else "k_prefill_tile")
    return {
        "metric": "prefill chunk alone: MFMA TFLOP/s of the unmasked (query, key) pairs",
        "value": tflops, "unit": "TFLOP/s", "higher_is_better": True,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": mean,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "flush_mb_read_before_each_step": args.flush_mb},
        "attention_ms_median": float(np.median(ms)),
        "items_q_tile_x_kv_head": items,
        "gflop": flops / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tflops / 2500.0, "traffic": None, "kernel": kernel,
                     "algorithmic_flops_per_launch": flops},
    }


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction


def run_swap(args):
    """Swap preemption's data move: all blocks of the 32 longest sequences of
    the 8B GQA decode batch go out to pinned host memory and come back."""
    import torch

    import workloads
    from paged_kv_attention_06_amd import _lib as L
    from paged_kv_attention_06_amd import step as gpu_step

    w = workloads.make(3)
    st = gpu_step.PagedStep(w, "cuda")
    st.build_history()
    st.prepare_step()
    torch.cuda.synchronize()
    longest = np.argsort(-w.seq_lens)[:32]
    blocks = [int(b) for s in longest for b in st.tables[s][:-(-int(w.seq_lens[s]) // 16)]]
    n = len(blocks)
    host = torch.empty(n * st.block_bytes, dtype=torch.uint8, pin_memory=True)
    used = {int(b) for s in range(w.batch) for b in st.tables[s][:-(-int(w.seq_lens[s]) // 16)]}
    fresh = [b for b in range(w.num_blocks) if b not in used][:n]
    out_pairs = torch.tensor([[b, i] for i, b in enumerate(blocks)], dtype=torch.int64).cuda()
    in_pairs = torch.tensor([[i, b] for i, b in enumerate(fresh)], dtype=torch.int64).cuda()
    stream = torch.cuda.current_stream()
    t_out = _timed(lambda: L.block_swap(st.cache, host, out_pairs, True), args.steps,
                   args.warmup, stream)
    t_in = _timed(lambda: L.block_swap(st.cache, host, in_pairs, False), args.steps,
                  args.warmup, stream)
    nbytes = n * st.block_bytes
    gb_out = nbytes / (float(t_out.mean()) * 1e-3) / 1e9
    gb_in = nbytes / (float(t_in.mean()) * 1e-3) / 1e9
    return {
        "metric": "block swap GB/s over the host link (swap out / swap in)",
        "value": gb_out, "unit": "GB/s", "higher_is_better": True, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": float(t_out.mean()),
        "scaling": "weak", "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": f"8B GQA pool (64 KiB blocks): all {n} blocks of the 32 longest "
                               f"sequences ({nbytes / 2**20:.0f} MiB) to pinned host memory and back"},
        "swap_out_ms": float(t_out.mean()), "swap_in_ms": float(t_in.mean()),
        "swap_out_gbps": gb_out, "swap_in_gbps": gb_in,
        "roofline": {"bound": "host link", "achieved": gb_out, "peak": HOST_LINK_PEAK_GBPS,
                     "unit": "GB/s", "frac": gb_out / HOST_LINK_PEAK_GBPS, "traffic": None,
                     "kernel": "block_swap (k_block_swap)", "algorithmic_bytes_per_launch": nbytes},
    }


def run_prefix_cache(args):
    """Host prefix caching (pkv_pool_match_prefix / append / cache_blocks /
    release) on the pages' shared-prefix example: requests share a 341-token
    few-shot prefix and add 16..400 tokens of their own; 256 are alive at a
    time in a 200,000-block pool, the oldest finishing as new ones arrive."""
    from paged_kv_attention_06_amd import _lib as L

    rng = np.random.default_rng(5)
    n_req = 20000
    prefix = rng.integers(0, 32000, size=341).tolist()
    reqs = [prefix + rng.integers(0, 32000, size=int(rng.integers(16, 401))).tolist()
            for _ in range(n_req)]
    pool = L.Pool(200_000, rng.permutation(200_000).astype(np.int32))
    live = []
    hit_blocks = full_blocks = saved_tokens = all_tokens = 0
    t0 = time.perf_counter()
    for toks in reqs:
        if len(live) >= 256:
            t, n = live.pop(0)
            pool.release(t, n)
        table = np.zeros(64, np.int32)
        hits = pool.match_prefix(toks, table)
        pool.append(table, hits * 16, len(toks) - hits * 16)
        pool.cache_blocks(toks, table, len(toks) // 16)
        live.append((table, -(-len(toks) // 16)))
        hit_blocks += hits
        full_blocks += len(toks) // 16
        saved_tokens += hits * 16
        all_tokens += len(toks)
    dt = time.perf_counter() - t0
    return {
        "metric": "host prefix caching: requests/s through match + append + register + release",
        "value": n_req / dt, "unit": "requests/s", "higher_is_better": True, "n_gpus": 1,
        "steps": n_req, "warmup": 0, "ms_per_step": dt / n_req * 1e3, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32 token ids", "data": "synthetic",
        "config": {"workload": "requests sharing one 341-token prefix (21 full blocks) plus "
                               "16..400 tokens of their own; 256 alive; 200,000-block pool"},
        "block_hit_rate": hit_blocks / full_blocks,
        "prefill_tokens_saved": saved_tokens / all_tokens,
        "us_per_request": dt / n_req * 1e6,
        "note": "host C++ through ctypes (the per-call ctypes marshalling is included); a step "
                "is one request, all 20,000 timed whatever --steps says",
    }


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["decode", "mixed", "decode-fp8", "verify", "swap",
                                           "prefix-cache", "decode-7b", "decode-13b", "tiny",
                                           "prefill"],
                    default="decode",
                    help="decode: the headline 8B GQA batch-256 step; mixed: the chunked "
                         "prefill step; decode-fp8: the headline step on an FP8 E4M3 KV "
                         "cache; verify: the same batch querying k + 1 = 4 positions per "
                         "sequence (speculative decoding); all but decode are reported "
                         "separately")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="decode workload: skip the read ceiling, mixed step and prefill chunk")
    ap.add_argument("--chunk-rows", type=int, default=512,
                    help="prefill workload: query rows of the chunk")
    ap.add_argument("--cached", type=int, default=1048,
                    help="prefill workload: cached tokens before the chunk")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="read this many MiB of scratch before every timed step, so that no "
                         "step reuses the last one's cached data (0 = back to back)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: run with --gpus 1"}))
        sys.exit(2)

    if args.workload == "prefix-cache":
        print(json.dumps(run_prefix_cache(args)), flush=True)
        return

    import workloads

    lib = os.path.join(ROOT, "paged_kv_attention_06_amd", "libpkv.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()

    fp8 = args.workload == "decode-fp8"
    verify = args.workload == "verify"
    other = {"decode-7b": 2, "decode-13b": 5, "tiny": 1}.get(args.workload)
    headline = args.workload == "decode"
    w = None
    cpu = None
    if args.workload not in ("mixed", "swap", "prefill"):
        if fp8:
            w = workloads.make_fp8(3)
        elif verify:
            w = workloads.make_verify()
        else:
            w = workloads.make(other or 3)
        # the oracle on the host cores, before anything touches the GPU
        if headline and not args.no_cpu_baseline:
            cpu = cpu_baseline(w)

    import torch

    from paged_kv_attention_06_amd import step as gpu_step

    if args.workload == "mixed":
        print(json.dumps(run_mixed(args)), flush=True)
        return
    if args.workload == "swap":
        print(json.dumps(run_swap(args)), flush=True)
        return
    if args.workload == "prefill":
        print(json.dumps(run_prefill(args)), flush=True)
        return

    st = gpu_step.PagedStep(w, "cuda")
    st.build_history()
    st.prepare_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    flush = make_flush(args.flush_mb)

    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    def timed_loop(flush_fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            flush_fn()
            a, b, c = ev[i]
            a.record(stream)
            st.copy_and_write()
            b.record(stream)
            st.attend()
            c.record(stream)
        torch.cuda.synchronize()
        return ev, time.perf_counter() - t0

    ev, wall = timed_loop(flush)
    # the same steps back to back, for reference (cache state left by the last step)
    ev_warm, _ = timed_loop(lambda: None) if args.flush_mb > 0 else (ev, wall)
    attn_warm = float(np.mean([b.elapsed_time(c) for _, b, c in ev_warm]))

    step_ms = np.array([a.elapsed_time(c) for a, _, c in ev])
    attn_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    ms_per_step = float(step_ms.mean())
    attn_mean = float(attn_ms.mean())
    alg = algorithmic_bytes(w)
    achieved = alg / (attn_mean * 1e-3) / 1e9
    value = w.num_tokens / (ms_per_step * 1e-3)

    rec = {
        "metric": (METRIC if not (fp8 or verify or other) else
                   {1: "decode step latency (launch-bound): 4 fp32 sequences, head 64",
                    2: "decode attention tokens/s & achieved HBM GB/s (% of peak), 7B-MHA batch 64",
                    5: "decode attention tokens/s & achieved HBM GB/s (% of peak), 13B-MHA batch "
                       "32, shared prefix + long context"}[other] if other else
                   "decode attention tokens/s & achieved HBM GB/s (% of peak), 8B-GQA batch 256, "
                   + ("FP8 KV cache" if fp8 else "speculative verify, 4 query rows per sequence")),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 cache, bf16 q, f32 accumulate" if fp8 else
                  "f32" if other == 1 else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": ({1: "tiny decode: 4 sequences of 5, 16, 17, 40 tokens, 4 q = 4 kv heads, "
                             "head 64, fp32 U[-1,1], 64-block pool",
                          2: "Llama-7B-shaped MHA decode: 32 q / 32 kv heads, head 128, bf16 "
                             "N(0,1), batch 64, contexts U[128, 2048], pool 1.25x the blocks "
                             "needed, shuffled",
                          5: "13B-shaped MHA decode: 40 / 40 heads, head 128, bf16 N(0,1), "
                             "16 forks of a 1032-token prompt (copy-on-write of the shared "
                             "partial block in the step) + 16 sequences U[1, 16384] incl. "
                             "one at 16384"}[other] if other else
                        "Llama-3-8B-shaped GQA decode: 32 q / 8 kv heads, head 128, bf16 "
                        "N(0,1), batch 256, lognormal contexts (median 800, sigma 1, "
                        "clipped 16..8192), 16-token blocks scattered in a 200,000-block pool")
                        + (", KV cache FP8 E4M3 with K/V scales 1/64" if fp8 else "")
                        + (", each sequence appends and queries its last token plus 3 draft "
                           "tokens (causal)" if verify else ""),
            "global_batch": w.batch,
            "sum_context_tokens": int(w.seq_lens.sum()),
            "parallelism": "none (1 GPU)",
            "flush_mb_read_before_each_step": args.flush_mb,
        },
        "attention_ms": attn_mean,
        "attention_ms_back_to_back": attn_warm,
        "pct_hbm_peak_back_to_back": 100.0 * alg / (attn_warm * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "attention_ms_median": float(np.median(attn_ms)),
        "attention_ms_p10_p90": [float(np.percentile(attn_ms, 10)), float(np.percentile(attn_ms, 90))],
        "write_ms": float((step_ms - attn_ms).mean()),
        "hbm_gbps": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "unique_kv_bytes": unique_kv_bytes(w, st.tables),
        "hbm_gbps_unique_blocks": (alg - algorithmic_kv_bytes(w) + unique_kv_bytes(w, st.tables))
        / (attn_mean * 1e-3) / 1e9,
        "device_copy_gbps": copy_bandwidth(),
        "wall_s_timed_region": wall,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None if other else measured_traffic(
                "verify_8b_gqa_b256_k3" if verify else
                "decode_8b_gqa_b256_fp8" if fp8 else "decode_8b_gqa_b256"),
            "kernel": ("paged_attention_mixed (k_prefill_mq)" if verify else
                       "paged_attention_decode (k_decode_stream, one launch)"),
            "algorithmic_bytes_per_launch": alg,
        },
        "cpu_baseline": cpu,
    }
    if headline and not args.headline_only:
        # beside the headline: the read ceiling of this batch's access
        # pattern, then the mixed chunked-prefill step and its chunk alone
        rec["gather_ceiling"] = measure_gather(st, w, args.steps, args.warmup, args.flush_mb,
                                               attn_mean)
        del st
        torch.cuda.empty_cache()
        rec["mixed_step"], rec["prefill_chunk"] = measure_mixed(args.steps, args.warmup,
                                                                args.flush_mb)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
