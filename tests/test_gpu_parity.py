"""Parity of the HIP path with the fp64 oracle, on the GPU.

Bars: KV writes, block copies, slots and tables bit-exact; attention within
max|d| <= 5e-3 and relative L2 <= 1e-3 for bf16 inputs (fp32 accumulation),
and within 1e-5 for the fp32 tiny decode.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import paged_oracle as po
from oracle import scenario

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_attention_06_amd import step as gpu_step  # noqa: E402

MAX_ABS_BF16, REL_L2_BF16 = 5e-3, 1e-3
MAX_ABS_F32 = 1e-5


def _announce(what):
    print(f"\n[gpu case] {what}", file=sys.stderr, flush=True)


def _check_attention(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    diff = np.abs(gpu.astype(np.float64) - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(gpu.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-30))
    if dtype == "f32":
        assert max_abs <= MAX_ABS_F32, f"{what}: max|d| {max_abs:.3e}"
    else:
        assert max_abs <= MAX_ABS_BF16, f"{what}: max|d| {max_abs:.3e}"
        assert rel <= REL_L2_BF16, f"{what}: rel L2 {rel:.3e}"
    return max_abs, rel


@pytest.mark.parametrize("cfg", [1, 2, 3, 5, 4])
def test_small_workload_full_parity(cfg):
    """Whole pool bit-exact and every output row within tolerance."""
    w = workloads.small(cfg)
    _announce(f"small {w.name}: B={w.batch} T={w.num_tokens} L={w.seq_lens.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.h_slots, ref["slots"])
    assert np.array_equal(st.h_cow, ref["cow_pairs"])
    pool = st.pool_codes()
    assert np.array_equal(pool, ref["pool"]), "pool differs from the oracle's"
    _check_attention(st.out.cpu().numpy(), ref["out"], w.dtype, f"small {w.name}")


def _blocks_of(st, w, ids):
    """Codes of whole blocks [n][Hkv][2][16 D] gathered on the GPU."""
    bb = st.block_bytes
    es = st.es
    view = st.kv.view(w.num_blocks, bb)
    idx = torch.as_tensor(np.asarray(ids, np.int64), device=st.kv.device)
    raw = view.index_select(0, idx).cpu().numpy().view({1: np.uint8, 2: np.uint16, 4: np.uint32}[es])
    return raw.reshape(len(ids), w.num_kv_heads, 2, 16 * w.head_size)


@pytest.mark.parametrize("cfg", [2, 3, 5, 4])
def test_full_size_parity(cfg):
    """Full-size workload in the bench's launch configuration: every decode
    row against the oracle (for the mixed step also every 5th row of the
    chunk and its last), every written token at the oracle's slot with its
    drawn values, and every copy-on-write destination equal to its source."""
    w = workloads.make(cfg)
    _announce(f"full {w.name}: B={w.batch} T={w.num_tokens} blocks={w.num_blocks}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    assert np.all(np.isfinite(out)), "non-finite output"
    qsl = w.query_start_loc
    got, want = [], []
    for s in range(w.batch):
        q_len = int(w.q_len[s])
        rows = [0] if q_len == 1 else sorted(set(range(0, q_len, 5)) | {q_len - 1})
        want.append(scenario.sequence_attention(w, s, rows))
        got.append(out[qsl[s] + np.asarray(rows)])
    _check_attention(np.concatenate(got), np.concatenate(want), w.dtype, f"full {w.name}")

    # the step's written tokens sit at the oracle's slots with their drawn values
    tabs = scenario.build_tables(w, with_pool=False)
    assert np.array_equal(st.h_slots, tabs["slots"])
    assert np.array_equal(st.h_cow, tabs["cow_pairs"])
    kidx = po.k_tile_index(w.head_size, w.dtype)
    vidx = po.v_tile_index(w.head_size, w.dtype)
    slots = tabs["slots"]
    for a in range(0, len(slots), 512):
        part = slots[a:a + 512]
        blocks = _blocks_of(st, w, part // 16)
        for i, slot in enumerate(part):
            off = int(slot) % 16
            t = a + i
            assert np.array_equal(blocks[i, :, 0][:, kidx[off]], w.new_k[t]), f"K of token {t}"
            assert np.array_equal(blocks[i, :, 1][:, vidx[off]], w.new_v[t]), f"V of token {t}"
    # a copy-on-write destination holds its source's tokens before the append
    pairs = tabs["cow_pairs"]
    if len(pairs):
        src, dst = _blocks_of(st, w, pairs[:, 0]), _blocks_of(st, w, pairs[:, 1])
        n_old = int(w.prompt_len[0]) % 16
        for off in range(n_old):
            assert np.array_equal(src[:, :, 0][:, :, kidx[off]], dst[:, :, 0][:, :, kidx[off]])
            assert np.array_equal(src[:, :, 1][:, :, vidx[off]], dst[:, :, 1][:, :, vidx[off]])


def test_decode_is_deterministic_and_layout_invariant():
    """Two runs give identical bits; moving every block to another physical
    id (a different free order) gives identical bits too."""
    w = workloads.small(3)
    _announce("determinism / block permutation, small 8B GQA decode")
    a = gpu_step.run_workload(w).out.cpu().numpy()
    b = gpu_step.run_workload(w).out.cpu().numpy()
    assert np.array_equal(a, b)
    w2 = workloads.small(3)
    w2.free_order = np.random.default_rng(99).permutation(w2.num_blocks).astype(np.int32)
    c = gpu_step.run_workload(w2).out.cpu().numpy()
    assert np.array_equal(a, c)


def test_empty_sequence_row_is_zero():
    w = workloads.small(3)
    w.hist_len = w.hist_len.copy()
    _announce("empty decode row")
    st = gpu_step.PagedStep(w)
    st.build_history()
    st.prepare_step()
    st.copy_and_write()
    st.h_seq_lens = st.h_seq_lens.copy()
    st.h_seq_lens[1] = 0
    st.seq_lens = torch.from_numpy(st.h_seq_lens).cuda()
    st.out.fill_(7.0)
    st.attend()
    torch.cuda.synchronize()
    out = st.out.cpu().numpy()
    assert np.all(out[1] == 0)
    ref = scenario.run_step(w)["out"]
    keep = [s for s in range(w.batch) if s != 1]
    _check_attention(out[keep], ref[keep], w.dtype, "rows next to an empty one")


def test_split_boundaries():
    """Lengths at and around the 256-token partition and 16-token block edges."""
    lens = [1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1024, 1025]
    w = workloads.small(3)
    B = len(lens)
    rng = np.random.default_rng(5)
    L = np.asarray(lens, np.int32)
    w2 = workloads._build(3, "split edges", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                          np.ones(B, np.int32), 400, [rng, np.random.default_rng(6),
                                                       np.random.default_rng(7), rng])
    _announce(f"split boundaries L={lens}")
    st = gpu_step.run_workload(w2)
    ref = scenario.run_step(w2)
    assert np.array_equal(st.pool_codes(), ref["pool"])
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", "split boundaries")
    del w


def test_many_sequences_and_long_rows():
    """More sequences than one 256-wide length scan covers, and rows longer
    than 64 partitions."""
    rng = np.random.default_rng(11)
    B = 600
    L = rng.integers(1, 600, size=B, endpoint=True).astype(np.int32)
    L[7] = 20000                                    # 79 partitions of 256
    streams = [np.random.default_rng(x) for x in (21, 22, 23, 24)]
    pool = int(1.25 * sum((int(x) + 15) // 16 for x in L)) + 1
    w = workloads._build(3, "many seqs", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                         np.ones(B, np.int32), pool, streams)
    _announce(f"many sequences B={B}, longest {int(L.max())}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    rows = [0, 7, 255, 256, 257, 511, 512, 599]
    want = np.concatenate([scenario.sequence_attention(w, s) for s in rows])
    got = np.concatenate([out[s:s + 1] for s in rows])
    _check_attention(got, want, "bf16", "many sequences")


def _times_pow2(codes: np.ndarray, k: int) -> np.ndarray:
    """bf16 codes times 2^k, exactly (exponent field + k; zeros stay zero)."""
    out = codes.copy()
    nz = (out & 0x7F80) != 0
    out[nz] = out[nz] + np.uint16(k << 7)
    return out


def test_prefill_values_beyond_fp16_range():
    """V values of magnitude >= 2^16 in some blocks of a prefill sequence: the
    prefill path's power-of-two block scaling (both directions) against the
    oracle.  The absolute bar scales with the output's magnitude here."""
    w = workloads.small(4)
    s = w.batch - 1                                   # the prefill chunk
    a, b = int(w.hist_start[s]), int(w.hist_start[s + 1])
    hv = w.hist_v.copy()
    hv[a + 3:a + 9] = _times_pow2(hv[a + 3:a + 9], 22)      # ~4e6 in block 0
    hv[a + 20:a + 30] = _times_pow2(hv[a + 20:a + 30], 12)  # ~4e3, below 2^16
    w.hist_v = hv
    nv = w.new_v.copy()
    q0 = int(w.query_start_loc[s])
    nv[q0 + 60:q0 + 64] = _times_pow2(nv[q0 + 60:q0 + 64], 30)  # ~1e9 later on
    nv[q0 + 100:q0 + 101] = _times_pow2(nv[q0 + 100:q0 + 101], 17)
    w.new_v = nv
    _announce(f"prefill with |v| >= 2^16: L={int(w.seq_lens[s])} q_len={int(w.q_len[s])}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)["out"]
    got = st.out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    rows = slice(int(w.query_start_loc[s]), int(w.query_start_loc[s + 1]))
    for name, sl in (("prefill rows", rows), ("decode rows", slice(0, rows.start))):
        g, r = got[sl], ref[sl]
        scale = max(float(np.abs(r).max()), 1.0)
        max_abs = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        assert max_abs <= MAX_ABS_BF16 * scale, f"{name}: max|d| {max_abs:.3e} (scale {scale:.3e})"
        assert rel <= REL_L2_BF16, f"{name}: rel L2 {rel:.3e}"


def test_one_long_row_split_over_many_waves():
    """A single 32768-token row: each (row, kv head) item is split over more
    than 64 waves, so the in-kernel merge walks partials in several chunks."""
    L = np.array([32768], np.int32)
    streams = [np.random.default_rng(x) for x in (31, 32, 33, 34)]
    w = workloads._build(3, "one long row", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                         np.ones(1, np.int32), 2100, streams)
    _announce("one long row L=32768")
    st = gpu_step.run_workload(w)
    _check_attention(st.out.cpu().numpy(), scenario.sequence_attention(w, 0)[None],
                     "bf16", "one long row")


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_fixed_partition_decode_path(cfg, monkeypatch):
    """The fixed 256-token split-K path with its separate merge launch
    (PKV_DECODE_SPLIT=units), which mixed batches also use, on pure decode
    batches."""
    monkeypatch.setenv("PKV_DECODE_SPLIT", "units")
    w = workloads.small(cfg)
    _announce(f"units split, small {w.name}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    _check_attention(st.out.cpu().numpy(), ref["out"], w.dtype, f"units split {w.name}")


@pytest.mark.parametrize("size", ["small", "full"])
def test_fused_mixed_path(size, monkeypatch):
    """Mixed calls run the prefill tiles on the library's side stream beside
    the stream decode; PKV_MIXED=fused runs the single k_mixed launch (fixed
    decode partitions + merge launch) instead.  Both against the oracle, and
    the two paths against each other on the same step."""
    w = workloads.small(4) if size == "small" else workloads.make(4)
    _announce(f"fused mixed path, {size} {w.name}")
    st = gpu_step.run_workload(w)
    concurrent = st.out.cpu().numpy()
    monkeypatch.setenv("PKV_MIXED", "fused")
    st.out.fill_(0)
    st.attend()
    torch.cuda.synchronize()
    fused = st.out.cpu().numpy()
    if size == "small":
        ref = scenario.run_step(w)["out"]
        _check_attention(fused, ref, "bf16", "fused mixed")
        _check_attention(concurrent, ref, "bf16", "concurrent mixed")
    else:
        qsl = w.query_start_loc
        for s in range(w.batch):
            q_len = int(w.q_len[s])
            rows = [0] if q_len == 1 else sorted(set(range(0, q_len, 7)) | {q_len - 1})
            ref = scenario.sequence_attention(w, s, rows)
            _check_attention(fused[qsl[s] + np.asarray(rows)], ref, "bf16", f"fused sequence {s}")
    assert float(np.abs(fused - concurrent).max()) <= MAX_ABS_BF16, "fused and concurrent paths differ"


def test_workspace_reused_with_new_queries():
    """Two calls in a row on one workspace with different queries: the second
    call's merged rows must not see partials or counters left by the first."""
    import copy
    L = np.array([4000, 33, 2500, 700, 9000, 1], np.int32)
    streams = [np.random.default_rng(x) for x in (41, 42, 43, 44)]
    pool = int(1.25 * sum((int(x) + 15) // 16 for x in L)) + 1
    w = workloads._build(3, "reuse", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                         np.ones(len(L), np.int32), pool, streams)
    _announce("workspace reuse with new queries")
    st = gpu_step.run_workload(w)
    first = st.out.cpu().numpy()
    w2 = copy.copy(w)
    rng = np.random.default_rng(45)
    w2.q = workloads._bf16_codes(rng.standard_normal(w.q.shape).astype(np.float32))
    st.q.copy_(torch.from_numpy(w2.q.view(np.int16)).cuda())
    st.attend()
    torch.cuda.synchronize()
    second = st.out.cpu().numpy()
    for s in range(w.batch):
        _check_attention(first[s:s + 1], scenario.sequence_attention(w, s), "bf16", f"call 1 row {s}")
        _check_attention(second[s:s + 1], scenario.sequence_attention(w2, s), "bf16", f"call 2 row {s}")


def test_prefill_chunk_rows_dense_sample():
    """The 1950-row prefill chunk on 1048 cached tokens: its q tiles need 17
    to 47 key tiles and are split into key chunks merged in-launch, so every
    7th row (and the last) is checked against the oracle."""
    w = workloads.make(4)
    _announce(f"prefill chunk dense sample: T={w.num_tokens}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    s = int(np.argmax(w.q_len))
    ql = int(w.q_len[s])
    rows = sorted(set(range(0, ql, 7)) | {ql - 1})
    ref = scenario.sequence_attention(w, s, rows)
    got = out[int(w.query_start_loc[s]) + np.asarray(rows)]
    _check_attention(got, ref, "bf16", "prefill chunk rows")


# ------------------------------------------------- multi-query rows (k_prefill_mq)
@pytest.mark.parametrize("G,D", [(4, 128), (2, 128), (1, 128), (4, 64), (1, 64)])
def test_multi_query_rows(G, D, monkeypatch):
    """Pure prefill calls whose sequences all have at most 32 / G query rows
    go to k_prefill_mq (MFMA rows = the G heads x 32 / G positions).  Short
    and long histories, a sequence inside one block, q_len from 2 to 32 / G;
    every row against the oracle, and the same call through the tile kernel
    (PKV_PREFILL_MQ=0)."""
    rng = np.random.default_rng(90 + G + D)
    hkv = 4
    maxq = 32 // G
    ql = np.concatenate([[2, maxq, 3], rng.integers(2, maxq + 1, 9)]).astype(np.int32)
    hist = np.concatenate([[5, 0, 1000], rng.integers(0, 700, 9)]).astype(np.int32)
    hist[1] = max(0, 9 - int(ql[1]))  # L = 9 or q_len: one partly filled block
    streams = [np.random.default_rng(91 + G + D + x) for x in range(4)]
    pool = int(1.25 * sum((int(a) + int(b) + 15) // 16 for a, b in zip(hist, ql))) + 8
    w = workloads._build(4, "multi-query rows", "bf16", hkv * G, hkv, D, D ** -0.5,
                         hist, ql, pool, streams)
    _announce(f"multi-query rows G={G} D={D}: q_len={w.q_len.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"multi-query G={G} D={D}")
    monkeypatch.setenv("PKV_PREFILL_MQ", "0")
    st.out.fill_(0)
    st.attend()
    torch.cuda.synchronize()
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"tile kernel G={G} D={D}")


def test_multi_query_rows_many_sequences():
    """More sequences than the kernel arguments' longest-first order holds
    (1024): the workgroups take the sequences in index order instead."""
    rng = np.random.default_rng(97)
    n = 1100
    ql = rng.integers(2, 9, n).astype(np.int32)
    hist = rng.integers(0, 60, n).astype(np.int32)
    streams = [np.random.default_rng(98 + x) for x in range(4)]
    pool = int(1.25 * sum((int(a) + int(b) + 15) // 16 for a, b in zip(hist, ql))) + 8
    w = workloads._build(4, "multi-query rows, 1100 sequences", "bf16", 16, 4, 64, 64 ** -0.5,
                         hist, ql, pool, streams)
    _announce(f"multi-query rows, {n} sequences")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", "multi-query, 1100 sequences")


# ------------------------------------------------------------- FP8 KV cache
@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_fp8_small_workload_full_parity(cfg):
    """FP8 E4M3 cache: quantized writes give the oracle's pool bit for bit
    (every code and untouched byte), attention within the bars."""
    w = workloads.make_fp8(cfg, small_size=True)
    _announce(f"fp8 small {w.name}: B={w.batch} L={w.seq_lens.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"]), "fp8 pool differs from the oracle's"
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"fp8 small {w.name}")


@pytest.mark.parametrize("cfg", [3, 5])
def test_fp8_full_size_parity(cfg):
    """FP8 cache at full size: every decode row against the oracle."""
    w = workloads.make_fp8(cfg)
    _announce(f"fp8 full {w.name}: B={w.batch} blocks={w.num_blocks}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    assert np.all(np.isfinite(out))
    want = np.concatenate([scenario.sequence_attention(w, s) for s in range(w.batch)])
    _check_attention(out, want, "bf16", f"fp8 full {w.name}")


def test_fp8_every_code_decodes_exactly():
    """One token per sequence (its own, written this step): the output is
    that token's V times the V scale, exactly.  V holds every E4M3 code once
    (bf16 inputs equal to code value * scale, which quantize to the code);
    the stored bytes and the outputs are checked bit for bit."""
    streams = [np.random.default_rng(x) for x in (51, 52, 53, 54)]
    w = workloads._build(3, "fp8 codes", "bf16", 2, 2, 128, 128 ** -0.5, np.zeros(1, np.int32),
                         np.ones(1, np.int32), 4, streams)
    w.cache_dtype, w.k_scale, w.v_scale, w.pool_fill = "fp8", 0.5, 1.0 / 64, workloads.FP8_NAN
    table = po.e4m3_table()
    vals = (table * w.v_scale).astype(np.float32)              # exact in bf16 (4 significant bits)
    codes = np.arange(256).reshape(2, 128)
    w.new_v = workloads._bf16_codes(np.nan_to_num(vals, nan=0.0)[codes][None])
    nan = np.isnan(vals[codes])                                # codes 0x7F and 0xFF
    w.new_v[0][nan] = 0x7FC0 | ((codes[nan] & 0x80) << 8)      # NaN inputs with their sign
    w.new_k = np.zeros_like(w.new_v)
    _announce("fp8 every code")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"])
    blk = int(st.tables[0, 0])
    vt = st.pool_codes()[blk, :, 1].reshape(2, 128, 16)[:, :, 0]   # V of token 0, every d
    assert np.array_equal(vt, codes.astype(np.uint8)), "written codes"
    out = st.out.cpu().numpy()[0]                              # [Hq=2][128]
    want = vals[codes]
    assert np.array_equal(np.isnan(out), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(out[ok], want[ok]), "decoded values"


# ------------------------------------------------- speculative verify (q_len = k + 1)
def test_verify_small_full_parity():
    """Each sequence queries its last token and 3 draft tokens, causally."""
    w = workloads.make_verify(small_size=True)
    _announce(f"verify small: L={w.seq_lens.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"])
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", "verify small")


def test_verify_full_size_parity():
    """The full verify batch: every query row of every sequence."""
    w = workloads.make_verify()
    _announce(f"verify full: B={w.batch} T={w.num_tokens}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    assert np.all(np.isfinite(out))
    want = np.concatenate([scenario.sequence_attention(w, s) for s in range(w.batch)])
    _check_attention(out, want, "bf16", "verify full")


# ------------------------------------------------------------------ block swap
def test_block_swap_out_and_back_in():
    """Swap the blocks of two sequences out to pinned host memory (they equal
    the oracle pool's blocks bit for bit), then back in to other device
    blocks; with the tables rewritten, attention gives the same bits."""
    from paged_kv_attention_06_amd import _lib as L
    w = workloads.small(3)
    _announce("block swap out / in")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    before = st.out.cpu().numpy().copy()
    seqs = [3, 4]
    nblk = [-(-int(w.seq_lens[s]) // 16) for s in seqs]
    blocks = [int(b) for s, n in zip(seqs, nblk) for b in st.tables[s][:n]]
    bb = st.block_bytes
    host = torch.zeros(len(blocks) * bb, dtype=torch.uint8, pin_memory=True)
    out_pairs = torch.tensor([[b, i] for i, b in enumerate(blocks)], dtype=torch.int64).cuda()
    L.block_swap(st.cache, host, out_pairs, to_host=True)
    torch.cuda.synchronize()
    hp = host.numpy().view(np.uint16).reshape(len(blocks), w.num_kv_heads, 2, 16 * w.head_size)
    assert np.array_equal(hp, ref["pool"][blocks]), "swapped-out blocks"
    used = {int(b) for s in range(w.batch)
            for b in st.tables[s][:-(-int(w.seq_lens[s]) // 16)]}
    fresh = [b for b in range(w.num_blocks) if b not in used][:len(blocks)]
    in_pairs = torch.tensor([[i, b] for i, b in enumerate(fresh)], dtype=torch.int64).cuda()
    L.block_swap(st.cache, host, in_pairs, to_host=False)
    k = 0
    for s, n in zip(seqs, nblk):
        st.tables[s][:n] = fresh[k:k + n]
        k += n
    st.block_tables = torch.from_numpy(st.tables).cuda()
    st.out.fill_(0)
    st.attend()
    torch.cuda.synchronize()
    pool = st.pool_codes()
    assert np.array_equal(pool[fresh], ref["pool"][blocks]), "swapped-in blocks"
    assert np.array_equal(st.out.cpu().numpy(), before), "attention after swap in"


@pytest.mark.parametrize("vpath", ["bf16", "fp16"])
@pytest.mark.parametrize("case", ["verify", "chunk"])
def test_prefill_v_paths(case, vpath, monkeypatch):
    """Pure prefill calls read V either as bf16 straight from the pool (P as
    a bf16 hi + lo pair; keys past L zeroed in LDS) or from the fp16 copy;
    both against the oracle, on a verify batch and on a 150-row chunk that
    starts mid-block and ends in a partly filled block."""
    monkeypatch.setenv("PKV_PREFILL_V", vpath)
    if case == "verify":
        w = workloads.make_verify(small_size=True)
    else:
        streams = [np.random.default_rng(x) for x in (61, 62, 63, 64)]
        w = workloads._build(4, "chunk alone", "bf16", 32, 8, 128, 128 ** -0.5,
                             np.array([37], np.int32), np.array([150], np.int32), 40, streams)
    _announce(f"prefill V path {vpath}, {case}: L={w.seq_lens.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"{case} via {vpath} V")


# ------------------------------------- pure prefill, key tiles split over two groups
@pytest.mark.parametrize("split", ["1", "0"])
@pytest.mark.parametrize("G,D", [(4, 128), (2, 128), (1, 128), (4, 64), (1, 64)])
def test_prefill_split_groups(G, D, split, monkeypatch):
    """k_prefill_split (forced with PKV_PREFILL_SPLIT=1; chosen by itself when
    every item has a CU of its own): two 4-wave groups share each q tile's
    key tiles and merge (max, sum, O) in LDS.
    Histories from 0 to 1300 tokens give odd and even key-tile counts and
    q tiles of one key tile (group 1 idle).  V of magnitude >= 2^16 sits in
    keys that only one group reads, so the merge meets two different
    power-of-two exponents.  Every row against the oracle; the same batch
    through k_prefill_tile (PKV_PREFILL_SPLIT=0)."""
    monkeypatch.setenv("PKV_PREFILL_SPLIT", split)
    hist = np.array([0, 37, 1300, 64, 5], np.int32)
    ql = np.array([150, 70, 200, 2, 40], np.int32)      # longest > 64: fp16 V copy
    streams = [np.random.default_rng(x) for x in (71 + G, 72 + D, 73, 74)]
    w = workloads._build(0, "prefill split", "bf16", 2 * G, 2, D, D ** -0.5, hist, ql, 400, streams)
    s2 = int(w.hist_start[2])
    hv = w.hist_v.copy()
    hv[s2 + 900:s2 + 906] = _times_pow2(hv[s2 + 900:s2 + 906], 22)   # keys 900..905: second half
    w.hist_v = hv
    nv = w.new_v.copy()
    nv[10:13] = _times_pow2(nv[10:13], 20)                          # sequence 0, keys 10..12
    w.new_v = nv
    _announce(f"prefill split={split} G={G} D={D}: L={w.seq_lens.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)["out"]
    got = st.out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    qsl = w.query_start_loc
    for s in range(w.batch):
        g, r = got[qsl[s]:qsl[s + 1]], ref[qsl[s]:qsl[s + 1]]
        scale = max(float(np.abs(r).max()), 1.0)
        max_abs = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        assert max_abs <= MAX_ABS_BF16 * scale, f"seq {s}: max|d| {max_abs:.3e} (scale {scale:.3e})"
        assert rel <= REL_L2_BF16, f"seq {s}: rel L2 {rel:.3e}"


# ------------------------------------------------------------ graph replay
@pytest.mark.parametrize("kind", ["decode", "mixed"])
def test_graph_replay_matches_eager(kind):
    """An attention call captured in a graph and replayed four times, with
    new queries copied in before each replay and eager calls in between:
    every replay equals the eager call on the same queries bit for bit.  The
    stream decode's split rows are merged by their last contributor through
    counters in the workspace; a replay reuses the captured call's epoch, so
    this fails if a finished counter is not put back.  The mixed call also
    forks its prefill tiles onto the library's side stream inside the
    capture."""
    w = workloads.make(3, batch=64) if kind == "decode" else workloads.small(4)
    _announce(f"graph replay, {kind}: B={w.batch} T={w.num_tokens}")
    st = gpu_step.run_workload(w)                     # eager first: side stream, warm-up
    rng = np.random.default_rng(5)
    qs = [torch.from_numpy((rng.standard_normal(tuple(st.q.shape)).astype(np.float32)
                            .view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).cuda()
          for _ in range(4)]
    assert qs[0].dtype == st.q.dtype
    eager = []
    for q in qs:
        st.q.copy_(q)
        st.attend()
        torch.cuda.synchronize()
        eager.append(st.out.clone())
    assert not torch.equal(eager[0], eager[1])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.attend()
    torch.cuda.synchronize()
    for i, q in enumerate(qs):
        st.q.copy_(q)
        st.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, eager[i]), f"replay {i} differs from the eager call"
        st.q.copy_(qs[(i + 1) % 4])                   # an eager call between replays
        st.attend()
        torch.cuda.synchronize()
        assert torch.equal(st.out, eager[(i + 1) % 4]), f"eager call after replay {i} differs"


@pytest.mark.parametrize("mode", ["concurrent", "fused"])
@pytest.mark.parametrize("G,D", [(4, 128), (2, 128), (1, 128), (4, 64), (2, 64), (1, 64)])
def test_mixed_paths_group_and_head_sizes(G, D, mode, monkeypatch):
    """Mixed calls for every supported query-head group and head size: the
    side-stream path (tiles with their LDS request beside the stream decode)
    and the single fused launch (PKV_MIXED=fused).  Decode rows of assorted
    lengths (one of length 1), a 130-row chunk starting mid-block and a short
    multi-row sequence; every row against the oracle."""
    if mode == "fused":
        monkeypatch.setenv("PKV_MIXED", "fused")
    hist = np.array([300, 0, 17, 1000, 37, 90], np.int32)
    ql = np.array([1, 1, 1, 1, 130, 5], np.int32)
    streams = [np.random.default_rng(x) for x in (81 + G, 82 + D, 83, 84)]
    w = workloads._build(4, "mixed shapes", "bf16", 2 * G, 2, D, D ** -0.5, hist, ql, 300, streams)
    _announce(f"mixed {mode} G={G} D={D}: L={w.seq_lens.tolist()} q_len={w.q_len.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"mixed {mode} G={G} D={D}")


# --------------------------------- 8 query heads per kv head; fp32 at head size 128
@pytest.mark.parametrize("kv,G,D", [("bf16", 8, 128), ("bf16", 8, 64), ("fp8", 8, 128),
                                    ("fp8", 8, 64), ("f32", 1, 128), ("f32", 4, 128),
                                    ("f32", 8, 128), ("f32", 8, 64)])
def test_decode_wide_groups_and_fp32_head128(kv, G, D):
    """Decode shapes the library accepts beyond the workloads' own: 8 query
    heads per kv head (bf16 and FP8 caches) and fp32 caches at head size 128,
    whose kernels run one wave per SIMD where their registers need it.
    Lengths at block and step edges and one 5000-token row split over many
    waves; the pool bit for bit and every row against the oracle."""
    L = np.array([1, 16, 17, 33, 300, 1024, 5000, 64, 2], np.int32)
    hkv = 2
    dtype = "f32" if kv == "f32" else "bf16"
    streams = [np.random.default_rng(x) for x in (101 + G, 102 + D, 103, 104 + len(kv))]
    pool = int(1.25 * sum((int(x) + 15) // 16 for x in L)) + 8
    w = workloads._build(3, f"decode {kv} G={G} D={D}", dtype, hkv * G, hkv, D, D ** -0.5, L - 1,
                         np.ones(len(L), np.int32), pool, streams,
                         cache_dtype="fp8" if kv == "fp8" else "",
                         kv_scale=workloads.FP8_SCALE if kv == "fp8" else 1.0)
    _announce(f"decode {kv} G={G} D={D}: L={L.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"]), "pool differs from the oracle's"
    _check_attention(st.out.cpu().numpy(), ref["out"], dtype, f"decode {kv} G={G} D={D}")


@pytest.mark.parametrize("G,D", [(4, 128), (1, 128), (2, 64), (4, 64)])
def test_fp8_decode_step_edges(G, D):
    """FP8 caches decode in steps of four blocks (64 tokens): lengths at and
    around every block and step edge of the first 257 tokens, and one
    4097-token row that the stream split shares among many waves; the pool
    bit for bit and every row against the oracle."""
    L = np.array([1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 127, 128, 129, 191, 192,
                  193, 255, 256, 257, 4097], np.int32)
    hkv = 4
    streams = [np.random.default_rng(x) for x in (201 + G, 202 + D, 203, 204)]
    pool = int(1.25 * sum((int(x) + 15) // 16 for x in L)) + 8
    w = workloads._build(3, f"fp8 step edges G={G} D={D}", "bf16", hkv * G, hkv, D, D ** -0.5,
                         L - 1, np.ones(len(L), np.int32), pool, streams, cache_dtype="fp8",
                         kv_scale=workloads.FP8_SCALE)
    _announce(f"fp8 step edges G={G} D={D}: L={L.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"]), "fp8 pool differs from the oracle's"
    _check_attention(st.out.cpu().numpy(), ref["out"], "bf16", f"fp8 step edges G={G} D={D}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_batch_of_empty_rows_is_zero(kv):
    """A decode call whose every sequence has length 0 returns PKV_OK and
    writes zero rows (the oracle's reading of an empty sequence)."""
    w = workloads.small(3) if kv == "bf16" else workloads.make_fp8(3, small_size=True)
    _announce(f"all-empty decode batch, {kv}")
    st = gpu_step.PagedStep(w)
    st.build_history()
    st.prepare_step()
    st.h_seq_lens = np.zeros_like(st.h_seq_lens)
    st.seq_lens = torch.from_numpy(st.h_seq_lens).cuda()
    st.out.fill_(7.0)
    st.attend()
    torch.cuda.synchronize()
    assert torch.count_nonzero(st.out).item() == 0


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replay_follows_growing_lengths(kv):
    """A decode call captured once and replayed for three more decode steps:
    before each replay every sequence appends one token through the
    library's allocator (new blocks enter the same table tensor), its K/V
    are written (an FP8 cache quantizes them), and the device lengths grow
    by one.  The replay plans its work from the device lengths, so every row
    matches the oracle at the new lengths; a last replay after every length
    shrank to a few tokens (fewer cost units than the captured grid's waves)
    too."""
    from paged_kv_attention_06_amd import _lib as L
    w = workloads.make(3, batch=64)
    if kv == "fp8":  # as workloads.make_fp8 does for the full-size batch
        w.cache_dtype = "fp8"
        w.k_scale = w.v_scale = workloads.FP8_SCALE
        w.pool_fill = workloads.FP8_NAN

    def values(codes, scale):  # what the cache holds, as float64
        if kv == "fp8":
            return po.decode(po.fp8_quantize(codes, scale), "fp8") * scale
        return po.decode(codes, "bf16")

    _announce(f"graph replay with growing lengths: B={w.batch}, {kv} cache")
    st = gpu_step.PagedStep(w)
    st.max_blocks += 1
    st.tables = np.zeros((w.batch, st.max_blocks), np.int32)
    st.build_history()
    st.prepare_step()
    st.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.attend()
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    Ks = [scenario.sequence_kv(w, s)[0] for s in range(w.batch)]
    Vs = [scenario.sequence_kv(w, s)[1] for s in range(w.batch)]
    lens = w.seq_lens.astype(np.int32).copy()
    for step in range(3):
        shape = (w.batch, w.num_kv_heads, w.head_size)
        k_new = workloads._bf16_codes(rng.standard_normal(shape).astype(np.float32))
        v_new = workloads._bf16_codes(rng.standard_normal(shape).astype(np.float32))
        q = workloads._bf16_codes(rng.standard_normal((w.batch, w.num_q_heads, w.head_size))
                                  .astype(np.float32))
        slots = np.concatenate([st.pool.append(st.tables[s], int(lens[s]), 1)[0]
                                for s in range(w.batch)])
        st.block_tables.copy_(torch.from_numpy(st.tables))
        L.paged_kv_write(st.cache, torch.from_numpy(k_new.view(np.int16)).cuda(),
                         torch.from_numpy(v_new.view(np.int16)).cuda(),
                         torch.from_numpy(slots).cuda())
        lens += 1
        st.seq_lens.copy_(torch.from_numpy(lens))
        st.q.copy_(torch.from_numpy(q.view(np.int16)))
        st.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        want = []
        for s in range(w.batch):
            Ks[s] = np.concatenate([Ks[s], k_new[s:s + 1]])
            Vs[s] = np.concatenate([Vs[s], v_new[s:s + 1]])
            want.append(po.attention_rows(po.decode(q[s:s + 1], "bf16"), values(Ks[s], w.k_scale),
                                          values(Vs[s], w.v_scale), [int(lens[s]) - 1], w.scale))
        _check_attention(out, np.concatenate(want), "bf16", f"{kv} replay after growth step {step}")
    # then every length shrinks to 1..5 tokens: fewer cost units than the
    # captured grid has waves, so the kernel narrows its split of the work
    lens = rng.integers(1, 6, size=w.batch).astype(np.int32)
    st.seq_lens.copy_(torch.from_numpy(lens))
    st.out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    want = [po.attention_rows(po.decode(q[s:s + 1], "bf16"), values(Ks[s][:lens[s]], w.k_scale),
                              values(Vs[s][:lens[s]], w.v_scale), [int(lens[s]) - 1], w.scale)
            for s in range(w.batch)]
    _check_attention(st.out.cpu().numpy(), np.concatenate(want), "bf16",
                     f"{kv} replay after shrinking")


@pytest.mark.parametrize("cfg", [5, 4])
def test_debug_validate_mode_accepts_valid_calls(cfg, monkeypatch):
    """PKV_DEBUG_VALIDATE=1 copies slots, copy pairs, tables and lengths to
    the host and checks them before each launch; on valid steps (copies,
    writes, mixed attention) the results are bit for bit those of the normal
    mode."""
    w = workloads.small(cfg)
    _announce(f"debug-validate mode, small {w.name}")
    plain = gpu_step.run_workload(w)
    monkeypatch.setenv("PKV_DEBUG_VALIDATE", "1")
    checked = gpu_step.run_workload(w)
    assert np.array_equal(plain.pool_codes(), checked.pool_codes())
    assert torch.equal(plain.out, checked.out)


@pytest.mark.parametrize("waves", [1, 7, 300])
def test_read_probe_checksums(waves):
    """pkv_read_slices reads every listed (block, kv head) slice once: the
    XOR of the 32-bit words each wave read equals the XOR of the same
    slices of the pool computed on the host, for wave counts that leave
    some waves idle and runs longer than one 64-slice id chunk."""
    from paged_kv_attention_06_amd import _lib as L
    w = workloads.small(3)
    _announce(f"read probe, {waves} waves")
    st = gpu_step.run_workload(w)
    pool = st.pool_codes().view(np.uint32)            # [blocks][Hkv][2 * 16 * D / 2]
    ids = [int(b) * w.num_kv_heads + h for s in range(w.batch) for h in range(w.num_kv_heads)
           for b in st.tables[s][:-(-int(w.seq_lens[s]) // 16)]]
    ids += ids[:5]                                    # a slice read twice is folded twice
    sl = torch.tensor(ids, dtype=torch.int64, device="cuda")
    sink = torch.full((waves,), -1, dtype=torch.int32, device="cuda")
    L.pkv_read_slices(st.cache, sl, waves, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    n = len(ids)
    for wv in range(waves):
        a, b = wv * n // waves, (wv + 1) * n // waves
        x = np.uint32(0)
        for i in ids[a:b]:
            x ^= np.bitwise_xor.reduce(pool[i // w.num_kv_heads, i % w.num_kv_heads].reshape(-1))
        assert got[wv] == x, f"wave {wv} of {waves}"


@pytest.mark.parametrize("case", ["long row", "large batch"])
def test_decode_size_limits(case):
    """Sizes at the ends of the range the workloads span: one 65,536-token row
    (4,096 blocks of table, its 8 (row, kv head) items each split over
    hundreds of waves) beside short ones; and 4,096 sequences of 1..64
    tokens, whose lengths the kernel scans in 16 chunks of 256.  Every row
    against the oracle."""
    rng = np.random.default_rng(131 if case == "long row" else 132)
    if case == "long row":
        L = np.array([65536, 1, 17, 300], np.int32)
    else:
        L = rng.integers(1, 65, size=4096).astype(np.int32)
    streams = [np.random.default_rng(x) for x in rng.integers(0, 2**31, 4)]
    pool = int(1.25 * sum((int(x) + 15) // 16 for x in L)) + 8
    w = workloads._build(3, f"decode {case}", "bf16", 32, 8, 128, 128 ** -0.5, L - 1,
                         np.ones(len(L), np.int32), pool, streams)
    _announce(f"decode {case}: B={w.batch} max L={int(L.max())} pool={pool}")
    st = gpu_step.run_workload(w)
    out = st.out.cpu().numpy()
    want = np.concatenate([scenario.sequence_attention(w, s) for s in range(w.batch)])
    _check_attention(out, want, "bf16", f"decode {case}")


# ------------------------------------------------------ random shapes (hypothesis)
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as hst  # noqa: E402


@hst.composite
def _random_calls(draw):
    kind = draw(hst.sampled_from(["decode", "decode", "mixed", "fp8"]))
    D = draw(hst.sampled_from([64, 128]))
    hkv = draw(hst.integers(1, 4))
    B = draw(hst.integers(1, 8))
    hist = draw(hst.lists(hst.integers(0, 600), min_size=B, max_size=B))
    if kind == "mixed":
        G = draw(hst.sampled_from([1, 2, 4]))
        ql = draw(hst.lists(hst.sampled_from([1, 1, 2, 3, 5, 8, 33, 70, 140]), min_size=B, max_size=B))
        dtype = "bf16"
    else:
        G = draw(hst.sampled_from([1, 2, 4, 8]))
        ql = [1] * B
        dtype = draw(hst.sampled_from(["bf16", "bf16", "f32"])) if kind == "decode" else "bf16"
    seed = draw(hst.integers(0, 2**31 - 1))
    streams = [np.random.default_rng(seed + k) for k in range(4)]
    pool = sum((h + q + 15) // 16 for h, q in zip(hist, ql)) + draw(hst.integers(1, 40))
    return workloads._build(0, f"random {kind}", dtype, hkv * G, hkv, D, D ** -0.5, hist, ql, pool,
                            streams, cache_dtype="fp8" if kind == "fp8" else "",
                            kv_scale=workloads.FP8_SCALE if kind == "fp8" else 1.0)


@settings(max_examples=32, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(_random_calls())
def test_random_shapes_against_the_oracle(w):
    """Random decode, mixed (prefill rows of 2..140 queries beside decode
    rows, or prefill rows alone) and FP8-cache calls over 1-4 kv heads, 1, 2,
    4 or 8 query heads per kv head, head sizes 64 and 128, 1-8 sequences of
    up to 740 tokens in pools with spare blocks: the pool bit for bit and
    every row within the bars (derandomized, so every run draws the same
    cases)."""
    _announce(f"random {w.name}: dtype={w.kv_dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
              f"D={w.head_size} L={w.seq_lens.tolist()} q_len={w.q_len.tolist()}")
    st = gpu_step.run_workload(w)
    ref = scenario.run_step(w)
    assert np.array_equal(st.pool_codes(), ref["pool"]), "pool differs from the oracle's"
    _check_attention(st.out.cpu().numpy(), ref["out"], w.dtype, w.name)
