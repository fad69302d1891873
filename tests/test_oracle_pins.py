"""Pins of the CPU oracle against what the pages print and what mathematics
fixes.  None of these calls the HIP library."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import paged_oracle as po
from oracle import scenario

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def _rand_codes(rng, shape, dtype):
    if dtype == "f32":
        return rng.uniform(-1, 1, size=shape).astype(np.float32).view(np.uint32)
    return workloads._bf16_codes(rng.standard_normal(shape).astype(np.float32))


# ---------------------------------------------------------------- page values
def test_byte_formula_13b_per_token():
    g = GOLD["kv_bytes_per_token_13b"]
    per_block = po.block_bytes(g["block_size"], g["num_kv_heads"], g["head_size"], g["dtype_bytes"])
    per_token = g["layers"] * per_block // g["block_size"]
    assert per_token == 819_200                      # 800 KiB
    assert abs(per_token / 1000 - g["per_token_kb_approx"]) / g["per_token_kb_approx"] < 0.03
    total = per_token * g["tokens"]
    assert abs(total / 1e9 - g["total_gb_approx"]) / g["total_gb_approx"] < 0.06


@pytest.mark.parametrize("cfg,expected", [(1, 32_768), (2, 262_144), (3, 65_536), (4, 65_536), (5, 327_680)])
def test_pool_bytes_match_page_formula(cfg, expected):
    w = workloads.small(cfg)
    pool = po.new_pool(3, w.num_kv_heads, w.head_size, w.dtype, 0)
    assert pool.nbytes // 3 == expected
    assert po.block_bytes(16, w.num_kv_heads, w.head_size, w.dtype_bytes) == expected


def test_block_count_rule():
    g = GOLD["block_count"]
    assert po.blocks_for_tokens(g["new_tokens"]) == g["blocks"]
    alloc = po.CowPool(8)
    table = []
    alloc.append(table, 0, g["new_tokens"])
    assert len(table) == g["blocks"]
    # the 17th token starts a fresh block at offset 0
    t2 = []
    s2, _ = po.CowPool(8).append(t2, 0, 17)
    assert s2[16] % 16 == 0 and s2[16] // 16 == t2[1]


def test_address_translation_example():
    g = GOLD["address_translation"]
    slot = po.slot_of(g["block_table"] + [99], g["token"])
    assert divmod(slot, 16) == (g["physical_block"], g["offset"])
    assert g["token"] // 16 == g["logical_block"]


def test_copy_on_write_walkthrough():
    g = GOLD["copy_on_write"]
    # free list arranged so the prompt gets 0,1,2 and the next free block is 7
    alloc = po.CowPool(10, free_order=[0, 1, 2, 7, 3, 4, 5, 6, 8, 9])
    prompt = []
    alloc.append(prompt, 0, 40)                     # 3 blocks, last one partly filled
    assert prompt == g["prompt_blocks"]
    samples = [prompt] + [alloc.fork(prompt) for _ in range(g["samples"] - 1)]
    assert [alloc.ref[b] for b in prompt] == g["refs_after_fork"]
    slots, cow = alloc.append(samples[0], 40, 1)
    assert cow == tuple(g["copy"])
    assert samples[0] == g["table_after"]
    assert alloc.ref[2] == g["ref_of_old_after"]
    assert slots == [7 * 16 + 40 % 16]
    # the rule: only a shared block is copied; the last holder writes in place
    for s in samples[1:3]:
        _, c = alloc.append(s, 40, 1)
        assert c is not None and c[0] == 2
    assert alloc.ref[2] == 1
    _, c = alloc.append(samples[3], 40, 1)
    assert c is None and samples[3][-1] == 2


def test_chunked_prefill_step_shape():
    g = GOLD["chunked_prefill_step"]
    assert g["budget"] - g["decodes"] == g["chunk"]
    w = workloads.make(4)
    assert w.num_tokens == 2048                     # the 2048-token budget
    assert int(w.q_len.max()) == 1950 and int((w.q_len == 1).sum()) == 98


# ---------------------------------------------------------------- allocator
def test_release_order_and_reuse():
    alloc = po.CowPool(6, free_order=[5, 4, 3, 2, 1, 0])
    t = []
    alloc.append(t, 0, 33)                          # 3 blocks: 5, 4, 3
    assert t == [5, 4, 3]
    alloc.release(t)
    assert list(alloc.free)[:3] == [5, 4, 3]        # returned last-first to the head
    t2 = []
    alloc.append(t2, 0, 1)
    assert t2 == [5]


def test_pool_exhaustion_raises():
    alloc = po.CowPool(2)
    t = []
    with pytest.raises(MemoryError):
        alloc.append(t, 0, 33)


def test_slot_mapping_agrees_with_allocator():
    w = workloads.small(4)
    st = scenario.build_tables(w, with_pool=False)
    bt = scenario.table_matrix(st["tables"])
    assert np.array_equal(po.slot_mapping(bt, w.query_start_loc, w.seq_lens), st["slots"])


# ---------------------------------------------------------------- data movement
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layout_offsets(dtype):
    """Every element lands at the offset the documented layout gives, computed
    here one element at a time from byte arithmetic."""
    rng = np.random.default_rng(1)
    Hkv, D, nb = 2, 64, 5
    es = po.dtype_bytes(dtype)
    E = 16 // es
    pool = po.new_pool(nb, Hkv, D, dtype, 0)
    k = rng.integers(1, 2 ** (8 * es) - 1, size=(1, Hkv, D)).astype(po.code_dtype(dtype))
    v = rng.integers(1, 2 ** (8 * es) - 1, size=(1, Hkv, D)).astype(po.code_dtype(dtype))
    blk, off = 3, 11
    po.kv_write(pool, dtype, k, v, [blk * 16 + off])
    raw = pool.view(np.uint8).reshape(-1)
    blk_bytes = 2 * 16 * Hkv * D * es
    for h in range(Hkv):
        for d in range(D):
            kb = blk * blk_bytes + h * 2 * 16 * D * es + ((d // E) * 16 + off) * 16 + (d % E) * es
            vb = (blk * blk_bytes + h * 2 * 16 * D * es + 16 * D * es
                  + ((off // E) * D + d) * 16 + (off % E) * es)
            assert raw[kb:kb + es].view(po.code_dtype(dtype))[0] == k[0, h, d]
            assert raw[vb:vb + es].view(po.code_dtype(dtype))[0] == v[0, h, d]
    assert np.count_nonzero(pool) == 2 * Hkv * D


def test_kv_write_skip_and_untouched():
    rng = np.random.default_rng(2)
    pool = po.new_pool(4, 2, 64, "bf16", workloads.BF16_NAN)
    before = pool.copy()
    k = _rand_codes(rng, (3, 2, 64), "bf16")
    v = _rand_codes(rng, (3, 2, 64), "bf16")
    po.kv_write(pool, "bf16", k, v, [5, -1, 63])
    K, V = po.gather_kv(pool, "bf16", [0, 1, 2, 3], 64, 64)
    assert np.array_equal(K[5], k[0]) and np.array_equal(V[63], v[2])
    changed = np.argwhere((pool != before).any(axis=(1, 2, 3))).ravel().tolist()
    assert changed == [0, 3]
    untouched_rows = [j for j in range(64) if j not in (5, 63)]
    assert np.all(K[untouched_rows] == workloads.BF16_NAN)


def test_block_copy_reads_pre_call_contents():
    rng = np.random.default_rng(3)
    pool = _rand_codes(rng, (6, 2, 2, 16 * 64), "bf16")
    snap = pool.copy()
    po.block_copy(pool, [(1, 4), (1, 5), (2, 0)])
    assert np.array_equal(pool[4], snap[1]) and np.array_equal(pool[5], snap[1])
    assert np.array_equal(pool[0], snap[2])
    assert np.array_equal(pool[[1, 2, 3]], snap[[1, 2, 3]])


# ---------------------------------------------------------------- attention
def _dense_attention_einsum(q, K, V, positions, scale, group):
    """A second, differently written textbook attention on dense arrays."""
    Kx = np.repeat(K, group, axis=1)                # [L][Hq][D]
    Vx = np.repeat(V, group, axis=1)
    s = np.einsum("nhd,lhd->nhl", q, Kx) * scale
    L = K.shape[0]
    mask = np.arange(L)[None, None, :] > np.asarray(positions)[:, None, None]
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=2, keepdims=True)
    return np.einsum("nhl,lhd->nhd", p, Vx)


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_paged_equals_contiguous(cfg):
    w = workloads.small(cfg)
    st = scenario.run_step(w)
    qsl = w.query_start_loc
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.batch):
        K, V = scenario.sequence_kv(w, s)
        L = int(w.seq_lens[s])
        q_len = int(w.q_len[s])
        q = po.decode(w.q[qsl[s]:qsl[s + 1]], w.dtype)
        ref = _dense_attention_einsum(q, po.decode(K, w.dtype), po.decode(V, w.dtype),
                                      [L - q_len + i for i in range(q_len)], w.scale, G)
        np.testing.assert_allclose(st["out"][qsl[s]:qsl[s + 1]], ref, rtol=0, atol=1e-13)


def test_torch_sdpa_matches_mixed_step():
    """The library routine: PyTorch's scaled_dot_product_attention in float64
    with an explicit causal-with-offset mask and GQA-expanded heads."""
    w = workloads.small(4)
    st = scenario.run_step(w)
    qsl = w.query_start_loc
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.batch):
        K, V = scenario.sequence_kv(w, s)
        L, q_len = int(w.seq_lens[s]), int(w.q_len[s])
        q = torch.from_numpy(po.decode(w.q[qsl[s]:qsl[s + 1]], w.dtype)).permute(1, 0, 2)
        k = torch.from_numpy(po.decode(K, w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        v = torch.from_numpy(po.decode(V, w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        pos = torch.arange(L - q_len, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale)
        np.testing.assert_allclose(st["out"][qsl[s]:qsl[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_block_permutation_invariance():
    """Moving every block to another physical id and rewriting the tables
    leaves the output bit-identical."""
    w = workloads.small(3)
    st = scenario.run_step(w)
    rng = np.random.default_rng(7)
    perm = rng.permutation(w.num_blocks)
    pool2 = np.empty_like(st["pool"])
    pool2[perm] = st["pool"]
    bt2 = perm[st["block_tables"]].astype(np.int32)
    out2 = po.paged_attention(pool2, w.dtype, w.q, bt2, w.seq_lens, w.query_start_loc, w.scale)
    assert np.array_equal(out2, st["out"])


def test_brute_force_tiny_decode():
    """The tiny fp32 decode workload recomputed with scalar Python loops and math.exp."""
    w = workloads.make(1)
    st = scenario.run_step(w)
    qsl = w.query_start_loc
    for s in range(w.batch):
        K, V = scenario.sequence_kv(w, s)
        Kf, Vf = po.decode(K, "f32"), po.decode(V, "f32")
        L = int(w.seq_lens[s])
        qrow = po.decode(w.q[qsl[s]], "f32")
        for h in range(w.num_q_heads):
            xs = [w.scale * sum(qrow[h, d] * Kf[j, h, d] for d in range(w.head_size)) for j in range(L)]
            mx = max(xs)
            ws = [math.exp(x - mx) for x in xs]
            tot = sum(ws)
            o = [sum(ws[j] * Vf[j, h, d] for j in range(L)) / tot for d in range(w.head_size)]
            np.testing.assert_allclose(st["out"][qsl[s], h], o, rtol=0, atol=1e-13)


def test_closed_form_single_key():
    rng = np.random.default_rng(4)
    pool = po.new_pool(2, 1, 64, "bf16", workloads.BF16_NAN)
    k = _rand_codes(rng, (1, 1, 64), "bf16")
    v = _rand_codes(rng, (1, 1, 64), "bf16")
    po.kv_write(pool, "bf16", k, v, [16])
    q = _rand_codes(rng, (1, 2, 64), "bf16")
    out = po.paged_attention(pool, "bf16", q, np.array([[1]]), [1], [0, 1], 0.125)
    assert np.array_equal(out[0, 0], po.decode(v[0, 0], "bf16"))
    assert np.array_equal(out[0, 1], po.decode(v[0, 0], "bf16"))


def test_closed_form_zero_query_is_mean():
    rng = np.random.default_rng(5)
    L = 37
    pool = po.new_pool(4, 2, 64, "f32", workloads.F32_NAN)
    k = _rand_codes(rng, (L, 2, 64), "f32")
    v = _rand_codes(rng, (L, 2, 64), "f32")
    po.kv_write(pool, "f32", k, v, [16 * [2, 0, 3][j // 16] + j % 16 for j in range(L)])
    q = np.zeros((1, 2, 64), np.uint32)
    out = po.paged_attention(pool, "f32", q, np.array([[2, 0, 3]]), [L], [0, 1], 1.0)
    np.testing.assert_allclose(out[0], po.decode(v, "f32").mean(axis=0), rtol=0, atol=1e-15)


def test_closed_form_dominant_key():
    rng = np.random.default_rng(6)
    L = 20
    pool = po.new_pool(2, 1, 64, "f32", workloads.F32_NAN)
    k = np.zeros((L, 1, 64), np.float32)
    k[13, 0, :] = 1.0
    v = _rand_codes(rng, (L, 1, 64), "f32")
    po.kv_write(pool, "f32", k.view(np.uint32), v, list(range(L)))
    q = np.full((1, 1, 64), 1.0, np.float32).view(np.uint32)
    out = po.paged_attention(pool, "f32", q, np.array([[0, 1]]), [L], [0, 1], 10.0)
    # weight of key 13 is 1 / (1 + 19 e^-640) == 1 in float64
    assert np.array_equal(out[0, 0], po.decode(v[13, 0], "f32"))


def test_causal_rows_see_only_their_prefix():
    """Changing a key after position p must not change query rows at <= p."""
    w = workloads.small(4)
    st = scenario.run_step(w)
    s = w.batch - 1                                 # the prefill chunk
    bt = st["block_tables"]
    L = int(w.seq_lens[s])
    pool2 = st["pool"].copy()
    blk = bt[s][(L - 1) // 16]
    pool2[blk, :, :, :] = workloads.BF16_NAN       # poison the last block
    out2 = po.paged_attention(pool2, w.dtype, w.q, bt, w.seq_lens, w.query_start_loc, w.scale)
    first_poisoned = ((L - 1) // 16) * 16
    q_len = int(w.q_len[s])
    r0 = int(w.query_start_loc[s])
    for i in range(q_len):
        pos = L - q_len + i
        same = np.array_equal(out2[r0 + i], st["out"][r0 + i])
        assert same == (pos < first_poisoned)


def test_empty_sequence_gives_zeros():
    pool = po.new_pool(2, 1, 64, "bf16", workloads.BF16_NAN)
    q = np.zeros((1, 1, 64), np.uint16)
    out = po.paged_attention(pool, "bf16", q, np.array([[0]]), [0], [0, 1], 0.125)
    assert np.all(out == 0)


def test_13b_prefix_forks_all_copy_on_write():
    w = workloads.small(5)
    st = scenario.build_tables(w, with_pool=False)
    n_fork = int((w.fork_of >= 0).sum())
    assert len(st["cow_pairs"]) == n_fork
    shared_last = st["prompt_tables"][0][-1]
    assert all(int(p[0]) == shared_last for p in st["cow_pairs"])
    assert st["alloc"].ref[shared_last] == 1        # only the owner holds it now


# ------------------------------------------------------------- FP8 KV cache
def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    """The library routine: torch's float8_e4m3fn reads all 256 codes the
    same way (NaN at 0x7F and 0xFF only)."""
    mine = po.e4m3_table()
    ref = _torch_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.isnan(mine).sum() == 2 and np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_format_values():
    """Values the E4M3 definition fixes: bias 7, 3 mantissa bits, subnormals
    at exponent field 0, largest finite 448."""
    assert po.e4m3_value(0x38) == 1.0            # exponent field 7, mantissa 0
    assert po.e4m3_value(0x7E) == 448.0          # 1.75 * 2^8
    assert po.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert po.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert po.e4m3_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert po.e4m3_value(0xC0) == -2.0
    assert po.e4m3_value(0x80) == 0.0 and math.copysign(1, po.e4m3_value(0x80)) < 0
    values = po.e4m3_table()[:0x7F]
    assert np.all(np.diff(values) > 0)           # codes 0..126 increase strictly


def test_e4m3_encode_matches_torch_in_range():
    """Within |x| <= 464 (where no saturation applies) the encoder rounds to
    nearest with ties to the even code, as torch's cast does; the tests use
    random values, every representable value, and every midpoint (a tie)."""
    rng = np.random.default_rng(3)
    vals = po.e4m3_table()[:0x7F]
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-464, 464, 20000),
                        rng.uniform(-0.02, 0.02, 20000), vals, -vals, mids, -mids,
                        [464.0, -464.0, 0.0, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(po.e4m3_encode(x), ref)


def test_e4m3_encode_saturates_and_keeps_nan():
    big = np.array([465.0, 480.0, 1e6, 3.0e38, np.inf], np.float32)
    assert np.all(po.e4m3_encode(big) == 0x7E)
    assert np.all(po.e4m3_encode(-big) == 0xFE)
    assert po.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(po.e4m3_encode(po.e4m3_table()[codes]), codes)  # round trip


def test_fp8_quantize_is_float32_product_then_cast():
    """x * (1 / scale), both in float32, then the cast: checked against torch
    doing the same float32 arithmetic, for bf16 inputs in range."""
    rng = np.random.default_rng(4)
    codes = workloads._bf16_codes(rng.standard_normal(50000).astype(np.float32) * 2)
    for scale in (workloads.FP8_SCALE, 0.37, 3.0):
        x = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).float()
        y = x * (torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32))
        y = torch.clamp(y, -448, 448)
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(po.fp8_quantize(codes, scale), ref)


def test_fp8_pool_bytes_halve():
    """Per-block byte formula with one byte per element."""
    assert po.block_bytes(16, 8, 128, po.dtype_bytes("fp8")) == 32768
    assert po.new_pool(3, 8, 128, "fp8", 0x7F).nbytes == 3 * 32768


def test_fp8_paged_equals_contiguous_on_dequantized_values():
    """The FP8 step's output equals textbook attention (separately written
    einsum) on the quantized K/V times their scales."""
    w = workloads.make_fp8(3, small_size=True)
    st = scenario.run_step(w)
    qsl = w.query_start_loc
    G = w.num_q_heads // w.num_kv_heads
    table = _torch_e4m3(np.arange(256))
    for s in range(w.batch):
        K, V = scenario.sequence_kv(w, s)
        Kq = torch.from_numpy(K.astype(np.int16)).view(torch.bfloat16).float() * (1 / np.float32(w.k_scale))
        Vq = torch.from_numpy(V.astype(np.int16)).view(torch.bfloat16).float() * (1 / np.float32(w.v_scale))
        Kd = table[Kq.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()] * w.k_scale
        Vd = table[Vq.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()] * w.v_scale
        L, q_len = int(w.seq_lens[s]), int(w.q_len[s])
        q = po.decode(w.q[qsl[s]:qsl[s + 1]], "bf16")
        ref = _dense_attention_einsum(q, Kd, Vd, [L - q_len + i for i in range(q_len)], w.scale, G)
        np.testing.assert_allclose(st["out"][qsl[s]:qsl[s + 1]], ref, rtol=0, atol=1e-13)


def test_fp8_kv_write_layout_and_skip():
    """An FP8 write stores each quantized element at the layout's byte and
    leaves every other byte (and skipped tokens) untouched."""
    rng = np.random.default_rng(5)
    pool = po.new_pool(6, 2, 64, "fp8", 0x7F)
    k = workloads._bf16_codes(rng.standard_normal((3, 2, 64)).astype(np.float32))
    v = workloads._bf16_codes(rng.standard_normal((3, 2, 64)).astype(np.float32))
    slots = [5 * 16 + 3, -1, 2 * 16 + 15]
    po.kv_write(pool, "fp8", k, v, slots, k_scale=0.25, v_scale=0.5)
    kq, vq = po.fp8_quantize(k, 0.25), po.fp8_quantize(v, 0.5)
    for t, slot in ((0, slots[0]), (2, slots[2])):
        blk, off = divmod(slot, 16)
        for hh in range(2):
            for d in range(64):
                # K granule: 16 consecutive d of one token; V granule: 16 tokens of one d
                assert pool[blk, hh, 0, ((d // 16) * 16 + off) * 16 + d % 16] == kq[t, hh, d]
                assert pool[blk, hh, 1, d * 16 + off] == vq[t, hh, d]
    touched = 2 * 2 * 2 * 64
    assert int((pool != 0x7F).sum()) <= touched


def test_block_swap_round_trip_and_untouched():
    """Swap out to host blocks, swap back in to other device blocks: the
    blocks come back bit for bit; nothing else changes."""
    rng = np.random.default_rng(8)
    dev = rng.integers(0, 1 << 16, size=(10, 2, 2, 16 * 64), dtype=np.uint16)
    host = np.zeros((6, 2, 2, 16 * 64), np.uint16)
    before = dev.copy()
    po.block_swap(dev, host, [(3, 0), (7, 5), (1, 2)], to_host=True)
    assert np.array_equal(host[[0, 5, 2]], before[[3, 7, 1]])
    assert not host[[1, 3, 4]].any() and np.array_equal(dev, before)
    po.block_swap(dev, host, [(0, 8), (5, 9), (2, 0)], to_host=False)
    assert np.array_equal(dev[[8, 9, 0]], before[[3, 7, 1]])
    untouched = [b for b in range(10) if b not in (8, 9, 0)]
    assert np.array_equal(dev[untouched], before[untouched])


# ------------------------------------------------------------- prefix caching
def test_fnv1a64_published_vectors():
    assert po.fnv1a64(b"") == 0xCBF29CE484222325
    assert po.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert po.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_hashes_chain_the_prefix():
    """A block's hash stands for the whole prefix up to it: equal prefixes
    give equal hashes; one changed token changes its block's hash and every
    later one; a partly filled last block gets none."""
    rng = np.random.default_rng(9)
    a = rng.integers(0, 32000, size=16 * 5 + 7).tolist()
    b = list(a)
    b[16 * 2 + 3] += 1
    ha, hb = po.prefix_hashes(a), po.prefix_hashes(b)
    assert len(ha) == 5
    assert ha[:2] == hb[:2]
    assert all(x != y for x, y in zip(ha[2:], hb[2:]))
    assert po.prefix_hashes(a[:40]) == ha[:2]


def test_prefix_cache_walkthrough():
    """Inside vLLM "Prefix caching": the first request with a long prefix
    finds nothing and registers its full blocks; after it finishes they sit
    in the free queue with their hashes; a second request with the same
    prefix reuses all of them (taken off the queue); had the first still been
    alive, the counts would be 2."""
    pool = po.PrefixCachePool(64)
    prefix = list(range(1000, 1000 + 16 * 4))              # n = 4 full blocks
    r1 = prefix + [7, 8, 9]
    assert pool.match_prefix(r1) == []
    t1 = []
    pool.append(t1, 0, len(r1))
    pool.cache_blocks(r1, t1, len(r1) // 16)
    shared = t1[:4]
    pool.release(t1)
    assert all(pool.ref[b] == 0 for b in shared)
    assert pool.free[-4:] == shared[::-1]                  # hashed blocks at the tail, the first block last
    r2 = prefix + [5, 5]
    hit = pool.match_prefix(r2)
    assert hit == shared and all(pool.ref[b] == 1 for b in hit)
    assert not any(b in pool.free for b in hit)
    hit3 = pool.match_prefix(prefix)                       # a third, concurrent request
    assert hit3 == shared and all(pool.ref[b] == 2 for b in hit3)


def test_prefix_cache_eviction_and_release_order():
    """A block loses its hash only when it is taken from the head for a new
    use; released unhashed blocks go to the head, hashed ones to the tail."""
    pool = po.PrefixCachePool(6)
    toks = list(range(16 * 2))
    t = []
    pool.append(t, 0, 32)
    pool.cache_blocks(toks, t, 2)
    t_other = []
    pool.append(t_other, 0, 16)                            # unhashed
    pool.release(t)
    pool.release(t_other)
    assert pool.free[0] == 2 and pool.free[-2:] == [1, 0]
    grab = []
    pool.append(grab, 0, 16 * 4)                           # takes 2, 3, 4, 5
    assert pool.match_prefix(toks) == [0, 1]               # still cached
    pool.release([0, 1])
    pool.release(grab)
    pool2 = po.PrefixCachePool(3)
    t2 = []
    pool2.append(t2, 0, 32)
    pool2.cache_blocks(toks, t2, 2)
    pool2.release(t2)                                      # free: 2, 1, 0
    x = []
    pool2.append(x, 0, 32)                                 # takes 2 then 1: 1 is evicted
    assert pool2.key[1] is None and pool2.match_prefix(toks) == [0]


# ------------------------------------------------------------ code decoding
def test_decode_bf16_every_code_matches_torch():
    """All 65,536 bf16 codes decode to the value torch's own bfloat16 type
    gives them (NaN codes to NaN, the sign of zero kept): the stored bit
    patterns are read as their exact values (Continuous batching +
    PagedAttention 3.6 computes on the cached K/V as stored)."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = po.decode(codes, "bf16")
    want = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert got.dtype == np.float64 and got.shape == codes.shape
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_format_values():
    """Values the bf16 and binary32 formats fix, written out by hand."""
    bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x3E80: 0.25, 0x4049: 3.140625,
            0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
            0x7F80: math.inf, 0xFF80: -math.inf}
    for c, v in bf16.items():
        assert po.decode(np.array([c], np.uint16), "bf16")[0] == v, hex(c)
    assert math.copysign(1.0, po.decode(np.array([0x8000], np.uint16), "bf16")[0]) == -1.0
    f32 = {0x3F800000: 1.0, 0xBF000000: -0.5, 0x00000001: 2.0 ** -149,
           0x00800000: 2.0 ** -126, 0x7F7FFFFF: (2 - 2 ** -23) * 2.0 ** 127,
           0x3DCCCCCD: 0.100000001490116119384765625}
    for c, v in f32.items():
        assert po.decode(np.array([c], np.uint32), "f32")[0] == v, hex(c)
    assert math.isnan(po.decode(np.array([0x7FC00000], np.uint32), "f32")[0])


def test_decode_f32_random_codes_match_torch():
    """Random binary32 codes (normal, subnormal, NaN and infinite ones among
    them), decoded in a strided 3-D view: same shape, and torch's float32
    reading of every code."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 1 << 32, size=(8, 64, 66), dtype=np.uint64).astype(np.uint32)
    codes[0, 0, :6] = [0x7F800000, 0xFF800000, 0x7FC00001, 0x00000001, 0x807FFFFF, 0x80000000]
    view = codes[:, ::2, 1:65]
    got = po.decode(view, "f32")
    assert got.shape == view.shape and got.dtype == np.float64
    want = torch.from_numpy(np.ascontiguousarray(view).view(np.int32)).view(torch.float32).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    # bf16 decoding of a strided view keeps the shape and each element's value
    b = workloads._bf16_codes(rng.standard_normal((4, 6, 10)).astype(np.float32))[:, 1::2, ::3]
    gb = po.decode(b, "bf16")
    assert gb.shape == b.shape
    assert np.array_equal(gb, torch.from_numpy(np.ascontiguousarray(b).view(np.int16))
                          .view(torch.bfloat16).double().numpy())


# ------------------------------------------- logical-order reference rows
def _check_sequence_attention_rows(w):
    out = scenario.run_step(w)["out"]
    qsl = w.query_start_loc
    for s in range(w.batch):
        got = scenario.sequence_attention(w, s)
        assert got.shape == (int(w.q_len[s]), w.num_q_heads, w.head_size)
        assert np.array_equal(got, out[qsl[s]:qsl[s + 1]]), f"{w.name}: sequence {s}"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_sequence_attention_equals_paged_step(cfg):
    """The reference rows that full-size parity uses, computed from each
    sequence's K/V in logical order straight from the draws, equal the
    paged oracle step (allocator, copies, scatter, gather through the block
    table) row for row and bit for bit."""
    _check_sequence_attention_rows(workloads.small(cfg))


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_sequence_attention_equals_paged_step_fp8(cfg):
    """The same on FP8 caches: quantized values, scales applied alike."""
    _check_sequence_attention_rows(workloads.make_fp8(cfg, small_size=True))


def test_sequence_attention_row_subsets_of_the_chunk():
    """Row subsets of the prefill chunk (first rows, rows at block edges, the
    last row, unsorted and repeated picks) equal those rows of the full step."""
    w = workloads.small(4)
    out = scenario.run_step(w)["out"]
    s = int(np.argmax(w.q_len))
    ql = int(w.q_len[s])
    r0 = int(w.query_start_loc[s])
    for rows in ([0], [ql - 1], [0, 1, 15, 16, 17, ql // 2, ql - 1], [ql - 1, 3, 3, 0]):
        got = scenario.sequence_attention(w, s, rows)
        assert np.array_equal(got, out[r0 + np.asarray(rows)]), rows
