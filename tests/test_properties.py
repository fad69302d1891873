"""Property tests over random small shapes (hypothesis, derandomized).  CPU
only: the oracle against a separately written dense computation and under
block permutation; write-then-gather round trips; and the library's host
allocator (ctypes) against the oracle's on random operation sequences."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads
from oracle import paged_oracle as po
from oracle import scenario

SETTINGS = dict(max_examples=30, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


@st.composite
def small_workloads(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    hkv = draw(st.integers(1, 3))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    D = draw(st.sampled_from([64, 128]))
    B = draw(st.integers(1, 5))
    hist = draw(st.lists(st.integers(0, 70), min_size=B, max_size=B))
    ql = draw(st.lists(st.integers(1, 20), min_size=B, max_size=B))
    seed = draw(st.integers(0, 2**31 - 1))
    streams = [np.random.default_rng(seed + k) for k in range(4)]
    blocks = sum((h + q + 15) // 16 for h, q in zip(hist, ql))
    pool = blocks + draw(st.integers(0, 10))
    return workloads._build(0, "property", dtype, hkv * G, hkv, D, D ** -0.5, hist, ql, pool,
                            streams)


def _dense(q, K, V, positions, scale, group):
    """Textbook attention written with explicit loops over heads and rows."""
    n, Hq, Dd = q.shape
    out = np.empty((n, Hq, Dd))
    for i in range(n):
        for h in range(Hq):
            k = K[: positions[i] + 1, h // group]
            v = V[: positions[i] + 1, h // group]
            x = np.array([scale * float(np.dot(q[i, h], kk)) for kk in k])
            e = np.exp(x - x.max())
            out[i, h] = (e[:, None] * v).sum(axis=0) / e.sum()
    return out


@settings(**SETTINGS)
@given(small_workloads())
def test_paged_step_equals_dense_attention(w):
    """Paging, copy-on-write and the scatter change where K/V live, never the
    result: the paged oracle step equals dense textbook attention over each
    sequence's own tokens (juhe.plus 3.6; Inside vLLM "Forward pass")."""
    out = scenario.run_step(w)["out"]
    qsl, G = w.query_start_loc, w.num_q_heads // w.num_kv_heads
    for s in range(w.batch):
        K, V = scenario.sequence_kv(w, s)
        L, q_len = int(w.seq_lens[s]), int(w.q_len[s])
        ref = _dense(po.decode(w.q[qsl[s]:qsl[s + 1]], w.dtype), po.decode(K, w.dtype),
                     po.decode(V, w.dtype), [L - q_len + i for i in range(q_len)], w.scale, G)
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref, rtol=0, atol=1e-12)


@settings(**SETTINGS)
@given(small_workloads(), st.integers(0, 2**31 - 1))
def test_block_permutation_changes_nothing(w, seed):
    st_ = scenario.run_step(w)
    perm = np.random.default_rng(seed).permutation(w.num_blocks)
    pool2 = np.empty_like(st_["pool"])
    pool2[perm] = st_["pool"]
    out2 = po.paged_attention(pool2, w.dtype, w.q, perm[st_["block_tables"]], w.seq_lens,
                              w.query_start_loc, w.scale)
    assert np.array_equal(out2, st_["out"])


@settings(**SETTINGS)
@given(st.sampled_from(["f32", "bf16", "fp8"]), st.integers(1, 3), st.sampled_from([64, 128]),
       st.integers(1, 40), st.integers(0, 2**31 - 1))
def test_write_then_gather_round_trip(dtype, hkv, D, n, seed):
    """Rows scattered to distinct random slots read back through any table
    that lists their blocks in order (vLLM 源码精读 5.1)."""
    rng = np.random.default_rng(seed)
    nb = -(-n // 16) + 3
    table = rng.permutation(nb)[: -(-n // 16)]
    slots = [int(table[j // 16]) * 16 + j % 16 for j in range(n)]
    in_dtype = "bf16" if dtype == "fp8" else dtype
    vals = workloads._values(rng, (2, n, hkv, D), in_dtype)
    pool = po.new_pool(nb, hkv, D, dtype, 0)
    po.kv_write(pool, dtype, vals[0], vals[1], slots, k_scale=0.5, v_scale=0.25)
    K, V = po.gather_kv(pool, dtype, table, n, D)
    if dtype == "fp8":
        assert np.array_equal(K, po.fp8_quantize(vals[0], 0.5))
        assert np.array_equal(V, po.fp8_quantize(vals[1], 0.25))
    else:
        assert np.array_equal(K, vals[0]) and np.array_equal(V, vals[1])


P = pytest.importorskip("paged_kv_attention_06_amd")


@settings(**SETTINGS)
@given(st.lists(st.tuples(st.integers(0, 3), st.integers(0, 10**6)), min_size=1, max_size=60),
       st.integers(0, 2**31 - 1))
def test_library_allocator_takes_the_oracles_decisions(ops, seed):
    """Random new requests, forks (parallel sampling), appends (decode steps
    and chunks, with copy-on-write of shared partial blocks) and releases:
    the host library's pkv_pool and the oracle's CowPool hand out the same
    blocks and slots, emit the same copy pairs and keep the same reference
    counts (vLLM 技术内幕 2.2; juhe.plus 3.8)."""
    NB, MAXB = 60, 12
    order = np.random.default_rng(seed).permutation(NB).astype(np.int32)
    lib, ora = P.Pool(NB, order), po.CowPool(NB, order)
    live = []   # (library table, oracle table, length)
    for op, x in ops:
        if op == 0 or not live:
            n = 1 + x % 100
            t_lib = np.zeros(MAXB, np.int32)
            t_ora = []
            try:
                slots_o, _ = ora.append(t_ora, 0, n)
            except MemoryError:
                with pytest.raises(P.PkvError):
                    lib.append(t_lib, 0, n)
                continue
            slots_l, cow = lib.append(t_lib, 0, n)
            assert cow is None and slots_l.tolist() == slots_o
            live.append((t_lib, t_ora, n))
        elif op == 1:
            t_lib, t_ora, n = live[x % len(live)]
            nb = -(-n // 16)
            f_lib = np.zeros(MAXB, np.int32)
            f_lib[:nb] = lib.fork(t_lib, nb)[:nb]
            live.append((f_lib, ora.fork(t_ora), n))
        elif op == 2:
            i = x % len(live)
            t_lib, t_ora, n = live[i]
            k = 1 + (x >> 8) % 20
            if -(-(n + k) // 16) > MAXB:
                continue
            try:
                slots_o, cow_o = ora.append(t_ora, n, k)
            except MemoryError:
                with pytest.raises(P.PkvError):
                    lib.append(t_lib, n, k)
                continue
            slots_l, cow_l = lib.append(t_lib, n, k)
            assert slots_l.tolist() == slots_o and cow_l == cow_o
            live[i] = (t_lib, t_ora, n + k)
        else:
            t_lib, t_ora, n = live.pop(x % len(live))
            lib.release(t_lib, -(-n // 16))
            ora.release(t_ora)
        for t_lib, t_ora, n in live:
            assert t_lib[: -(-n // 16)].tolist() == t_ora
    assert lib.num_free() == ora.num_free()
    assert [lib.refcnt(b) for b in range(NB)] == ora.ref
