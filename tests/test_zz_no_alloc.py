"""The no-allocation decode entry point (paged_attention_decode_noalloc)
against paged_attention_decode with a caller workspace, through the C ABI:
two calls in a row on the library's scratch array, the second with a
smaller batch, each equal bit for bit to the workspace call and within the
bars of the oracle (bf16 and FP8 caches); and a batch too large for the
array is refused before any launch."""
import sys

import numpy as np
import pytest

import workloads
from oracle import scenario

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_attention_06_amd import _lib as L  # noqa: E402
from paged_kv_attention_06_amd import step as gpu_step  # noqa: E402


def _announce(what):
    print(f"\n[gpu case] {what}", file=sys.stderr, flush=True)


def _noalloc(st, w, out):
    L.paged_attention_decode_noalloc(st.cache, out, st.q, st.block_tables, st.seq_lens,
                                     st.h_seq_lens, w.scale)


def _against_oracle(out, w, what):
    ref = np.concatenate([scenario.sequence_attention(w, s) for s in range(w.batch)])
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert max_abs <= 5e-3 and rel <= 1e-3, f"{what}: max|d| {max_abs:.3e} rel {rel:.3e}"


def _fp8(w):
    """The same batch with an FP8 E4M3 cache (as workloads.make_fp8 builds it)."""
    w.name = w.name + " (fp8 KV)"
    w.cache_dtype = "fp8"
    w.k_scale = w.v_scale = workloads.FP8_SCALE
    w.pool_fill = workloads.FP8_NAN
    return w


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_decode_equals_workspace_decode_twice(kv):
    first = workloads.make(3)                  # the 8B GQA batch of 256
    second = workloads.make(3, batch=40)       # a smaller batch on the same scratch
    if kv == "fp8":
        first, second = _fp8(first), _fp8(second)
    for w in (first, second):
        _announce(f"no-allocation decode ({kv} cache): B={w.batch} sum L={int(w.seq_lens.sum())}")
        st = gpu_step.run_workload(w)          # workspace call: st.out
        out = torch.full_like(st.out, float("nan"))
        _noalloc(st, w, out)
        torch.cuda.synchronize()
        assert torch.equal(out, st.out), f"B={w.batch}: differs from the workspace call"
        _against_oracle(out, w, f"no-allocation B={w.batch}")
        del st


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    """600,000 sequences x 8 kv heads need 38.4 MB of counters alone, more
    than the 32 MiB array: PKV_ERR_WORKSPACE before anything is launched.
    (The device buffers are sized for the batch and its device lengths are
    0, so even a launch would stay in bounds.)"""
    w = workloads.small(3)
    st = gpu_step.run_workload(w)
    n = 600_000
    assert n * w.num_kv_heads * 8 > (32 << 20)
    h_lens = np.full(n, 300, np.int32)
    d_lens = torch.zeros(n, dtype=torch.int32, device="cuda")
    tables = torch.zeros((n, 19), dtype=torch.int32, device="cuda")
    q = torch.zeros((n, w.num_q_heads, w.head_size), dtype=torch.int16, device="cuda")
    out = torch.empty((n, w.num_q_heads, w.head_size), dtype=torch.float32, device="cuda")
    _announce(f"no-allocation decode refuses B={n}")
    with pytest.raises(L.PkvError) as e:
        L.paged_attention_decode_noalloc(st.cache, out, q, tables, d_lens, h_lens, w.scale)
    assert e.value.status == 4 and "scratch" in str(e.value)
