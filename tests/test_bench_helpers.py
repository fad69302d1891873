"""Host-side helpers of bench.py that decide what its JSON line reports:
the digest that keys the measured traffic figures to the kernel code they
were taken on, and the lookup that returns a figure only while that code is
unchanged."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

SAMPLE = """// header comment
#include <hip/hip_runtime.h>
/* a block
   comment */
__global__ void k(float* x) {  // trailing comment
  x[threadIdx.x] = 2.0f * x[threadIdx.x];
}
"""


def _digest_of(tmp_path, text, name="k.hip"):
    p = tmp_path / name
    p.write_text(text, encoding="utf-8")
    return bench.kernel_code_digest(str(p))


def test_digest_ignores_comments_and_blank_space(tmp_path):
    base = _digest_of(tmp_path, SAMPLE)
    edited = SAMPLE.replace("// trailing comment", "// another remark") \
                   .replace("/* a block\n   comment */", "") \
                   .replace("  x[threadIdx.x] =", "\n\n      x[threadIdx.x]   =")
    assert _digest_of(tmp_path, edited, "k2.hip") == base


def test_digest_follows_any_code_change(tmp_path):
    base = _digest_of(tmp_path, SAMPLE)
    for old, new in [("2.0f", "3.0f"), ("float* x", "double* x"), ("#include", "#include <cmath>\n#include")]:
        assert _digest_of(tmp_path, SAMPLE.replace(old, new, 1), "k3.hip") != base, (old, new)


def test_traffic_reported_only_for_the_code_it_was_taken_on(tmp_path, monkeypatch):
    src = tmp_path / "pkv_kernels.hip"
    src.write_text(SAMPLE, encoding="utf-8")
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps({"w": {"bytes_per_launch": 1234,
                                       "kernel_code_sha256": bench.kernel_code_digest(str(src))}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench.kernel_code_digest, "__defaults__", (str(src),))
    assert bench.measured_traffic("w") == 1234
    assert bench.measured_traffic("missing") is None
    src.write_text(SAMPLE.replace("// trailing comment", "// edited"), encoding="utf-8")
    assert bench.measured_traffic("w") == 1234
    src.write_text(SAMPLE.replace("2.0f", "4.0f"), encoding="utf-8")
    assert bench.measured_traffic("w") is None


def test_committed_traffic_table_is_well_formed():
    table = json.load(open(bench.TRAFFIC_FILE))
    for key, rec in table.items():
        assert int(rec["bytes_per_launch"]) > 0, key
        assert len(rec["kernel_code_sha256"]) == 64, key
        assert os.path.exists(os.path.join(ROOT, rec["profile"])), key


def test_host_workload_prints_one_contract_line():
    """The host-only prefix-cache workload runs without a GPU and prints one
    JSON line with the fields every bench line carries."""
    import subprocess
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "prefix-cache"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in rec, key
    assert rec["value"] > 0 and rec["n_gpus"] == 1 and "workload" in rec["config"]
    assert 0.0 < rec["block_hit_rate"] < 1.0


def test_more_than_one_gpu_is_refused():
    import subprocess
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in json.loads(out.stdout.strip().splitlines()[-1])["error"]
