"""Host-side behaviour of bench.py (no GPU): argument refusal, and the
committed-profile lookups that attach rocprofv3 figures to the JSON line
only while they describe the current kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    out = _run("--gpus", "2")
    assert out.returncode == 2
    assert "one GPU" in out.stderr


@pytest.mark.parametrize("args", [("--steps", "0"), ("--warmup", "-1"), ("--streams", "0"), ("--graph-steps", "0")])
def test_bad_counts_are_refused(args):
    out = _run(*args)
    assert out.returncode == 2
    assert "at least" in out.stderr


def test_profile_keys_parse_the_committed_summaries():
    kv = bench.read_profile_keys("traffic_paged_q4.txt")
    assert kv is not None
    assert int(kv["algorithmic_bytes_per_launch"]) == 2 * 32 * 256 * bench.q_row_bytes(4)
    assert bench.read_profile_keys("no_such_summary.txt") is None


def test_rocprof_check_reports_the_offset_or_why_not(monkeypatch):
    kv = bench.read_profile_keys("paged_q4_kernel_trace.txt")
    assert kv is not None and "sources_sha256" in kv
    tq = float(kv["quant_trace_mean_ns"]) / 1000.0
    td = float(kv["dequant_trace_mean_ns"]) / 1000.0
    monkeypatch.setattr(bench, "sources_digest", lambda: kv["sources_sha256"])
    r = bench.rocprof_check({"quant": tq * 1.02, "dequant": td * 0.99})
    assert r["trace_mean_us"] == {"quant": round(tq, 3), "dequant": round(td, 3)}
    assert r["event_vs_trace"] == {"quant": "+2.0%", "dequant": "-1.0%"}
    monkeypatch.setattr(bench, "sources_digest", lambda: "0" * 64)
    r = bench.rocprof_check({"quant": tq, "dequant": td})
    assert "trace_mean_us" not in r and r["reason"] == "taken on other kernel sources"


def test_traffic_is_dropped_for_other_kernel_sources(monkeypatch):
    kv = bench.read_profile_keys("traffic_paged_q4.txt")
    monkeypatch.setattr(bench, "sources_digest", lambda: kv["sources_sha256"])
    t, src = bench.traffic_for("quant", int(kv["algorithmic_bytes_per_launch"]))
    assert t == float(kv["quant_traffic_bytes_per_launch"]) and "same kernel sources" in src
    monkeypatch.setattr(bench, "sources_digest", lambda: "0" * 64)
    t, src = bench.traffic_for("quant", int(kv["algorithmic_bytes_per_launch"]))
    assert t is None and "other kernel sources" in src


def test_source_digest_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "kv_cache_quantization_kvq_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("kvq_kernels.hip", "kvq_device.h", "kvq_internal.h"):
        (csrc / f).write_text("int f(int a) { return a + 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.sources_digest()
    (csrc / "kvq_device.h").write_text("// a comment\nint f(int a)\n{\n    return a + 1;   /* same */\n}\n")
    assert bench.sources_digest() == d0
    (csrc / "kvq_device.h").write_text("int f(int a) { return a + 2; }\n")
    assert bench.sources_digest() != d0
