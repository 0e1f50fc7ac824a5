"""Host logic of bench.py, on the CPU: the one-GPU refusal, the choice of
extras, the kernel-code hash that decides whether committed counters still
describe the kernel, and the roofline object built from them."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_extra_is_refused():
    r = _run("--extras", "ring32k,nonsense", "--no-cpu")
    assert r.returncode == 2
    assert "nonsense" in r.stderr


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {  // add one\n  return x + 1;\n}\n")
    h = bench.kernel_source_hash(str(src))
    src.write_text("// a new comment\n\nint f(int x) {  // add one more time\n  return x + 1;\n\n}\n")
    assert bench.kernel_source_hash(str(src)) == h
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash(str(src)) != h


def test_committed_profiles_parse_and_name_their_kernel():
    files = [f for pair in bench.ATTN_COUNTERS.values() for f in pair]
    files += [os.path.basename(bench.PERMUTE_TRAFFIC_FILE), os.path.basename(bench.REPLICATION_TRAFFIC_FILE)]
    for name in files:
        with open(os.path.join(bench.PROFILES, name)) as f:
            t = json.load(f)
        assert len(t["kernel_source_sha256_16"]) == 16, name
        assert t["commands"], name
        assert all("rocprofv3" in c for c in t["commands"]), name


def test_roofline_reads_counters_only_for_the_current_kernel(monkeypatch):
    ts = [10.0, 10.0, 12.0]
    live = bench.attn_roofline(bench.HEADLINE, 25 * 10 ** 12, ts)
    assert live["bound"] == "mfma" and live["peak"] == bench.PEAK_BF16_TFLOPS
    assert live["achieved"] == pytest.approx(25e12 / (32 / 3 * 1e-3) / 1e12, rel=1e-3)
    assert live["frac"] == pytest.approx(live["achieved"] / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert live["launch_ms_median"] == 10.0
    # the committed summaries either match the kernel (figures present) or do
    # not (null): never a figure taken on other code
    monkeypatch.setattr(bench, "kernel_source_hash", lambda path=None: "0" * 16)
    stale = bench.attn_roofline(bench.HEADLINE, 25 * 10 ** 12, ts)
    assert stale["traffic"] is None and stale["mfma_busy_pct_counters"] is None
