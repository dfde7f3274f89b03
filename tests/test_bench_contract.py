"""bench.py's contract: one JSON line with the fields the measurement needs, a
refusal to run on more than one GPU, HBM-traffic figures reported only for the
build they were measured on, and the oracle's CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_hash_follows_sources_and_flags(monkeypatch):
    from diffusion_transformer_video_amd import build as b
    h = bench.kernel_sha()
    assert h == bench.kernel_sha() and len(h) == 16
    flags = dict(b.FILE_FLAGS)
    flags["k_attn_bf16.hip"] = flags["k_attn_bf16.hip"] + ["-DSOMETHING_ELSE"]
    monkeypatch.setattr(b, "FILE_FLAGS", flags)
    assert bench.kernel_sha() != h


def test_traffic_only_for_the_measured_build(tmp_path, monkeypatch):
    tj = tmp_path / "traffic.json"
    tj.write_text(json.dumps({"w_same": {"source_sha": bench.kernel_sha(), "traffic_bytes_per_launch": 123},
                              "w_old": {"source_sha": "0" * 16, "traffic_bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tj))
    assert bench.traffic_for("w_same") == 123
    assert bench.traffic_for("w_old") is None
    assert bench.traffic_for("w_missing") is None


def test_committed_traffic_figures_name_their_kernel():
    t = json.load(open(bench.TRAFFIC_FILE))
    for name, e in t.items():
        assert e["kernel"].startswith("attn_bf16_"), name
        assert e["traffic_bytes_per_launch"] > 0 and len(e["source_sha"]) == 16
        assert os.path.exists(os.path.join(ROOT, e["summary"])), e["summary"]


def test_cpu_baseline_fields():
    import synth
    r = bench.cpu_baseline(synth.WORKLOADS["c1_tiny_f32"], 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1 and "oracle" in r["sample"]


@pytest.mark.gpu
def test_bench_json_line_on_the_gpu():
    from gpu_util import need_gpu
    need_gpu()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "c1", "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["config"]["workload"] == "c1_tiny_f32"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in d["roofline"], key
