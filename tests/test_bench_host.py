"""Host-side parts of bench.py (no GPU): the one-GPU guard, the traffic figure read
from the committed rocprofv3 summaries, and the CPU-baseline record."""

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tpmlp_inputs import mlp_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


@pytest.mark.parametrize("kernel_file,summary", [("gemm_bf16.hip", "gemm_bf16_gpt8p3b_t8_traffic.md"),
                                                 ("reduce.hip", "reduce_gpt8p3b_t8_traffic.md")])
def test_recorded_traffic_follows_the_source_hash(kernel_file, summary):
    # the figure is reported exactly when the counters were taken on this source
    text = open(os.path.join(ROOT, "profiles", summary)).read()
    src = open(os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc", kernel_file), "rb").read()
    same = f"source_sha256: {hashlib.sha256(src).hexdigest()}" in text
    v = bench.recorded_traffic(kernel_file, summary)
    if same:
        assert v is not None and v > 0
    else:
        assert v is None


def test_recorded_traffic_is_withheld_for_a_changed_source(tmp_path, monkeypatch):
    # a summary whose hash names another source: the figure is not reported
    prof = tmp_path / "profiles"
    prof.mkdir()
    text = open(os.path.join(ROOT, "profiles", "reduce_gpt8p3b_t8_traffic.md")).read()
    lines = [("source_sha256: " + "0" * 64) if ln.startswith("source_sha256:") else ln for ln in text.splitlines()]
    (prof / "reduce_gpt8p3b_t8_traffic.md").write_text("\n".join(lines))
    csrc = tmp_path / "megatron_tensor_transformer_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "reduce.hip").write_bytes(
        open(os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc", "reduce.hip"), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("reduce.hip", "reduce_gpt8p3b_t8_traffic.md") is None
    assert bench.recorded_traffic("reduce.hip", "missing.md") is None


def test_cpu_baseline_record():
    inp = mlp_inputs(64, 32, 64, 2, dtype="bf16", seed=0)
    rec = bench.cpu_baseline(inp, 2, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "whole-shard passes" in rec["sample"]
