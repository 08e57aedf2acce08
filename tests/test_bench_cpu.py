"""Host-side checks of bench.py: the one-GPU guard, the roofline bound, the
rule that a counter summary only counts while the kernel sources match, and
the CPU-baseline leg (run on a tiny workload)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from seeded_inputs import WORKLOADS, make_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_counts_each_tensor_once():
    w = WORKLOADS["long_causal_16k"]
    # Q, K, V: 2 B/element; O: 2 B/element; LSE: 4 B per row
    assert bench.algorithmic_bytes(w, "bf16") == 16 * 16384 * (3 * 256 + 256 + 4)
    w8 = WORKLOADS["fp8_outliers_8k"]
    assert bench.algorithmic_bytes(w8, "fp8") == 4 * 32 * 8192 * (3 * 128 + 256 + 4)


@pytest.mark.parametrize("name,kind,bound", [
    ("long_causal_16k", "bf16", "mfma"),     # 4080 FLOP/B, far above the ridge
    ("llm_layer_4k", "bf16", "mfma"),
    ("fp8_outliers_8k", "fp8", "mfma"),
    ("vit_b16_batch64", "bf16", "hbm"),      # 97 FLOP/B, below the ~312 FLOP/B ridge
])
def test_roofline_bound_follows_the_ridge_point(name, kind, bound):
    w = WORKLOADS[name]
    peak = bench.PEAK["bf16"] if kind == "bf16" else 1 / (0.5 / bench.PEAK["fp8"] + 0.5 / bench.PEAK["bf16"])
    roof, alg = bench.roofline(w, kind, 1.0, peak)
    assert roof["bound"] == bound
    if bound == "hbm":
        assert roof["unit"] == "GB/s" and roof["peak"] == bench.HBM_PEAK_GBS
        assert roof["achieved"] == pytest.approx(alg / 1e-3 / 1e9, rel=1e-3)
    else:
        assert roof["unit"] == "TFLOP/s"
        assert roof["achieved"] == pytest.approx(w.flops / 1e-3 / 1e12, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)


def test_traffic_only_while_sources_match(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_hash": bench.kernel_hash("bf16"), "bytes_per_launch": 12345}
    (prof / "traffic_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_hash reads the sources under ROOT: point it back at the repository
    monkeypatch.setattr(bench, "kernel_hash", lambda kind, _h=rec["kernel_hash"]: _h)
    assert bench.traffic_from_profile("wl", "bf16") == 12345
    monkeypatch.setattr(bench, "kernel_hash", lambda kind: "0" * 16)
    assert bench.traffic_from_profile("wl", "bf16") is None
    assert bench.traffic_from_profile("missing", "bf16") is None


def test_committed_traffic_summaries_name_their_kernel_sources():
    for wl, kind in (("long_causal_16k", "bf16"), ("fp8_outliers_8k", "fp8")):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"traffic_{wl}.json")))
        assert len(rec["kernel_hash"]) == 16
        assert abs(rec["bytes_per_launch"] - rec["read_bytes"] - rec["write_bytes"]) <= 1
        assert os.path.exists(os.path.join(ROOT, rec["source"]))


def test_cpu_baseline_reports_the_oracle_sample():
    w = WORKLOADS["long_causal_16k"].with_(B=1, H=2, N=64)
    inp = make_inputs(w)
    r = bench.cpu_baseline(inp, budget_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert r["sample"].startswith("1 head evaluations over the workload's 2 heads (all 64 query rows each)")


def test_backward_is_counted_as_two_and_a_half_forwards():
    w = WORKLOADS["long_causal_16k"]
    assert bench.algorithmic_flops(w, "bwd") == 2.5 * w.flops
    assert bench.algorithmic_bytes(w, "bwd") == 16 * 16384 * (10 * 128 + 4 + 6 * 128 + 8)
    roof, _ = bench.roofline(w, "bwd", 1.0, bench.PEAK["bf16"])
    assert roof["bound"] == "mfma"
    assert roof["achieved"] == pytest.approx(2.5 * w.flops / 1e-3 / 1e12, rel=1e-3)


def test_cpu_baseline_of_the_backward_reports_the_oracle_sample():
    from seeded_inputs import make_output_grad
    w = WORKLOADS["long_causal_16k"].with_(B=1, H=2, N=64)
    r = bench.cpu_baseline_bwd(make_inputs(w), make_output_grad(w), budget_s=0.0)
    assert r["kind"] == "oracle" and r["value"] > 0
    assert r["sample"].startswith("1 head evaluations over the workload's 2 heads (dQ, dK, dV of all 64 rows")
