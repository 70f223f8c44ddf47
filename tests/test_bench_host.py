"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
bytes and flops per head-token it divides by, and the rule that counter-based
traffic is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8", "--steps", "1"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_forward_bytes_and_flops_per_token():
    """q, k, v (and gate inputs) read once, o written once; chunk-64 MFMA work."""
    assert bench.algorithmic_per_token(WORKLOADS["causal_elu1"]) == (512, 24704.0)
    assert bench.algorithmic_per_token(WORKLOADS["gla_gate"])[0] == 1280       # + g, r per token
    assert bench.algorithmic_per_token(WORKLOADS["outer_gate"])[0] == 1536     # + g and gv
    assert bench.algorithmic_per_token(WORKLOADS["ssm_scalar"])[0] == 514      # + one g per token
    assert bench.algorithmic_per_token(WORKLOADS["favor_causal"]) == (512, 151872.0)
    assert bench.algorithmic_per_token(WORKLOADS["noncausal_elu1_f32"])[0] == 4 * (2 * 32 + 32) + 4 * 32


def test_backward_bytes_per_token():
    """q, k, v, dO read, dq, dk, dv written (gate inputs and dg on top)."""
    assert bench.backward_algorithmic_per_token(WORKLOADS["causal_elu1"])[0] == 896
    gla64 = WORKLOADS["gla_gate"].resized(d_k=64, d_v=64, r=64)
    assert bench.backward_algorithmic_per_token(gla64)[0] == 1152
    assert bench.backward_algorithmic_per_token(WORKLOADS["ssm_scalar"])[0] == 900
    # the outer-product gate: q, k, v, dO, dq, dk, dv, g, dg (d = 128) and gv, dgv (d_v = 128), bf16
    assert bench.backward_algorithmic_per_token(WORKLOADS["outer_gate"])[0] == 2 * 128 * 11
    assert bench.backward_algorithmic_per_token(WORKLOADS["noncausal_elu1_f32"])[0] == 4 * (2 * 32 + 2 * 32) + 4 * (2 * 32 + 32)


def test_traffic_only_for_the_measured_sources(monkeypatch, tmp_path):
    """Counter traffic is reported per kernel, and only for the kernel sources
    the counters were taken on."""
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "gla_gate", "source_digest": "abcd" * 4,
           "kernels": {"causal_chunk_forward": {"hbm_bytes_per_launch": 123456789}}}
    (tmp_path / "profiles" / "traffic_gla_gate.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abcd" * 4)
    assert bench.measured_traffic("gla_gate", "causal_chunk_forward") == 123456789
    assert bench.measured_traffic("gla_gate", "segment_scan_kernel") is None
    assert bench.measured_traffic("no_such_workload", "causal_chunk_forward") is None
    # the matrix-core counters ride in the same record
    assert bench.measured_mfma("gla_gate", "causal_chunk_forward") is None
    rec["kernels"]["causal_chunk_forward"].update(kernel="causal_chunk_forward<128, 128, 128, 0, 2>",
                                                 mfma_flops=4.8e10, mfma_tflops=240.0, mfma_frac=0.0954,
                                                 mfma_busy=0.0977, avg_us=200.0)
    (tmp_path / "profiles" / "traffic_gla_gate.json").write_text(json.dumps(rec))
    m = bench.measured_mfma("gla_gate", "causal_chunk_forward")
    assert m["issued_flops_per_launch"] == 4.8e10 and m["busy_frac"] == 0.0977 and m["issued_frac"] == 0.0954
    # any change to the kernel sources voids it
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.measured_traffic("gla_gate", "causal_chunk_forward") is None
    assert bench.measured_mfma("gla_gate", "causal_chunk_forward") is None


def test_roofline_takes_the_dominant_kernel(monkeypatch):
    wl = WORKLOADS["gla_gate"]
    monkeypatch.setattr(bench, "measured_traffic", lambda w, k: None)
    res = {"kernels": [{"name": "causal_segment_state", "avg_ms": 0.1}, {"name": "segment_scan_kernel", "avg_ms": 0.01},
                       {"name": "causal_chunk_forward", "avg_ms": 0.2}],
           "hbm_alg_GBs": 1.0, "hbm_frac": 0.1, "ms_per_step": 0.31}
    r = bench.roofline(wl, res)
    assert r["kernel"] == "causal_chunk_forward"
    alg = wl.head_tokens * 1280
    assert r["alg_bytes_per_launch"] == alg
    assert abs(r["achieved"] - alg / 0.2e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4


def test_kernel_names_follow_the_plan():
    assert bench.forward_kernel_names(WORKLOADS["gla_gate"], 8) == [
        "gla_segment_state", "segment_scan_kernel", "causal_chunk_forward"]
    assert bench.forward_kernel_names(WORKLOADS["causal_elu1"], 8) == [
        "causal_segment_state", "segment_scan_kernel", "causal_chunk_forward"]
    assert bench.forward_kernel_names(WORKLOADS["gla_gate"].resized(d_k=32, r=32), 8)[0] == "causal_segment_state"
    assert bench.forward_kernel_names(WORKLOADS["favor_causal"], 1) == ["favor_chunk_forward"]
    assert bench.forward_kernel_names(WORKLOADS["noncausal_elu1_f32"], 1) == ["nc_partial", "nc_readout"]
    t = bench.kernel_table([[1.0, 2.0], [3.0, 4.0]], ["a", "b"])
    assert t == [{"name": "a", "avg_ms": 2.0, "min_ms": 1.0}, {"name": "b", "avg_ms": 3.0, "min_ms": 2.0}]
