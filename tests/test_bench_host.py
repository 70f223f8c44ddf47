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
    assert bench.backward_algorithmic_per_token(WORKLOADS["noncausal_elu1_f32"])[0] == 4 * (2 * 32 + 2 * 32) + 4 * (2 * 32 + 32)


def test_traffic_only_for_the_measured_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_causal_elu1.json")
    with open(path) as f:
        rec = json.load(f)
    # reported for the sources the counters were taken on
    monkeypatch.setattr(bench, "source_digest", lambda: rec["source_digest"])
    assert bench.measured_traffic("causal_elu1") == rec["hbm_bytes_per_step"]
    # any change to the kernel sources voids it
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.measured_traffic("causal_elu1") is None
    assert bench.measured_traffic("no_such_workload") is None
