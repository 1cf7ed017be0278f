"""Host-side logic of bench.py (no GPU): the one-GPU contract and the traffic figure's guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def _recorded_fields():
    with open(bench.TRAFFIC_FILE) as f:
        return dict(line.strip("` \n").split("=", 1) for line in f
                    if line.startswith("`") and "=" in line)


def test_traffic_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    fields = _recorded_fields()
    assert set(fields) >= {"traffic_bytes_per_launch", "source_sha256"}
    recorded = int(float(fields["traffic_bytes_per_launch"]))
    # the counter summary is for the fused gate_up launch at decode T=1: 4 experts' gate_up
    # weight bytes (35,251,200) plus a few percent of activations, biases and logits
    assert 35_251_200 <= recorded < 1.1 * 35_251_200
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: fields["source_sha256"])
    assert bench.measured_traffic() == recorded
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic() is None


def test_source_hash_covers_the_fused_decode_sources():
    h0 = bench.kernel_source_hash()
    assert len(h0) == 64 and h0 == bench.kernel_source_hash()   # deterministic
    csrc = os.path.join(ROOT, "mxfp4_mixture_experts_route_amd", "csrc")
    for name in bench.TRAFFIC_SOURCES:
        assert os.path.exists(os.path.join(csrc, name)), name
