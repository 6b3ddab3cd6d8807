"""Host-side checks of bench.py that need no GPU: the single-GPU guard and the
rule that a stored HBM traffic figure applies only to the kernel source it was
measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_applies_only_to_the_measured_source(tmp_path, monkeypatch):
    sha = bench.source_sha256("ffn_prefill.hip")
    f = tmp_path / "traffic.txt"
    f.write_text("# comment\ngate_up_prefill_bytes=123\n"
                 f"gate_up_prefill_source_sha256={sha}\n"
                 "gate_up_decode_bytes=456\n"
                 f"gate_up_decode_source_sha256={'0' * 64}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("gate_up_prefill", "ffn_prefill.hip") == 123.0
    assert bench.measured_traffic("gate_up_decode", "ffn_decode.hip") is None  # source changed since
    assert bench.measured_traffic("dense_gate_up_prefill", "ffn_prefill.hip") is None  # never measured
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("gate_up_prefill", "ffn_prefill.hip") is None
