"""CPU checks of bench.py's contract: one GPU only, and profile figures
(HBM traffic, MFMA busy and clock) reported only while the committed
rocprofv3 summaries were taken on the current kernel source."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_digest_ignores_comments_only():
    a = "int f(int x) { return x + 1; } // one\n/* block */"
    b = "int f(int x) {\n  return x + 1;   // two\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("+ 1", "+ 2"))


def _with_profile(tmp_path, monkeypatch, name, payload):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    (prof / name).write_text(json.dumps(payload))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "d1")


def test_traffic_reported_only_for_the_current_digest(tmp_path, monkeypatch):
    _with_profile(tmp_path, monkeypatch, "dgrad_fused_target_traffic.json",
                  {"source_digest": "d1", "hbm_bytes_per_launch": 123})
    assert bench.measured_traffic("dgrad_fused_target") == 123
    monkeypatch.setattr(bench, "source_digest", lambda: "d2")
    assert bench.measured_traffic("dgrad_fused_target") is None
    assert bench.measured_traffic("no_such_kernel") is None


def test_mfma_counters_reported_only_for_the_current_digest(tmp_path, monkeypatch):
    _with_profile(tmp_path, monkeypatch, "dgrad_fused_target_mfma.json",
                  {"source_digest": "d1", "mfma_busy_pct": 62.0, "clock_ghz": 1.73,
                   "pct_of_peak_at_2p4ghz": 44.7, "command": "x"})
    assert bench.measured_mfma("dgrad_fused_target") == {"mfma_busy_pct": 62.0, "clock_ghz": 1.73,
                                                         "pct_of_peak_at_2p4ghz": 44.7}
    monkeypatch.setattr(bench, "source_digest", lambda: "d2")
    assert bench.measured_mfma("dgrad_fused_target") is None


def test_committed_profiles_name_their_digest():
    for name in ("dgrad_fused_target_traffic.json", "dgrad_fused_target_mfma.json",
                 "forward_decode_traffic.json", "dgrad_fused_moe_traffic.json"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            t = json.load(f)
        assert len(t["source_digest"]) == 16, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_byte_ledger_counts_the_tensors_each_step_moves():
    """bench.py's algorithmic bytes per launch (the roofline's `achieved`
    for the decode forward, the fused dgrad's byte figure) against the bf16
    sizes of the arrays the oracle's step functions read and write."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from test_oracle import _ledger_arrays
    M, D, I, Dout = 97, 64, 160, 48
    fused, forward, _ = _ledger_arrays(M, D, I, Dout)
    assert bench.fused_dgrad_bytes(M, I, Dout) == 2 * sum(a.size for a in fused)
    assert bench.forward_bytes(M, D, I, Dout) == 2 * sum(a.size for a in forward)
    # grouped over E experts: each expert's W_down is read once
    E = 5
    assert bench.fused_dgrad_bytes(M, I, Dout, experts=E) == 2 * sum(a.size for a in fused) + 2 * (E - 1) * I * Dout
