"""bench.py's host-side contract, on the CPU: the one-GPU guard, the
algorithmic byte counts it divides by, and the gating of counter-derived HBM
traffic on the kernel sources the counters were taken from."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes():
    # one [1536, 1536] GEMV: 1,327,104 weight bytes + 3,072 x + 6,144 y
    assert bench.q4_bytes(1536, 1536) == 1_336_320
    assert bench.weight_bytes(1536, 1536) == 1_327_104
    # E4B decode step: 42 x {QKV, O, gate+up, down} + the head
    mats = synth.stack_e4b_matrices()
    assert len(mats) == 42 * 4 + 1
    per_layer = sum(bench.weight_bytes(n, k) for _, n, k in mats[:4])
    assert per_layer == 51_609_600
    assert sum(bench.weight_bytes(n, k) for _, n, k in mats) == 2_545_090_560


def test_traffic_is_gated_on_the_kernel_sources(tmp_path, monkeypatch):
    good = {"kernel_source_hash": bench.kernel_source_hash(),
            "shapes": {"gate_up": {"hbm_bytes_per_launch": 12345}}}
    path = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.load_traffic("gate_up") is None  # no file
    path.write_text(json.dumps(good))
    assert bench.load_traffic("gate_up") == 12345
    assert bench.load_traffic("no such shape") is None
    stale = dict(good, kernel_source_hash="0" * 16)
    path.write_text(json.dumps(stale))
    assert bench.load_traffic("gate_up") is None


def test_host_cpu_model_is_named():
    m = bench.host_cpu_model()
    assert isinstance(m, str) and m


def test_profiler_modes_parse(monkeypatch):
    # the single-purpose runs that the rocprofv3 summaries are taken with
    monkeypatch.setattr(sys, "argv", ["bench.py", "--verify-pass"])
    assert bench.parse().verify_pass
    monkeypatch.setattr(sys, "argv", ["bench.py", "--heads-once"])
    assert bench.parse().heads_once
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gemm-shapes", "16384x2560,20480x2560"])
    a = bench.parse()
    assert not a.verify_pass
    assert [tuple(int(v) for v in s.split("x")) for s in a.gemm_shapes.split(",")] == [(16384, 2560), (20480, 2560)]
