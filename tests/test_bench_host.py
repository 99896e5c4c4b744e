"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic byte and flop counts its rooflines divide by."""

import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_counts_of_the_graded_workloads():
    d = synth.WORKLOADS["decode_large"]
    # K and V of every position (bf16), q and rho (bf16), fp32 out
    assert bench.decode_bytes(d.B, d.H, d.D, [d.L] * d.B) == 17_184_063_488
    p = synth.WORKLOADS["prefill_bf16"]
    # four contractions of 2 D flops per causal (query, key) pair
    assert bench.prefill_flops(p.B, p.N, p.H, p.D) == 1_099_780_063_232
    assert bench.backward_flops(p.B, p.N, p.H, p.D) == 2 * 1_099_780_063_232
    # one sequence of one head: N (N + 1) / 2 causal pairs
    assert bench.prefill_flops(1, 3, 1, 1) == 8 * 6


def test_traffic_is_dropped_when_the_kernel_source_changed(tmp_path, monkeypatch):
    rec = {"decode": {"source_sha256": bench.source_hash("decode.hip", "decode_common.h"),
                      "bytes_per_launch": 123.0},
           "prefill": {"source_sha256": "0" * 64, "bytes_per_launch": 456.0}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(f))
    assert bench.traffic_for("decode", ["decode.hip", "decode_common.h"]) == 123.0
    assert bench.traffic_for("prefill", ["fwd_mfma.hip", "pack.hip"]) is None
    assert bench.traffic_for("absent", ["decode.hip"]) is None
