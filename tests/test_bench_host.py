"""CPU-only checks of bench.py's host side: the one-GPU contract, the algorithmic
byte and FLOP counts the roofline divides by, the host description of the CPU
baseline, and the rule that a recorded HBM traffic figure is used only for the
kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _inp(ctx, Hkv=4, Lq=1, Hq=32, fp8=False):
    B = len(ctx)
    kdt = np.uint8 if fp8 else np.uint16
    return {"ctx_len": np.asarray(ctx, np.int32),
            "k": np.zeros((B, Hkv, 8, 128), kdt),
            "q_full": np.zeros((B, Lq, Hq, 128), np.uint16)}


def test_kv_bytes_closed_form():
    # every visible K and V row of every KV head once: 2 x 128 x 2 B (bf16), or
    # 2 x (128 B + one fp32 scale) (fp8)
    assert bench.kv_bytes(_inp([1 << 20])) == (1 << 20) * 4 * 2 * 128 * 2 == 2147483648
    assert bench.kv_bytes(_inp([262144], fp8=True)) == 262144 * 4 * 2 * (128 + 4)
    assert bench.kv_bytes(_inp([100, 50], Hkv=2)) == 150 * 2 * 2 * 256


def test_scan_flops_counts_causal_positions():
    # decode: ctx positions x Hq x 4 x 128; a chunk of Lq tokens sees ctx-Lq+1 .. ctx
    assert bench.scan_flops(_inp([1000])) == 1000 * 32 * 4 * 128
    vis = sum(10 - 4 + j + 1 for j in range(4))
    assert bench.scan_flops(_inp([10], Lq=4)) == vis * 32 * 4 * 128


def test_host_description():
    h = bench.host_description()
    assert set(h) == {"cpu_model", "nproc", "usable_threads"}
    assert h["nproc"] >= 1 and 1 <= h["usable_threads"] <= h["nproc"]


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    rec = {"million": {"scan_source_sha256": bench.scan_source_hash(), "hbm_bytes_per_launch": 123},
           "stale": {"scan_source_sha256": "0" * 64, "hbm_bytes_per_launch": 456}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("million") == 123
    assert bench.measured_traffic("stale") is None
    assert bench.measured_traffic("absent") is None
