"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the stored
HBM-traffic record that `roofline.traffic` is read from."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_traffic_record_parses_and_is_consistent():
    text = open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)).read()
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == 8 * 8192 * 2 * 8 * 128 * 2
    # the scaled counters are in bytes: fetch KiB x scale x 1024
    assert abs(rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] * 1024 - rec["hbm_read_bytes_per_launch"]) \
        < 1e-3 * rec["hbm_read_bytes_per_launch"]


def test_traffic_is_dropped_when_kernel_sources_change(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.stored_traffic() is None
    assert bench.roofline(268435456, 0.0625)["traffic"] is None


def test_prefill_flops_count_visible_keys_only():
    """Whole-prompt window of 10 tokens: rows see 1..10 keys (55 in all);
    a 5-token chunk over 15 cached tokens: rows see 16..20 keys (90)."""
    from workloads import AttnCase
    import numpy as np
    q = np.zeros((15, 2, 4), np.uint16)
    pool = np.zeros((1, 1, 256, 4), np.uint16)
    case = AttnCase("t", q, pool, pool, np.zeros((2, 1), np.int32), np.array([10, 20], np.int32),
                    np.array([10, 5], np.int32), 0.5)
    assert bench.prefill_flops(case) == (55 + 90) * 2 * 4 * 4
