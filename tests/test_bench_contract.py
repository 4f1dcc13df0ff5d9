"""The benchmark's host-side contract, checked without a GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_key_stream_bytes_per_entry():
    # D/2 code bytes + D/16 E4M3 scale bytes + the page's fp32 global scale and int32
    # block-table entry shared by the page's keys
    assert bench.key_bytes_per_entry(128, 64) == pytest.approx(72.125)
    assert bench.key_bytes_per_entry(64, 16) == pytest.approx(32 + 4 + 0.5)


def test_workloads_cover_the_five_configurations():
    configs = sorted(v for v in bench.WORKLOADS.values() if v != "diag")
    assert configs == [1, 2, 3, 4, 5]
    assert bench.WORKLOADS["decode_T8_S65536"] == 2
    assert set(bench.COLD_WORKLOADS) <= set(bench.WORKLOADS)


def test_traffic_entries_name_known_sources():
    for w, (kind, sha, fetch, write) in bench.SCORER_TRAFFIC.items():
        assert w in bench.WORKLOADS
        assert kind in bench.SCORER_SOURCES
        assert len(sha) == 16 and fetch > 0 and write > 0
