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
    configs = sorted(v for v in bench.WORKLOADS.values() if isinstance(v, int))
    assert configs == [1, 2, 3, 4, 5]
    assert bench.WORKLOADS["decode_T8_S65536"] == 2
    assert set(bench.COLD_WORKLOADS) <= set(bench.WORKLOADS)


def test_traffic_entries_name_known_sources():
    for w, (kind, sha, fetch, write) in bench.SCORER_TRAFFIC.items():
        assert w in bench.WORKLOADS
        assert kind in bench.SCORER_SOURCES
        assert len(sha) == 16 and fetch > 0 and write > 0


def test_default_workload_is_the_long_context_decode():
    assert bench.DEFAULT_WORKLOAD == "long_decode_T32_S262144"
    assert bench.WORKLOADS[bench.DEFAULT_WORKLOAD] == 3


def test_roofline_bound_follows_the_unique_byte_intensity():
    from workloads.configs import csa

    def wl(table):
        return csa("rf", [5], T=8, H=64, D=128, epb=64, P=8 * 40, max_lb=40, top_k=64,
                   valid_lens=[2560] * 8, dist="tiny", table=table)

    shared = bench.csa_roofline(wl("shared"), 10e-6, "mfma")     # 8 rows share every page
    own = bench.csa_roofline(wl("disjoint"), 10e-6, "mfma")       # every row on its own pages
    assert shared["bound"] == "mfma" and shared["unit"] == "TFLOP/s"
    assert own["bound"] == "hbm" and own["unit"] == "GB/s"
    flops = 2.0 * 8 * 2560 * 64 * 128
    assert shared["flops_per_launch"] == int(flops)
    assert shared["achieved"] == pytest.approx(flops / 10e-6 / 1e12, rel=1e-3)
    # per-stream bytes equal for both; the key bytes are 8x smaller when the pages are shared (q and
    # the scores are the same in both)
    assert shared["bytes_per_launch"] == own["bytes_per_launch"]
    assert own["unique_bytes_per_launch"] > 3 * shared["unique_bytes_per_launch"]
    # the FP32 path at D 128 runs on the fp32 matrix cores: its own peak, 157.3 TFLOP/s
    f32 = bench.csa_roofline(wl("shared"), 10e-6, "fp32")
    assert f32["bound"] == "mfma" and f32["peak"] == 157.3 and f32["kernel"] == "score_f32mfma_kernel"
    assert f32["frac"] == pytest.approx(flops / 10e-6 / 1e12 / 157.3, rel=1e-3)
