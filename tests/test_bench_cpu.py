"""bench.py's host logic on the CPU: the one-GPU refusal, the roofline choice and its
arithmetic, the traffic table, and the workloads' algorithmic bytes and flops."""
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)

import bench  # noqa: E402
from mla_split_kv_decode_amd import workloads as wk  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=REPO)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""  # no JSON line


def test_bad_step_counts_are_refused():
    res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--steps", "0"],
                         capture_output=True, text=True, timeout=120, cwd=REPO)
    assert res.returncode != 0 and res.stdout.strip() == ""


def test_roofline_hbm_side():
    # long32k: 37,748,736 KV bytes, 16 rows -> about 30 flop/B, far below the ridge
    kv_b = 37_748_736
    flops = 2 * (576 + 512) * 12 * 32_768
    r = bench.roofline_of(kv_b, flops, 10.0e-3, 44_474_368)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(kv_b / 10.0e-6 / 1e9, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    assert r["traffic"] == 44_474_368 and r["bytes_per_launch"] == kv_b


def test_roofline_mfma_side():
    # the 96-head FP8 shard: 363 flop/B, past the bf16 ridge of 312.5 flop/B
    wl = wk.make_workload("dcp_fp8")
    kv_b = wk.kv_bytes(wl.seq_lens, wl.kv_format)
    flops = bench.wk_flops(wl)
    assert flops / kv_b > bench.RIDGE_FLOP_PER_BYTE
    r = bench.roofline_of(kv_b, flops, 50.0e-3, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(flops / 50.0e-6 / 1e12, rel=1e-6)
    assert r["hbm_frac"] == pytest.approx(kv_b / 50.0e-6 / 1e9 / 8000.0, abs=1e-4)


def test_ridge_is_the_peak_ratio():
    assert bench.RIDGE_FLOP_PER_BYTE == pytest.approx(2500e12 / 8000e9)


def test_traffic_table():
    (name, splits, version), tr = next(iter(bench.TRAFFIC.items()))
    want = int(1024 * (tr["fetch_kib"] * tr["fetch_factor"] + tr["write_kib"] * tr["write_factor"]))
    assert bench.traffic_of(name, splits, version) == want
    # another library version (changed kernels) or split setting reads null
    assert bench.traffic_of(name, splits, version + " changed") is None
    assert bench.traffic_of(name, splits + 16, version) is None
    # every row is for one of the named workloads, at auto splits
    for (n, s, _), row in bench.TRAFFIC.items():
        assert n in wk.CONFIGS and s == 0
        assert row["fetch_kib"] > 0 and row["write_kib"] > 0


def test_traffic_covers_at_least_the_kv_bytes():
    # the counters can only add to the algorithmic bytes (the kernel reads every latent)
    for (n, s, v), _ in bench.TRAFFIC.items():
        wl = wk.make_workload(n) if n in ("tiny", "long32k", "dcp_fp8") else wk.timing_workload(n)
        assert bench.traffic_of(n, s, v) >= wk.kv_bytes(wl.seq_lens, wl.kv_format)


def test_algorithmic_bytes_and_flops():
    wl = wk.make_workload("long32k")
    assert wk.kv_bytes(wl.seq_lens, wl.kv_format) == 32_768 * 576 * 2
    # real heads only: 12 heads, one query token, every position visible
    assert bench.wk_flops(wl) == 2 * (576 + 512) * 12 * 32_768
