"""Host logic of bench.py (no GPU): the one-GPU guard and the HBM-traffic figures taken from
the committed rocprofv3 counter summaries."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("cls", ["gemm_head", "gemm_gateup"])
def test_traffic_only_for_the_counted_source_and_weights(cls):
    with open(os.path.join(ROOT, "profiles", f"pmc_{cls}_full.json")) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "dflash2_block_drafter_amd", "csrc", rec["source"])
    current = hashlib.sha256(open(src, "rb").read()).hexdigest() == rec["source_sha256"]
    got = bench.pmc_traffic(cls, "full")
    # reported exactly when the kernel source is the one the counters were taken on
    assert (got == rec["hbm_bytes_per_launch"]) if current else (got is None)
    # the counters were taken with bf16 weights: no figure for a 4-bit run
    assert bench.pmc_traffic(cls, "full", "q4") is None
    assert bench.pmc_traffic(cls, "long") is None  # no counters for that workload
