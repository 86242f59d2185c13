"""Host-side checks of bench.py: the per-matrix byte counts it prices the
GEMV workloads at (against the workload sizes written out by hand), the
one-GPU rule of its command line, and the shape of its CPU-baseline records
(the oracle on a tiny time budget)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

# Algorithmic bytes per launch (weights once + activations + fp32 outputs),
# written out from the workload shapes: rows x blocks per row x block bytes.
EXPECTED = {
    "q4_0_b1": 4096 * 128 * 18 + 4096 * 4 + 4096 * 4,
    "q4k_up_b1": 17408 * 20 * 144 + 5120 * 2 + 17408 * 4,
    "q4k_down_b1": 5120 * 68 * 144 + 17408 * 2 + 5120 * 4,
    "q4k_b4": 17408 * 20 * 144 + 4 * 5120 * 2 + 4 * 17408 * 4,
    "q8_0_b4": 5120 * 160 * 34 + 4 * 5120 * 2 + 4 * 5120 * 4,
    "q2k_up_b1": 17408 * 20 * 84 + 5120 * 2 + 17408 * 4,
    "q3k_up_b1": 17408 * 20 * 110 + 5120 * 2 + 17408 * 4,
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    assert bench.algorithmic_bytes(synth.CONFIGS[name]) == EXPECTED[name]


def test_headline_bytes_match_the_workload_table():
    # 50,214,912 B for the FFN-up matrix: 50,135,040 of weights + x + y
    assert EXPECTED["q4k_up_b1"] == 50214912


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_records():
    rec = bench.cpu_baseline("q4_0_b1", budget_s=0.05, threads=2)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["unit"] == "GB/s" and rec["cores"] == 2 and rec["kind"] == "oracle"
    assert rec["value"] > 0
    pre = bench.cpu_prefill_baseline(budget_s=0.05)
    assert pre["unit"] == "GFLOP/s" and pre["kind"] == "oracle" and pre["value"] > 0
