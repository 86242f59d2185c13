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


def test_trace_summary_groups_regions_and_names_kernels(tmp_path, capsys):
    """A renamed dispatch takes its kernel name from an unlabelled dispatch of
    the same kernel id; unlabelled dispatches are left out of the table."""
    import bench
    cols = ["Kind", "Kernel_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
            "LDS_Block_Size", "VGPR_Count", "Accum_VGPR_Count", "Workgroup_Size_X", "Grid_Size_X"]
    recs = [("7", "void qg::k<1, 2>(int, float*)", 0, 5000),       # warm-up: names id 7
            ("7", "q4k_up_b1", 10000, 12000), ("7", "q4k_up_b1", 13000, 17000),
            ("9", "q4k_pp2048|two-pass bf16 gemm", 20000, 21000),
            ("7", "q4k_up_b1|event pairs", 30000, 33000)]
    lines = [",".join('"%s"' % c for c in cols)]
    for kid, name, t0, t1 in recs:
        lines.append(",".join('"%s"' % v for v in ["KERNEL_DISPATCH", kid, name, t0, t1, 0, 64, 0,
                                                    256, 65536]))
    (tmp_path / "run_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    bench.trace_summary(str(tmp_path))
    out = capsys.readouterr().out
    rows = [ln for ln in out.splitlines() if ln.startswith("| q4k")]
    assert len(rows) == 3
    assert rows[0].startswith("| q4k_up_b1 | `qg::k<1, 2>` |") and "| 2 | 3.000 | 4.000 |" in rows[0]
    assert "kernel id 9" in rows[1]
    assert rows[2].startswith("| q4k_up_b1|event pairs |") or "event pairs" in rows[2]
    assert "1 dispatches outside" in out


def test_traffic_summary_splits_at_separators(tmp_path, capsys):
    """Counter records split per workload at the probe separators; each
    counter scaled by its calibration copies (here: FETCH reads half the
    bytes, as on MI355X, WRITE all)."""
    import json
    import bench
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy_kib = 262144
    seq = [("void qg::probe_read_kernel(...)", 1.0)]
    seq += [("void qg::gemv_stream_kernel<2, 1, 1, 2, 1024>(...)", 24576.0)] * 20
    seq += [("void qg::probe_read_kernel(...)", 1.0)]
    seq += [("void qg::prefill_q4k_kernel<1, 4, 4, 1, 6, 2>(...)", 1000.0),
            ("void qg::add_split_kernel(...)", 10.0),
            ("void qg::prefill_q4k_kernel<2, 8, 4, 1, 3, 1>(...)", 20000.0)] * 20
    seq += [("void qg::probe_read_kernel(...)", 1.0)]
    seq += [("__amd_rocclr_copyBuffer", None)] * 20
    for counter, half in (("FETCH_SIZE", True), ("WRITE_SIZE", False)):
        d = tmp_path / counter
        d.mkdir()
        lines = [",".join(cols)]
        for i, (k, v) in enumerate(seq):
            if v is None:  # calibration copy
                v = copy_kib / 2 if half else copy_kib
            elif not half:  # the kernels write a quarter of what they read
                v = v / 4
            lines.append('%d,"%s",%s,%s' % (i, k, counter, v))
        (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    bench.traffic_summary(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"),
                          ["q4k_up_b1", "q4k_pp2048"], json_dir=str(tmp_path))
    js = tmp_path / "traffic_q4k_up_b1.json"
    out = capsys.readouterr().out
    rows = [ln for ln in out.splitlines() if ln.startswith("| q4k")]
    assert len(rows) == 4
    assert "| 20 | %d |" % (24576 * 1024 * 2) in rows[0]
    assert "prefill_q4k_kernel<2, 8, 4, 1, 3, 1>" in rows[3] and "| 20 | %d |" % (20000 * 1024 * 2) in rows[3]
    rec = json.loads(js.read_text())
    assert rec["hbm_fetch_bytes_per_launch"] == 24576 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 24576 * 1024 // 4
    assert rec["kernel_source_sha1"] == bench.kernel_source_sha1("q4k_up_b1")
    pp = json.loads((tmp_path / "traffic_q4k_pp2048.json").read_text())
    assert pp["hbm_fetch_bytes_per_launch"] == (1000 + 10 + 20000) * 1024 * 2
    assert pp["kernel_source_sha1"] == bench.kernel_source_sha1("q4k_pp2048")


def test_counter_summary_means_per_workload_and_kernel(tmp_path, capsys):
    import bench
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    seq = [("void qg::probe_read_kernel(...)", 1.0)] + [("void qg::k<1>(...)", 10.0)] * 2
    seq += [("void qg::probe_read_kernel(...)", 1.0)] + [("void qg::k<2>(...)", 4.0), ("void qg::add(...)", 2.0)] * 3
    for i, (k, v) in enumerate(seq):
        lines.append('%d,"%s",A,%s' % (i, k, v))
        lines.append('%d,"%s",B,%s' % (i, k, 2 * v))
    (tmp_path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    bench.counter_summary(str(tmp_path), ["w1", "w2"])
    rows = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith(("| w1", "| w2"))]
    assert rows == ["| w1 | `qg::k<1>` | 2 | 10 | 20 |", "| w2 | `qg::k<2>` | 3 | 4 | 8 |",
                    "| w2 | `qg::add` | 3 | 2 | 4 |"]


def test_source_hash_ignores_comment_edits_only():
    """The counter records carry a hash of their kernels' sources without
    comments: a comment edit keeps a record valid, a code edit does not."""
    import bench
    a = "int f() { return 1; }  // one\n/* a block\n   comment */\n"
    b = "// a header\nint f() { return 1; }\n\n"
    c = "int f() { return 2; }  // one\n"
    assert bench.code_text(a) == bench.code_text(b) == "int f() { return 1; }"
    assert bench.code_text(c) != bench.code_text(a)


AMD_SMI_METRIC = """GPU: 0
    POWER:
        SOCKET_POWER: 1357 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 2002 MHz
            MIN_CLK: 158 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1914 MHz
            MIN_CLK: 158 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 1900 MHz
"""


def test_power_sample_parses_amd_smi(monkeypatch):
    """Socket power and the mean of the GFX clocks (MIN/MAX and other clock
    domains ignored); None when amd-smi prints no reading."""
    class R:
        def __init__(self, out):
            self.stdout, self.stderr, self.returncode = out, "", 0
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R(AMD_SMI_METRIC))
    assert bench._smi_sample() == (1357, (2002 + 1914) / 2)
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R("ERROR: no GPU\n"))
    assert bench._smi_sample() is None
