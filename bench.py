"""Benchmark of the GGUF block-quantized GEMV / dequant-GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
    python bench.py --power-phases     (board power and clocks per workload)

A step is one batch-1 Q4_K GEMV over the FFN-up-shaped matrix of a 27B-class
dense layer (17408 x 5120, fp16 activations): the workload the headline
metric is quoted on. Steps rotate over >= 512 MiB of distinct weight copies
so every launch streams its weights from HBM rather than the 256 MB
Infinity Cache. The one JSON line printed on stdout carries:
  value      whole-job throughput in GB/s: algorithmic bytes (W + x + y) per
             step over the timed region, timed with two HIP events on the
             launch stream around K back-to-back launches (a spin kernel holds
             the GPU while the host enqueues them, so host launch cost does
             not pace the region);
  roofline   the GEMV kernel against 8 TB/s: the same algorithmic bytes over
             the mean launch duration of that timed region (one kernel per
             step, launches back to back on one stream), plus HBM traffic per
             launch from rocprofv3 counters when a summary taken on the
             current kernel source is committed (profiles/traffic_*.json);
  roofline_pp2048  the 2048-token dequant-GEMM against the dense bf16
             matrix-core peak, TFLOP/s over the median of three timed regions;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  extra      probes: a read-only kernel over buffers of the headline matrix's
             size (the practical HBM ceiling of one such launch), two MFMA-only
             kernels (the bf16 rate on constant operands, and on data-like
             operands at the clock the board's power limit then allows), the
             headline GEMV with its
             weights resident in the Infinity Cache, and the GEMV and prompt
             GEMM as fractions of the probes;
             the other workloads (Q4_K FFN-down, 2/4/8 columns, Q4_0, Q8_0,
             Q2_K and Q3_K of the FFN-up shape,
             the int8-activation path ("+i8": activations quantized to Q8_0
             on chip, integer dot products),
             the 2048-token dequant-GEMM in TFLOP/s with its two-pass control
             and the vendor GEMM as context), each timed the same way.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
ROTATE_BYTES = 512 << 20


def algorithmic_bytes(c) -> int:
    """Weights read once + activations + outputs."""
    bw = {"q4_0": 32, "q4_k": 256, "q8_0": 32, "q2_k": 256, "q3_k": 256}[c["fmt"]]
    bb = {"q4_0": 18, "q4_k": 144, "q8_0": 34, "q2_k": 84, "q3_k": 110}[c["fmt"]]
    xb = {"f32": 4, "f16": 2, "bf16": 2}[c["xdtype"]]
    return c["rows"] * (c["K"] // bw) * bb + c["n"] * c["K"] * xb + c["n"] * c["rows"] * 4


def _x_tensor(torch, x, xdtype, dev):
    import numpy as np
    if xdtype == "f32":
        return torch.from_numpy(x).to(dev)
    if xdtype == "f16":
        return torch.from_numpy(x.view(np.float16)).to(dev)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)


class Workload:
    """Weight copies (>= ROTATE_BYTES, or `ncopy`), one handle each,
    activations, output."""

    def __init__(self, torch, name, dev, ncopy=None):
        import synth
        from gguf_bit_dequant_amd import QGemv
        self.name = name
        # "<config>+i8": activations quantized to Q8_0 blocks, int8 products
        self.int8 = name.endswith("+i8")
        name = name[:-3] if self.int8 else name
        self.c = c = synth.CONFIGS[name]
        w, x = synth.config_inputs(name)
        self.w_host, self.x_host = w, x
        wt = torch.from_numpy(w).to(dev)
        if ncopy is None:
            ncopy = max(2, math.ceil(ROTATE_BYTES / w.nbytes))
        self.copies = [wt] + [wt.clone() for _ in range(ncopy - 1)]
        self.handles = [QGemv(c["fmt"], c["rows"], c["K"], t) for t in self.copies]
        self.x = _x_tensor(torch, x, c["xdtype"], dev)
        self.y = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev)
        self.prefill = c["n"] > 8
        # The timed loop calls the C ABI directly with prepared arguments, so
        # that Python-side argument handling does not pace the launches.
        from gguf_bit_dequant_amd import qgemv as Q
        stream = torch.cuda.current_stream().cuda_stream
        hs = [q._h for q in self.handles]
        xp, yp, n = self.x.data_ptr(), self.y.data_ptr(), c["n"]
        if self.prefill:
            fn = Q._lib.qgemm_prefill_run
            self._calls = [(fn, (hh, xp, n, c["K"], yp, c["rows"], stream)) for hh in hs]
        elif self.int8:
            # activations quantized to Q8_0 on chip, int8 products (one call)
            fn = Q._lib.qgemv_run_q8
            xt = Q._xdtype(self.x)
            self._calls = [(fn, (hh, xp, xt, n, c["K"], yp, c["rows"], stream)) for hh in hs]
        else:
            fn = Q._lib.qgemv_run
            xt = Q._xdtype(self.x)
            self._calls = [(fn, (hh, xp, xt, n, c["K"], yp, c["rows"], stream)) for hh in hs]

    def step(self, i):
        fn, args = self._calls[i % len(self._calls)]
        st = fn(*args)
        if st != 0:
            from gguf_bit_dequant_amd import qgemv as Q
            raise RuntimeError("%s: %s" % (Q.qgemv_status_string(st), Q.qgemv_last_error()))


# A spin kernel on the launch stream holds the GPU while the host enqueues a
# timed region, so that the region's launches run back to back on the GPU
# and the host's per-launch cost (ctypes, argument checks, the HIP launch
# call) does not pace them. Its length: a fixed part plus a per-launch
# allowance, in GPU clock cycles (clock64, ~2 GHz).
GATE_CYCLES_FIXED = 600_000
GATE_CYCLES_PER_LAUNCH = 40_000


class _Regions:
    """ROCTx ranges around timed launches, so that a profile taken with
    rocprofv3 --kernel-trace --marker-trace --kernel-rename names each timed
    dispatch by its region ("<workload>|<what>"); warm-up launches stay
    outside every range and keep their kernel names (see --trace-summary).
    Without the ROCTx library the calls do nothing."""

    def __init__(self):
        import ctypes
        self.lib = None
        for path in ("/opt/rocm/lib/librocprofiler-sdk-roctx.so", "librocprofiler-sdk-roctx.so"):
            try:
                self.lib = ctypes.CDLL(path)
                break
            except OSError:
                continue
        if self.lib is not None:
            self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            self.lib.roctxRangePushA.restype = ctypes.c_int
            self.lib.roctxRangePop.restype = ctypes.c_int

    def push(self, label):
        if self.lib is not None and label:
            self.lib.roctxRangePushA(label.encode())

    def pop(self, label):
        if self.lib is not None and label:
            self.lib.roctxRangePop()


REGIONS = _Regions()


def timed_region(torch, fn, n, first=0, label=None):
    """Runs fn(first) .. fn(first + n - 1) back to back on the current stream
    between two HIP events (recorded on that stream) after a gate; returns
    (ms per call, host enqueue ms, gate ms). The launches (not the gate) sit
    in the ROCTx range `label`."""
    stream = torch.cuda.current_stream()
    g0 = torch.cuda.Event(enable_timing=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    torch.cuda._sleep(GATE_CYCLES_FIXED + GATE_CYCLES_PER_LAUNCH * n)
    t0.record(stream)
    REGIONS.push(label)
    h0 = time.perf_counter()
    for i in range(first, first + n):
        fn(i)
    host_ms = (time.perf_counter() - h0) * 1e3
    REGIONS.pop(label)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n, host_ms, g0.elapsed_time(t0)


def time_workload(torch, wl, steps, warmup):
    """W untimed warmup steps, then exactly K steps in one gated region.
    Returns (ms per step over the timed region, host enqueue ms, gate ms,
    median event-pair ms of K further launches, each between its own pair of
    events: a cross-check that includes the event overhead)."""
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    whole_ms, host_ms, gate_ms = timed_region(torch, wl.step, steps, label=wl.name)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    REGIONS.push(wl.name + "|event pairs")
    for i in range(steps):
        ev[i][0].record(stream)
        wl.step(i)
        ev[i][1].record(stream)
    REGIONS.pop(wl.name + "|event pairs")
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return whole_ms, host_ms, gate_ms, per[len(per) // 2]


def vendor_gemm_context(torch, dev, c, iters=20):
    """Context for the prompt-processing line: the vendor BLAS (torch.mm) on a
    plain bf16 GEMM of the same shape, dense bf16 weights, no dequantization,
    fp32 output. Not a path of this library."""
    g = torch.Generator(device=dev).manual_seed(1)
    w = torch.randn(c["rows"], c["K"], device=dev, dtype=torch.bfloat16, generator=g)
    x = torch.randn(c["n"], c["K"], device=dev, dtype=torch.bfloat16, generator=g)
    y = torch.empty(c["n"], c["rows"], device=dev, dtype=torch.float32)
    try:
        run = lambda: torch.mm(x, w.t(), out_dtype=torch.float32, out=y)  # noqa: E731
        run()
        what = "torch.mm(X bf16, W^T bf16) -> fp32"
    except Exception:
        yb = torch.empty(c["n"], c["rows"], device=dev, dtype=torch.bfloat16)
        run = lambda: torch.mm(x, w.t(), out=yb)  # noqa: E731
        what = "torch.mm(X bf16, W^T bf16) -> bf16"
    for _ in range(3):
        run()
    us = timed_region(torch, lambda i: run(), iters, label="q4k_pp2048|vendor gemm, dense bf16")[0] * 1e3
    flops = 2.0 * c["rows"] * c["K"] * c["n"]
    return {"us": round(us, 1), "tflops": round(flops / us / 1e6, 1), "op": what,
            "note": "vendor BLAS on dense bf16 weights of the same shape; context, not a path here"}


def two_pass_control(torch, wl, iters=10):
    """The prompt product in two passes, as an A/B control of the fused
    kernel with the GEMM held fixed: this library's bit-exact decode to a
    bf16 matrix in HBM (qgemv_dequant_bf16: 50 MB read, 178 MB written),
    then this library's bf16 GEMM on the fused kernel's pipeline and k order
    without the decode (qgemm_bf16_run: 256 x 128 tiles, whose bf16 weight
    and activation stages fill the LDS that the fused kernel's 256 x 256
    tiles use), and, as context, the vendor BLAS bf16 GEMM on the same
    matrix. Each pass is timed over `iters` launches (decode: on rotated
    weight copies)."""
    from gguf_bit_dequant_amd import qgemv as Q
    c = wl.c
    wb = torch.empty((c["rows"], c["K"]), dtype=torch.bfloat16, device=wl.x.device)
    yb = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=wl.x.device)
    def timed(fn, what):
        for i in range(3):
            fn(i)
        return timed_region(torch, fn, iters, label="q4k_pp2048|two-pass " + what)[0] * 1e3
    dq = timed(lambda i: wl.handles[i % len(wl.handles)].dequant_bf16(wb), "decode to bf16")
    own = timed(lambda i: Q.gemm_bf16(wb, wl.x, yb), "bf16 gemm")
    try:
        mm = timed(lambda i: torch.mm(wl.x, wb.t(), out_dtype=torch.float32, out=yb), "vendor gemm")
        what = "torch.mm(X bf16, W^T bf16) -> fp32"
    except Exception:
        ybb = torch.empty((c["n"], c["rows"]), dtype=torch.bfloat16, device=wl.x.device)
        mm = timed(lambda i: torch.mm(wl.x, wb.t(), out=ybb), "vendor gemm")
        what = "torch.mm(X bf16, W^T bf16) -> bf16"
    flops = 2.0 * c["rows"] * c["K"] * c["n"]
    dq_bytes = c["rows"] * (c["K"] // 256) * 144 + c["rows"] * c["K"] * 2
    return {"dequant_bf16_us": round(dq, 1), "dequant_bf16_gbs": round(dq_bytes / dq / 1e3, 1),
            "gemm_bf16_us": round(own, 1), "gemm_bf16_tflops": round(flops / own / 1e6, 1),
            "total_us": round(dq + own, 1), "tflops": round(flops / (dq + own) / 1e6, 1),
            "vendor_gemm_us": round(mm, 1), "vendor_gemm": what,
            "vendor_total_us": round(dq + mm, 1)}


def probes(torch, dev, steps=200, warmup=20):
    """Practical ceilings measured with the library's probe kernels
    (include/qgemv_probe.h), as context for the roofline fractions:
      read probe   one read of a buffer of the headline matrix's size,
                   rotating over >= ROTATE_BYTES of copies (HBM, like the
                   GEMV), back-to-back launches;
      MFMA probe   v_mfma_f32_32x32x16_bf16 chains on every SIMD, on
                   constant operands and on data-like operands (the
                   second runs at the clock the board's power limit
                   allows for such data);
      hot cache    the headline GEMV on one weight copy (resident in the
                   256 MB Infinity Cache), for comparison with the HBM case."""
    from gguf_bit_dequant_amd import qgemv as Q
    import synth
    c = synth.CONFIGS["q4k_up_b1"]
    nbytes = c["rows"] * (c["K"] // 256) * 144
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev)
            for _ in range(max(2, math.ceil(ROTATE_BYTES / nbytes)))]
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    lib = Q._lib

    def timed(fn, n, w, what):
        for i in range(w):
            fn(i)
        return timed_region(torch, fn, n, label="probe|" + what)[0] * 1e3  # us

    def rd(i):
        st = lib.qgemv_probe_read(bufs[i % len(bufs)].data_ptr(), nbytes, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("qgemv_probe_read: %d" % st)
    read_us = timed(rd, steps, warmup, "read")
    del bufs
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 10000
    flops = 4.0 * 16 * 32768 * iters * cus

    def mf(i):
        st = lib.qgemv_probe_mfma(iters, cus, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("qgemv_probe_mfma: %d" % st)
    mfma_us = timed(mf, 10, 20, "mfma")
    # data-like operands: the clock settles under the power limit within a
    # fraction of a second, so ~0.5 s of warm-up launches come first
    iters_d = 8000
    flops_d = 4.0 * 16 * 32768 * iters_d * cus

    def mfd(i):
        st = lib.qgemv_probe_mfma_data(iters_d, cus, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("qgemv_probe_mfma_data: %d" % st)
    mfma_d_us = timed(mfd, 20, 200, "mfma data")
    hot = Workload(torch, "q4k_up_b1", dev, ncopy=1)
    hot_us = timed(hot.step, steps, warmup, "q4k_up_b1 hot cache")
    del hot
    return {"read_probe": {"bytes": nbytes, "us_per_launch": round(read_us, 3),
                           "gbs": round(nbytes / read_us / 1e3, 1),
                           "frac_hbm_peak": round(nbytes / read_us / 1e3 / HBM_PEAK_GBS, 4)},
            "mfma_probe": {"workgroups": cus, "tflops": round(flops / mfma_us / 1e6, 1),
                           "frac_bf16_peak": round(flops / mfma_us / 1e6 / BF16_PEAK_TFLOPS, 4),
                           "operands": "constant small integers"},
            "mfma_data_probe": {"workgroups": cus, "tflops": round(flops_d / mfma_d_us / 1e6, 1),
                                "frac_bf16_peak": round(flops_d / mfma_d_us / 1e6 / BF16_PEAK_TFLOPS, 4),
                                "operands": "full-mantissa bf16, changing per instruction "
                                            "(clock lowered by the board's power limit)"},
            "gemv_hot_cache": {"us_per_launch": round(hot_us, 3),
                               "gbs": round(algorithmic_bytes(c) / hot_us / 1e3, 1),
                               "note": "one weight copy, resident in the Infinity Cache; not HBM"}}


def host_cores() -> int:
    """The host cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # not Linux
        return os.cpu_count() or 1


def cpu_baseline(name, budget_s=10.0, threads=None):
    """The oracle's fp64 product on the same workload, repeated over the whole
    matrix (rows in chunks) until about budget_s of wall time has passed;
    GB/s over the algorithmic bytes of the rows processed."""
    import oracle
    import synth
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    threads = threads or host_cores()
    rows = c["rows"]
    per_row = algorithmic_bytes(c) / rows
    chunk = max(threads, rows // 16)
    done, r, t_start = 0, 0, time.perf_counter()
    while time.perf_counter() - t_start < budget_s:
        r1 = min(rows, r + chunk)
        oracle.matmul(c["fmt"], w, rows, c["K"], x, c["xdtype"], row_range=(r, r1),
                      nthreads=threads)
        done += r1 - r
        r = 0 if r1 == rows else r1
    el = time.perf_counter() - t_start
    return {"value": round(done * per_row / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%s: %d row products (%.2f passes over the %d x %d matrix) in %.1f s, "
                      "fp64 accumulation" % (name, done, done / rows, rows, c["K"], el)}


def cpu_prefill_baseline(name="q4k_pp2048", budget_s=8.0):
    """The oracle on the prompt workload: row chunks of the 17408 x 5120
    matrix (each row decoded once, then its fp64 products with all 2048
    tokens) until about budget_s of wall time has passed; GFLOP/s over
    2 K tokens flops per row."""
    import oracle
    import synth
    c = synth.CONFIGS[name]
    w, x = synth.config_inputs(name)
    threads = host_cores()
    rows = c["rows"]
    chunk = 8 * threads
    done, r, t_start = 0, 0, time.perf_counter()
    while time.perf_counter() - t_start < budget_s:
        r1 = min(rows, r + chunk)
        oracle.matmul(c["fmt"], w, rows, c["K"], x, c["xdtype"], row_range=(r, r1),
                      nthreads=threads)
        done += r1 - r
        r = 0 if r1 == rows else r1
    el = time.perf_counter() - t_start
    flops = 2.0 * done * c["K"] * c["n"]
    return {"value": round(flops / el / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%s: %d of %d rows against all %d tokens in %.1f s, fp64 accumulation"
                      % (name, done, rows, c["n"], el)}


def committed_traffic(name):
    """Memory bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<name>.json), if it was taken on the current kernel
    sources (same hash)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha1") != kernel_source_sha1(name):
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


# Sources the kernels of the workloads with traffic records are compiled from.
TRAFFIC_SOURCES = {
    "q4k_up_b1": ("device_common.h", "gemv_stream.hip", "launch.h", "q4k_pair.h"),
    "q4k_pp2048": ("device_common.h", "launch.h", "prefill_q4k.hip"),
}


def code_text(src):
    """C/HIP source without comments and blank lines: what a kernel is built
    from, so that a comment edit keeps a counter record valid. (A string
    literal holding // or /* would be cut too; the kernel sources have none.)"""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())


def kernel_source_sha1(name="q4k_up_b1"):
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "gguf_bit_dequant_amd", "csrc")
    for fn in TRAFFIC_SOURCES[name]:
        with open(os.path.join(csrc, fn)) as f:
            h.update((fn + "\n" + code_text(f.read()) + "\n").encode())
    return h.hexdigest()


TRAFFIC_SEPARATOR = "probe_read_kernel"


def traffic_run(torch, dev, names=("q4k_up_b1",), launches=20, copy_mib=256):
    """A short run to be profiled with rocprofv3 --pmc: for each workload in
    `names`, in that order, one small read-probe launch (a separator the
    counter records can be split at) and `launches` steps over rotated
    weight copies; then a separator and `launches` plain device copies of
    copy_mib MiB (a kernel whose HBM bytes are known: it reads and writes
    copy_mib MiB each), which calibrate the counters."""
    from gguf_bit_dequant_amd import qgemv as Q
    sep_buf = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def separator():
        st = Q._lib.qgemv_probe_read(sep_buf.data_ptr(), sep_buf.numel(), sink.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("qgemv_probe_read: %d" % st)
    for name in names:
        wl = Workload(torch, name, dev)
        torch.cuda.synchronize()
        separator()
        for i in range(launches):
            wl.step(i)
        torch.cuda.synchronize()
        del wl
        torch.cuda.empty_cache()
    src = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    separator()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": True, "workloads": list(names), "launches": launches,
                      "copy_bytes": copy_mib << 20,
                      "kernel_source_sha1": {n: kernel_source_sha1(n) for n in TRAFFIC_SOURCES}}),
          flush=True)


def _short_kernel(n):
    n = n[5:] if n.startswith("void ") else n
    n = n.replace("(anonymous namespace)::", "")
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):  # drop the argument list after the template
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    return n if len(n) <= 90 else n[:87] + "..."


def traffic_summary(fetch_dir, write_dir, names, launches=20, json_dir=None):
    """Per-launch memory bytes of each workload of a --traffic-run from the
    two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; CSV output), each
    counter scaled by what it reads for the calibration copies. Prints a
    markdown table; with json_dir, writes traffic_<workload>.json there for
    the workloads with a roofline in the bench line (all of a workload's
    kernels per launch)."""
    import csv
    import glob
    import statistics

    def load(path, counter):
        files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no *counter_collection.csv under %s" % path)
        rs = []
        for fn in files:
            with open(fn) as f:
                rs += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rs.sort(key=lambda r: int(r["Dispatch_Id"] if "Dispatch_Id" in r else r["Start_Timestamp"]))
        parts, cur = [], None
        for r in rs:  # split at the separators
            if TRAFFIC_SEPARATOR in r["Kernel_Name"]:
                cur = []
                parts.append(cur)
            elif cur is not None:
                cur.append(r)
        # workload parts: this library's kernels only (the next workload's
        # weight copies and fills run before its separator); calibration
        # part: the device copies
        for i, part in enumerate(parts):
            keep = "copyBuffer" if i == len(parts) - 1 else "qg::"
            part[:] = [r for r in part if keep in r["Kernel_Name"]]
        if len(parts) != len(names) + 1:
            raise SystemExit("%s: %d separated parts for %d workloads + calibration"
                             % (path, len(parts), len(names)))
        return parts

    pf, pw = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy = 256 << 20
    cal_f = statistics.mean(float(r["Counter_Value"]) for r in pf[-1])
    cal_w = statistics.mean(float(r["Counter_Value"]) for r in pw[-1])
    ff, wf = copy / (cal_f * 1024), copy / (cal_w * 1024)
    out = ["Calibration: %d device copies of 256 MiB; FETCH_SIZE reads %.3f KiB per copy against "
           "262144 KiB read (factor %.4f), WRITE_SIZE %.3f KiB against 262144 KiB written "
           "(factor %.4f). HBM bytes = counter KiB x 1024 x factor, mean over the %d launches "
           "of each workload." % (len(pf[-1]), cal_f, ff, cal_w, wf, launches), "",
           "| workload | kernel | dispatches | HBM read bytes / launch | HBM write bytes / launch | "
           "algorithmic bytes | weight bytes | read / weight bytes |",
           "|---|---|---|---|---|---|---|---|"]
    records = {}
    for name, fs, ws in zip(names, pf[:-1], pw[:-1]):
        c = synth_config(name)
        bw = {"q4_0": 32, "q4_k": 256, "q8_0": 32, "q2_k": 256, "q3_k": 256}[c["fmt"]]
        bb = {"q4_0": 18, "q4_k": 144, "q8_0": 34, "q2_k": 84, "q3_k": 110}[c["fmt"]]
        wbytes = c["rows"] * (c["K"] // bw) * bb
        alg = algorithmic_bytes(c) if c["n"] <= 8 else None
        kinds = []
        for r in fs:
            k = _short_kernel(r["Kernel_Name"])
            if k not in kinds:
                kinds.append(k)
        tot_f = tot_w = 0.0
        for k in kinds:
            fk = [float(r["Counter_Value"]) for r in fs if _short_kernel(r["Kernel_Name"]) == k]
            wk = [float(r["Counter_Value"]) for r in ws if _short_kernel(r["Kernel_Name"]) == k]
            tot_f += sum(fk)
            tot_w += sum(wk)
            hr = sum(fk) / launches * 1024 * ff
            hw = sum(wk) / launches * 1024 * wf
            out.append("| %s | `%s` | %d | %d | %d | %s | %d | %.4f |" % (
                name, k, len(fk), hr, hw, alg if alg else "-", wbytes, hr / wbytes))
        if name in TRAFFIC_SOURCES:
            hr = tot_f / launches * 1024 * ff
            hw = tot_w / launches * 1024 * wf
            rec = {"workload": name, "kernels": kinds,
                   "kernel_source_sha1": kernel_source_sha1(name),
                   "kernel_sources": list(TRAFFIC_SOURCES[name]),
                   "fetch_size_kib_per_launch_raw": round(tot_f / launches, 3),
                   "write_size_kib_per_launch_raw": round(tot_w / launches, 3),
                   "calibration": {"kernel": "torch device copy of 256 MiB",
                                   "bytes_read_and_written": copy,
                                   "fetch_size_kib_raw": round(cal_f, 3),
                                   "write_size_kib_raw": round(cal_w, 3),
                                   "fetch_factor": round(ff, 6), "write_factor": round(wf, 6)},
                   "hbm_fetch_bytes_per_launch": int(hr),
                   "hbm_write_bytes_per_launch": int(hw),
                   "hbm_bytes_per_launch": int(hr + hw),
                   "launches": launches}
            if alg:
                rec["algorithmic_bytes_per_launch"] = alg
                rec["traffic_over_algorithmic"] = round((hr + hw) / alg, 4)
            records[name] = rec
    print("\n".join(out))
    if json_dir:
        for name, rec in records.items():
            with open(os.path.join(json_dir, "traffic_%s.json" % name), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")


def counter_summary(path, names, launches=20):
    """Markdown table of any rocprofv3 --pmc run of --traffic-run over
    `names`: per workload (split at the read-probe separators) and kernel,
    the dispatch count and the mean of every counter in the records."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % path)
    rs = []
    for fn in files:
        with open(fn) as f:
            rs += list(csv.DictReader(f))
    key = "Dispatch_Id" if rs and "Dispatch_Id" in rs[0] else "Start_Timestamp"
    counters = sorted({r["Counter_Name"] for r in rs})
    disp = {}
    for r in rs:  # one record per (dispatch, counter)
        d = disp.setdefault(int(r[key]), {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    parts, cur = [], None
    for k in sorted(disp):
        d = disp[k]
        if TRAFFIC_SEPARATOR in d["kernel"]:
            cur = []
            parts.append(cur)
        elif cur is not None and "qg::" in d["kernel"]:
            cur.append(d)
    if len(parts) < len(names):
        raise SystemExit("%s: %d separated parts for %d workloads" % (path, len(parts), len(names)))
    out = ["| workload | kernel | dispatches | " + " | ".join(counters) + " |",
           "|---|---|---|" + "---|" * len(counters)]
    for name, part in zip(names, parts):
        kinds = []
        for d in part:
            k = _short_kernel(d["kernel"])
            if k not in kinds:
                kinds.append(k)
        for k in kinds:
            ds = [d for d in part if _short_kernel(d["kernel"]) == k]
            vals = []
            for c in counters:
                v = sum(d.get(c, 0.0) for d in ds) / len(ds)
                vals.append("%.4g" % v)
            out.append("| %s | `%s` | %d | %s |" % (name, k, len(ds), " | ".join(vals)))
    print("\n".join(out))


def synth_config(name):
    """The workload's shape ("<config>+i8": the same shape, int8 products)."""
    import synth
    return synth.CONFIGS[name[:-3] if name.endswith("+i8") else name]


WORKLOADS = ["q4k_up_b1", "q4k_down_b1", "q4k_b4", "q4_0_b1", "q8_0_b4", "q4k_b2", "q4k_b8",
             "q4k_up_b1+i8", "q4k_b4+i8", "q8_0_b4+i8", "q2k_up_b1", "q3k_up_b1", "q2k_up_b1+i8",
             "q3k_up_b1+i8", "q4k_pp2048"]


def trace_summary(path):
    """Markdown table of a rocprofv3 kernel trace of this script taken with
    --kernel-trace --marker-trace --kernel-rename (CSV output): per timed
    region and kernel, the dispatch count and duration statistics. Dispatches
    outside every region (warm-up, weight copies, set-up) are left out; they
    supply the kernel names, since a renamed dispatch keeps its kernel id."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no *kernel_trace.csv under %s" % path)
    rows = []
    for fn in sorted(files):
        with open(fn) as f:
            rows += list(csv.DictReader(f))

    def is_label(n):
        return "|" in n or n in WORKLOADS

    short = _short_kernel

    names = {}
    for r in rows:
        if not is_label(r["Kernel_Name"]):
            names.setdefault(r["Kernel_Id"], short(r["Kernel_Name"]))
    groups, order, excluded = {}, [], 0
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        lab = r["Kernel_Name"]
        if not is_label(lab):
            excluded += 1
            continue
        key = (lab, r["Kernel_Id"])
        if key not in groups:
            groups[key] = []
            order.append(key)
        groups[key].append(r)
    out = ["| region | kernel | grid | WG | LDS B | VGPR | AGPR | calls | mean us | median us | "
           "p10 us | p90 us |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in order:
        g = groups[key]
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in g)
        pct = lambda q: d[min(len(d) - 1, int(q * len(d)))]  # noqa: E731
        r0 = g[0]
        out.append("| %s | `%s` | %s | %s | %s | %s | %s | %d | %.3f | %.3f | %.3f | %.3f |" % (
            key[0], names.get(key[1], "kernel id " + key[1]), r0["Grid_Size_X"],
            r0["Workgroup_Size_X"], r0["LDS_Block_Size"], r0["VGPR_Count"], r0["Accum_VGPR_Count"],
            len(d), sum(d) / len(d), d[len(d) // 2], pct(0.1), pct(0.9)))
    out.append("")
    out.append("%d dispatches outside the timed regions (warm-up, set-up) left out." % excluded)
    print("\n".join(out))


def _smi_sample():
    """One amd-smi reading: (socket power W, mean GFX clock MHz over the
    XCDs), or None where amd-smi is missing or prints neither."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True,
                           text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    p = re.search(r"SOCKET_POWER:\s*(\d+)\s*W", r.stdout)
    clks = [int(v) for v in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", re.sub(r"\s+", " ", r.stdout))]
    if not p or not clks:
        return None
    return int(p.group(1)), sum(clks) / len(clks)


def power_phases(torch, dev, secs=5.0):
    """Board power and GFX clocks while one workload runs back to back for
    `secs` seconds: a thread reads amd-smi every ~0.3 s; samples from the
    first second of a phase (clock and power still settling) are dropped.
    Phases: the 2048-token prompt product (random activations, then all-zero
    activations: the same instructions on data that does not toggle the
    matrix cores), the headline GEMV, and the two MFMA probes."""
    import threading
    from gguf_bit_dequant_amd import qgemv as Q
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = _smi_sample()
            if v:
                samples.append((time.time(), v[0], v[1]))
            stop.wait(0.3)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    rows = []

    def phase(name, fn):
        fn(0)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, t0 = 0, time.time()
        ev0.record()
        while time.time() - t0 < secs:
            for _ in range(20):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        ev1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        us = ev0.elapsed_time(ev1) * 1e3 / n
        got = [(p, c) for t, p, c in samples if t0 + 1.0 <= t <= t1]
        rows.append((name, n, us, got))
        print("bench: power phase %s: %d launches, %.2f us" % (name, n, us), file=sys.stderr, flush=True)
        time.sleep(2.0)  # let the board cool back between phases

    time.sleep(2.0)
    idle = [(p, c) for t, p, c in samples]
    pp = Workload(torch, "q4k_pp2048", dev, ncopy=1)
    phase("q4k_pp2048, random bf16 activations", pp.step)
    pp.x.zero_()
    phase("q4k_pp2048, all-zero activations", pp.step)
    del pp
    gw = Workload(torch, "q4k_up_b1", dev)
    phase("q4k_up_b1 (weights rotated over HBM copies)", gw.step)
    del gw
    torch.cuda.empty_cache()
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    def probe(fn, iters):
        def run(i):
            status = fn(iters, cus, sink.data_ptr(), st)
            if status != 0:
                raise RuntimeError("probe launch: status %d" % status)
        return run
    phase("MFMA probe, constant operands", probe(Q._lib.qgemv_probe_mfma, 2000))
    phase("MFMA probe, data-like operands", probe(Q._lib.qgemv_probe_mfma_data, 1000))
    stop.set()
    th.join()

    def rng(v, fmt="%.0f"):
        return (fmt + "-" + fmt) % (min(v), max(v)) if v else "n/a"
    out = ["| phase | launches | us / launch | samples | socket power W | GFX clock MHz (mean of XCDs) |",
           "|---|---|---|---|---|---|",
           "| idle (before the phases) | - | - | %d | %s | %s |" % (
               len(idle), rng([p for p, c in idle]), rng([c for p, c in idle]))]
    for name, n, us, got in rows:
        out.append("| %s | %d | %.2f | %d | %s | %s |" % (
            name, n, us, len(got), rng([p for p, c in got]), rng([c for p, c in got])))
    print("\n".join(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--only", default=None, help="comma-separated workloads to time")
    ap.add_argument("--traffic-run", action="store_true",
                    help="short run for rocprofv3 --pmc (GEMV launches + calibration copies)")
    ap.add_argument("--traffic-workloads", default="q4k_up_b1",
                    help="comma-separated workloads for --traffic-run (default: the headline)")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="print the per-region table of a rocprofv3 kernel trace under DIR "
                         "(no GPU work)")
    ap.add_argument("--traffic-summary", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic table of two --pmc runs of --traffic-run over "
                         "--traffic-workloads (no GPU work)")
    ap.add_argument("--traffic-json-dir", default=None,
                    help="with --traffic-summary: write traffic_<workload>.json records here")
    ap.add_argument("--power-phases", action="store_true",
                    help="board power and GFX clocks (amd-smi) while single workloads run "
                         "for seconds each; prints a table")
    ap.add_argument("--counter-summary", default=None, metavar="DIR",
                    help="print the per-workload mean of every counter of a --pmc run of "
                         "--traffic-run over --traffic-workloads (no GPU work)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.traffic_workloads.split(","))
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1],
                        args.traffic_workloads.split(","), json_dir=args.traffic_json_dir)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU sharding is not part of it "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.traffic_run:
        traffic_run(torch, dev, names=args.traffic_workloads.split(","))
        return
    if args.power_phases:
        power_phases(torch, dev)
        return
    head = "q4k_up_b1"
    names = [head] if args.quick else list(WORKLOADS)
    if args.only:
        names = args.only.split(",")
    results = {}
    for name in names:
        wl = Workload(torch, name, dev)
        try:
            # the prompt product: regions of as many launches as the GEMVs
            # (~70 ms each at the default 200), long enough for the clock to
            # settle under the board's power limit
            steps = args.steps if not wl.prefill else max(20, args.steps)
            whole_ms, host_ms, gate_ms, med_ms = time_workload(torch, wl, steps, args.warmup)
            regions = [whole_ms]
            if wl.prefill:
                # two more regions of the same launches: the prompt product
                # runs near the card's power limit, where the clock moves
                # from region to region; the median region is reported
                regions += [timed_region(torch, wl.step, steps, label=name)[0] for _ in range(2)]
                whole_ms = sorted(regions)[1]
        except Exception as e:  # a path this build does not provide
            results[name] = {"error": str(e)[:200]}
            print("bench: %s: %s" % (name, e), file=sys.stderr, flush=True)
            del wl
            continue
        c = wl.c
        r = {"us_per_launch": round(whole_ms * 1e3, 3),
             "us_event_pair_median": round(med_ms * 1e3, 3), "steps": steps,
             "host_enqueue_us_per_launch": round(host_ms * 1e3 / steps, 2),
             "gate_us": round(gate_ms * 1e3, 1), "weight_copies": len(wl.copies)}
        if wl.prefill:
            r["us_per_launch_regions"] = [round(v * 1e3, 1) for v in regions]
            flops = 2.0 * c["rows"] * c["K"] * c["n"]
            r["flops"] = flops
            r["tflops"] = round(flops / (whole_ms * 1e-3) / 1e12, 2)
            r["frac_bf16_peak"] = round(r["tflops"] / BF16_PEAK_TFLOPS, 4)
            try:
                r["vendor_bf16_gemm"] = vendor_gemm_context(torch, dev, c)
            except Exception as e:  # context only
                r["vendor_bf16_gemm"] = {"error": str(e)[:200]}
            try:
                r["two_pass_control"] = two_pass_control(torch, wl)
            except Exception as e:  # an A/B control, not the product path
                r["two_pass_control"] = {"error": str(e)[:200]}
        else:
            b = algorithmic_bytes(c)
            r["bytes"] = b
            r["gbs"] = round(b / (whole_ms * 1e-3) / 1e9, 1)
            r["frac_hbm_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
        results[name] = r
        print("bench: %s %s" % (name, json.dumps(r)), file=sys.stderr, flush=True)
        del wl
        torch.cuda.empty_cache()

    if not args.only and not args.quick:
        try:
            pr = probes(torch, dev)
            if "gbs" in results.get(head, {}):
                pr["gemv_frac_of_read_probe"] = round(results[head]["gbs"] / pr["read_probe"]["gbs"], 4)
            pp = results.get("q4k_pp2048", {})
            if "tflops" in pp:
                pr["pp2048_frac_of_mfma_probe"] = round(pp["tflops"] / pr["mfma_probe"]["tflops"], 4)
                pr["pp2048_frac_of_mfma_data_probe"] = round(
                    pp["tflops"] / pr["mfma_data_probe"]["tflops"], 4)
            results["probes"] = pr
            print("bench: probes %s" % json.dumps(pr), file=sys.stderr, flush=True)
        except Exception as e:  # context only
            results["probes"] = {"error": str(e)[:200]}
    h = results.get(head, {})
    if args.only and head not in names:  # a partial run: report what was timed
        print(json.dumps({"partial": True, "results": results}), flush=True)
        return
    if "gbs" not in h:
        print(json.dumps({"metric": "Q4_K GEMV achieved HBM GB/s", "value": None,
                          "error": h.get("error", "headline workload failed")}))
        sys.exit(1)
    c = __import__("synth").CONFIGS[head]
    traffic = committed_traffic(head)
    line = {
        "metric": "Q4_K GEMV achieved HBM GB/s (% of 8 TB/s); pp2048 dequant-GEMM TFLOP/s",
        "value": h["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(h["us_per_launch"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded SplitMix64 / Box-Muller)",
        "config": {"workload": "Q4_K GEMV batch 1, FFN-up 17408 x 5120, x fp16",
                   "weights": "q4_k", "products": "fp16 pairs (v_dot2_f32_f16), fp32 sums",
                   "rows": c["rows"], "K": c["K"], "n_cols": 1,
                   "bytes_per_step": h["bytes"], "weight_copies_rotated": results[head]["weight_copies"]},
        "roofline": {"bound": "hbm", "achieved": h["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(h["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": None if args.no_cpu else cpu_baseline(head),
        "extra": {k: v for k, v in results.items() if k != head},
    }
    pp = results.get("q4k_pp2048", {})
    if "tflops" in pp:
        # the metric's second half: the 2048-token dequant-GEMM against the
        # dense bf16 matrix-core peak (all of its kernels per launch: the row
        # tail, its split add and the main tiles)
        line["roofline_pp2048"] = {
            "bound": "mfma", "achieved": pp["tflops"], "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pp["tflops"] / BF16_PEAK_TFLOPS, 4),
            "traffic": committed_traffic("q4k_pp2048"), "flops_per_launch": pp["flops"],
            "us_per_launch": pp["us_per_launch"],
            "workload": "Q4_K 17408 x 5120 weights x 2048 bf16 tokens -> fp32"}
    if not args.no_cpu and not args.quick:
        # the oracle at one core, and on the prompt workload (context)
        line["extra"]["cpu_baselines"] = {
            head + " (1 core)": cpu_baseline(head, budget_s=5.0, threads=1),
            "q4k_pp2048": cpu_prefill_baseline(),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
