#!/usr/bin/env python3
"""Benchmark of the quantized matvec hot path on one MI355X.

Default workload: the fused greedy output head -- 4-bit group-64 affine
matrix-vector product of the 151936x2048 tied output matrix at batch 1,
returning the float32 logits and the argmax index (one step = one call).
It is the headline weight-bandwidth workload: the only matrix-vector
product large enough (175 MB) to get past launch and ramp latency. Weights are cache-cold: every step reads a different copy, from
a rotation of distinct copies that together exceed 512 MiB, so each read
comes from HBM rather than from the L2 or the 256 MB Infinity Cache.

Reported (one JSON line):
  value          effective weight GB/s = weight bytes read per step / step time
  roofline       the dominant call's algorithmic bytes (or FLOPs) over its
                 time per call, vs the 8 TB/s HBM peak (2.5 PFLOP/s bf16 for
                 the prefill product): for a step of one call, the timed
                 region's step time itself; `traffic` from rocprofv3 counters
                 and `trace` (median, p10, p90 of the kernel's duration) from
                 the committed profiles when they were taken from the current
                 kernel sources
  read_ceiling   the best cold streaming read of the same byte count by the
                 measurement-only read kernels, and the call's rate as a
                 percentage of it
  gpu_state      clocks, temperatures and power before and after the timed
                 region (the amdgpu kernel module's hwmon and pp_dpm files)
  cpu_baseline   the CPU oracle on the same workload, on all of this host's
                 threads and on one (with the CPU model)

Other workloads (--workload): any case name of gemm_qgemv_amd.synth.CASES, or
a config prefix (c0, c1, c2b1, c2b8, c3, c4gemv, c4gemm), or one of the extensions
(u4gemm, head16, head64, head128, embed, i8g, i8ggemm). GEMM workloads report TFLOP/s; the
embedding gather reports the GB/s of its ids, packed rows and float32 rows.

The timed region replays one HIP graph holding all the timed steps (captured
once) so that the host's launch cost does not pace the GPU; inputs are
resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MATRIX_PEAK_TFLOPS = 157.3
BF16_MATRIX_PEAK_TFLOPS = 2500.0
# bytes of weights per decoded token implied by the pages' measurements
# (effective GB/s divided by tok/s): 8-bit 0.8B backbone (either scale
# layout), 4-bit 2B model, 1-bit 27B model
BYTES_PER_TOKEN = {1: 0.99e9, 2: 1.10e9, 3: 3.9e9, 4: 0.99e9}

WORKLOADS = {
    "c0": ["c0_i8_gemv_1024x1024"],
    "c1": ["c1a_u4_gemv_6144x2048", "c1b_u4_gemv_2048x6144"],
    "c2b1": ["c2_u4_head_151936x2048_b1"],
    "c2b8": ["c2_u4_head_151936x2048_b8"],
    "c3": ["c3a_i8_gemm_3584x1024_n2048", "c3b_i8_gemm_1024x3584_n2048",
           "c3c_i8_gemm_3584x1024_n10240", "c3d_i8_gemm_1024x3584_n10240"],
    "c4gemv": ["c4a_b1_gemv_17408x5120", "c4b_b1_gemv_5120x17408"],
    "c4gemm": ["c4c_b1_gemm_17408x5120_n512", "c4d_b1_gemm_5120x17408_n512"],
    "u4gemm": ["n2a_u4_gemm_6144x2048_n2048", "n2b_u4_gemm_2048x6144_n2048"],
    "head64": ["n1a_u4_head_151936x2048_b64", "n1b_u4_head_151936x2048_b64_nologits"],
    "head128": ["n1c_u4_head_151936x2048_b128", "n1d_u4_head_151936x2048_b128_nologits"],
    "embed": ["n3_u4_embed_151936x2048_t2048"],
    "head16": ["n4_u4_head_151936x2048_b16"],
    "i8g": ["n2c_i8g_gemv_3584x1024", "n2d_i8g_gemv_1024x3584"],
    "i8ggemm": ["n2e_i8g_gemm_3584x1024_n2048", "n2f_i8g_gemm_1024x3584_n2048"],
}
METRIC = "effective weight GB/s and % of HBM peak, batch-1 qgemv; prefill qgemm TFLOP/s"
EMBED_METRIC = "embedding gather GB/s (ids + packed rows read + float32 rows written)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 (16 hex digits) of the sources libqg.so is built from."""
    h = hashlib.sha256()
    for p in sorted(q for q in glob.glob(os.path.join(ROOT, "gemm_qgemv_amd", "csrc", "*"))
                    if not q.endswith("probe.hip")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Launch:
    """One case on the device: rotated weight copies, x, y, workspace, and a
    launcher that calls the C ABI with pre-resolved pointers."""

    def __init__(self, case, rotate_bytes, torch, q, synth, tensors):
        self.case = case
        w, x = synth.case_inputs(case)     # x: token ids for "embed"
        base = tensors.to_device(w)
        self.copies = max(1, math.ceil(rotate_bytes / w.nbytes)) if case.op != "gemm" else 1
        self.weights = [base] + [
            tensors.DeviceWeights(base.fmt, base.M, base.K, base.codes.clone(), base.scales.clone(),
                                  None if base.biases is None else base.biases.clone())
            for _ in range(self.copies - 1)]
        self.x = torch.from_numpy(x).cuda()
        out_cols = case.K if case.op == "embed" else case.M
        self.y = torch.empty(case.rows * out_cols, dtype=torch.float32, device="cuda")
        op = {"gemv": q.QG_OP_GEMV, "gemv_argmax": q.QG_OP_GEMV_ARGMAX, "greedy": q.QG_OP_GEMV_ARGMAX,
              "gemm": q.QG_OP_GEMM, "embed": None}[case.op]
        self.ws = None if op is None else tensors.workspace(op, case.fmt, case.M, case.K, case.rows)
        self.ws_bytes = 0 if self.ws is None else self.ws.numel()
        self.idx = torch.empty(case.rows, dtype=torch.int32, device="cuda")
        self.lib = q._binding.lib()
        self.ptrs = [(wd.codes.data_ptr(), wd.scales.data_ptr(),
                      None if wd.biases is None else wd.biases.data_ptr()) for wd in self.weights]
        self.host_w, self.host_x = w, x

    def __call__(self, i, stream):
        c, s, b = self.ptrs[i % self.copies]
        L, case = self.lib, self.case
        ws = None if self.ws is None else self.ws.data_ptr()
        if case.op == "gemv":
            st = L.qgemv(case.fmt, c, s, b, self.x.data_ptr(), self.y.data_ptr(), case.M, case.K,
                         case.rows, ws, self.ws_bytes, stream)
        elif case.op in ("gemv_argmax", "greedy"):
            y = self.y.data_ptr() if case.op == "gemv_argmax" else None
            st = L.qgemv_argmax(case.fmt, c, s, b, self.x.data_ptr(), y,
                                self.idx.data_ptr(), case.M, case.K, case.rows, ws,
                                self.ws_bytes, stream)
        elif case.op == "embed":
            st = L.qembed(case.fmt, c, s, b, self.x.data_ptr(), self.y.data_ptr(), case.M, case.K,
                          case.rows, stream)
        else:
            st = L.qgemm(case.fmt, c, s, b, self.x.data_ptr(), self.y.data_ptr(), case.M, case.K,
                         case.rows, ws, self.ws_bytes, stream)
        if st != 0:
            raise RuntimeError(f"{case.name}: status {st}")

    @property
    def weight_bytes(self):
        """Algorithmic bytes of one call: the packed weights a product reads
        once; for the gather, the ids, the packed rows of those ids (codes,
        scales, biases) and the float32 rows written."""
        c = self.case
        if c.op == "embed":
            row = c.weight_bytes // c.M
            return c.rows * (4 + row + 4 * c.K)
        return c.weight_bytes


def per_launch_ms(torch, fn, stream, n, reps=5):
    """Average time per call of `fn` when it runs alone: one HIP graph of
    n * reps back-to-back calls (rotating over n weight copies), replayed
    once between two HIP events on the stream the kernels run on (the same
    method as the timed region; it includes the short gaps between
    consecutive kernels of the graph)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n * reps):
            fn(i, stream.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(launches, seconds):
    """The oracle as it stands, on a bounded sample of the step: timed once
    with all the threads OpenMP gives it and once on one thread, each for
    about `seconds` / 2. `value` is the all-threads rate."""
    import oracle
    orc = oracle.get()
    all_threads = orc.num_threads()
    gemm = launches[0].case.op == "gemm"

    def run(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for L in launches:
                w, x = L.host_w, L.host_x
                c = L.case
                if c.op == "gemm":
                    # bounded sample: the first 8 token rows
                    orc.qgemv(c.fmt, w.codes, w.scales, w.biases, x[:8], c.M, c.K)
                elif c.op == "embed":
                    orc.embed(w.codes, w.scales, w.biases, x, c.M, c.K)
                else:
                    orc.qgemv(c.fmt, w.codes, w.scales, w.biases, x, c.M, c.K)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    def rate(reps, el):
        if gemm:
            return sum(2 * L.case.M * L.case.K * 8 for L in launches) * reps / el / 1e12
        return sum(L.weight_bytes for L in launches) * reps / el / 1e9

    reps_n, el_n = run(seconds / 2)
    orc.set_threads(1)
    try:
        reps_1, el_1 = run(seconds / 2)
    finally:
        orc.set_threads(all_threads)
    what = ("first 8 token rows of each GEMM" if gemm else
            f"the whole step ({' + '.join(L.case.name for L in launches)})")
    return {"value": rate(reps_n, el_n), "unit": "TFLOP/s" if gemm else "GB/s",
            "cores": all_threads, "kind": "oracle",
            "sample": f"{what}: {reps_n} repetitions in {el_n:.1f} s on {all_threads} threads, "
                      f"{reps_1} in {el_1:.1f} s on 1 thread",
            "value_1_thread": rate(reps_1, el_1),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "cpus_allowed": len(os.sched_getaffinity(0))}


def vendor_ceiling(launches, torch, stream):
    """Benchmark-only comparison for prefill workloads (never a library
    path): the weights dequantized once into float32 with torch operations,
    then the vendor FP32 GEMM (torch.mm, i.e. rocBLAS / hipBLASLt) on them.
    Reports both times per call, the GEMM's TFLOP/s, and the largest error
    of a sample of its outputs against the oracle, as a fraction of the
    1e-5 * sum|w x| bound."""
    import numpy as np
    import oracle
    orc = oracle.get()
    res = []
    for L in launches:
        c, wd = L.case, L.weights[0]
        codes = wd.codes

        def dequant():
            if c.fmt == 1:      # 8-bit, per-row fp32 scale
                return codes.float() * wd.scales[:, None]
            if c.fmt == 4:      # 8-bit, fp32 scale per 64 inputs
                return codes.float() * wd.scales.repeat_interleave(64, dim=1)
            if c.fmt == 2:      # 4-bit, bf16 scale and bias per 64 inputs (int16 bits)
                b = codes.view(torch.uint8).int()
                q4 = torch.stack((b & 15, b >> 4), dim=-1).reshape(c.M, c.K).float()
                bf = lambda t: (t.int() << 16).view(torch.float32).repeat_interleave(64, dim=1)
                return q4 * bf(wd.scales) + bf(wd.biases)
            # 1-bit, fp16 scale per 128 inputs (stored as int16 bits)
            bits = (codes.view(torch.uint8)[..., None].int() >> torch.arange(8, device="cuda")) & 1
            signs = (bits * 2 - 1).float().reshape(c.M, c.K)
            sc = wd.scales.view(torch.float16).float().repeat_interleave(128, dim=1)
            return signs * sc

        W = dequant()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = 5
        with torch.cuda.stream(stream):
            dequant()
            torch.mm(L.x.view(c.rows, c.K), W.t())
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                dequant()
            e1.record()
            for _ in range(reps):
                Y = torch.mm(L.x.view(c.rows, c.K), W.t())
            e2.record()
        torch.cuda.synchronize()
        dq_ms, mm_ms = e0.elapsed_time(e1) / reps, e1.elapsed_time(e2) / reps
        rng = np.random.default_rng(0)
        n = rng.integers(0, c.rows, 2000).astype(np.int64)
        m = rng.integers(0, c.M, 2000).astype(np.int64)
        ref, a = orc.qgemv_sample(c.fmt, L.host_w.codes, L.host_w.scales, L.host_w.biases,
                                  L.host_x, c.M, c.K, n, m)
        got = Y.cpu().numpy()[n, m].astype(np.float64)
        ratio = float(np.max(np.abs(got - ref) / (1e-5 * a)))
        res.append({"case": c.name, "dequant_us": round(dq_ms * 1e3, 2), "sgemm_us": round(mm_ms * 1e3, 2),
                    "sgemm_tflops": round(c.flops / (mm_ms * 1e-3) / 1e12, 2),
                    "max_err_over_bound": round(ratio, 4)})
        log(f"  vendor {c.name}: dequantize {dq_ms * 1e3:.1f} us, FP32 GEMM {mm_ms * 1e3:.1f} us "
            f"({c.flops / (mm_ms * 1e-3) / 1e12:.1f} TFLOP/s), max err/bound {ratio:.3g}")
        del W, Y
    return res


def run_probe(args, torch, synth):
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "gemm_qgemv_amd", "libqgprobe.so"))
    L.qg_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_void_p]
    L.qg_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_void_p]
    L.qg_probe_read_blocked.argtypes = L.qg_probe_read.argtypes
    s = torch.cuda.current_stream().cuda_stream
    if args.probe == "copy":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(8):
            assert L.qg_probe_copy(src.data_ptr(), dst.data_ptr(), n, 4096, s) == 0
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "launches": 8}))
        return
    names = WORKLOADS.get(args.workload, [args.workload])
    size = sum(synth.CASES_BY_NAME[nm].weight_bytes for nm in names) // 16 * 16
    copies = max(1, math.ceil((args.rotate_mib << 20) / size))
    bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    out = torch.empty(8192, dtype=torch.int32, device="cuda")
    best, best_cfg = None, None
    variants = [("grid-stride", L.qg_probe_read), ("blocked", L.qg_probe_read_blocked)]
    grids = (1024, 2048, 4096, 8192)
    per = {}
    for name, fn in variants:
        for grid in grids:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in bufs:
                    assert fn(b.data_ptr(), size, out.data_ptr(), grid,
                              torch.cuda.current_stream().cuda_stream) == 0
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, 200 // copies)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            log(f"  {args.probe} probe {name} grid {grid}: {us:.2f} us, {size / us / 1e3:.1f} GB/s")
            if name not in per or us < per[name][0]:
                per[name] = (us, grid)
            if best is None or us < best:
                best, best_cfg = us, f"{name}, grid {grid}"
    rec = {"probe": args.probe, "bytes": size, "us": round(best, 3),
           "GB/s": round(size / best / 1e3, 1), "best": best_cfg}
    rec["per_variant_GB/s"] = {k: round(size / v[0] / 1e3, 1) for k, v in per.items()}
    print(json.dumps(rec))


def gpu_state(torch):
    """Clocks, temperatures and power of the GPU, read from the kernel
    driver's hwmon files of its PCI device (plain file reads)."""
    try:
        pr = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id,
                                                         pr.pci_device_id)
    except Exception as e:   # noqa: BLE001 - older torch without the PCI ids
        return {"error": f"no PCI id: {e}"}
    out = {"pci": os.path.basename(dev)}
    for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
        for f in sorted(glob.glob(os.path.join(hw, "*_input")) + glob.glob(os.path.join(hw, "power*_average"))):
            name = os.path.basename(f)
            base = name.rsplit("_", 1)[0]
            label = base
            try:
                with open(os.path.join(hw, base + "_label")) as g:
                    label = g.read().strip() or base
            except OSError:
                pass
            try:
                with open(f) as g:
                    v = int(g.read().strip())
            except (OSError, ValueError):
                continue
            if base.startswith("temp"):
                out[f"temp_{label}_C"] = v / 1000.0
            elif base.startswith("freq"):
                out[f"freq_{label}_MHz"] = v / 1e6
            elif base.startswith("power"):
                out[f"power_{label}_W"] = v / 1e6
    for clk in ("pp_dpm_sclk", "pp_dpm_mclk"):
        try:
            with open(os.path.join(dev, clk)) as g:
                cur = [l.split(":", 1)[1].strip() for l in g if l.rstrip().endswith("*")]
            if cur:
                out[clk] = cur[0].rstrip("*").strip()
        except OSError:
            pass
    return out


def read_ceiling(torch, nbytes, rotate_mib):
    """The best cold streaming-read rate over `nbytes` (the step's weight
    bytes) of the measurement-only read kernels: both read kernels at four
    grid sizes, over a rotation of copies, HIP graph replays timed with
    events. Returns (GB/s, description)."""
    import ctypes
    path = os.path.join(ROOT, "gemm_qgemv_amd", "libqgprobe.so")
    if not os.path.exists(path):
        return None, "libqgprobe.so not built"
    L = ctypes.CDLL(path)
    for fn in (L.qg_probe_read, L.qg_probe_read_blocked):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    size = nbytes // 16 * 16
    copies = max(1, math.ceil((rotate_mib << 20) / size))
    bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    out = torch.empty(8192, dtype=torch.int32, device="cuda")
    best, cfg = None, None
    for name, fn in (("grid-stride", L.qg_probe_read), ("blocked", L.qg_probe_read_blocked)):
        for grid in (1024, 2048, 4096, 8192):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in bufs:
                    assert fn(b.data_ptr(), size, out.data_ptr(), grid,
                              torch.cuda.current_stream().cuda_stream) == 0
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, 200 // copies)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            if best is None or us < best:
                best, cfg = us, f"{name} read kernel, grid {grid}, {size} bytes x {copies} copies"
    del bufs
    return size / best / 1e3, cfg


def trace_summary(csv_path, workload, src_hash, command):
    """Markdown summary of a rocprofv3 kernel-trace CSV: per kernel the
    number of dispatches, average, median, p10 and p90 duration, with the
    dominant kernel's algorithmic rate, and a JSON line that bench.py reads
    back (profiles/trace_<workload>.md)."""
    import csv
    import statistics
    from gemm_qgemv_amd import synth
    durs = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName")
            t = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            durs.setdefault(name, []).append(t)
    names = WORKLOADS.get(workload, [workload])
    cases = [synth.CASES_BY_NAME[n] for n in names]
    rows = []
    for k, v in durs.items():
        v = sorted(v)
        q = statistics.quantiles(v, n=10) if len(v) >= 10 else [v[0]] * 9
        rows.append({"kernel": k, "calls": len(v), "avg_us": statistics.fmean(v),
                     "median_us": statistics.median(v), "p10_us": q[0], "p90_us": q[8],
                     "total_us": sum(v)})
    rows.sort(key=lambda r: -r["total_us"])
    dom = rows[0]
    gemm = cases[0].op == "gemm"
    lines = [f"# Kernel trace: workload {workload} ({', '.join(names)})", "",
             "Command (repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | average (us) | median (us) | p10 (us) | p90 (us) | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    tot = sum(r["total_us"] for r in rows)
    for r in rows:
        lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | {r['median_us']:.2f} | "
                     f"{r['p10_us']:.2f} | {r['p90_us']:.2f} | {100 * r['total_us'] / tot:.1f} |")
    rec = {"workload": workload, "kernel": dom["kernel"], "calls": dom["calls"],
           "avg_us": round(dom["avg_us"], 3), "median_us": round(dom["median_us"], 3),
           "p10_us": round(dom["p10_us"], 3), "p90_us": round(dom["p90_us"], 3),
           "kernel_source_hash": src_hash}
    if len(cases) == 1:
        c = cases[0]
        if gemm:
            rec["tflops_at_median"] = round(c.flops / (dom["median_us"] * 1e-6) / 1e12, 2)
            rec["frac_of_bf16_peak_at_median"] = round(rec["tflops_at_median"] / BF16_MATRIX_PEAK_TFLOPS, 4)
        else:
            # the gather: ids, the packed rows of those ids and the float32 rows
            b = c.rows * (4 + c.weight_bytes // c.M + 4 * c.K) if c.op == "embed" else c.weight_bytes
            rec["algorithmic_bytes"] = b
            rec["GBs_at_average"] = round(b / (dom["avg_us"] * 1e-6) / 1e9, 1)
            rec["GBs_at_median"] = round(b / (dom["median_us"] * 1e-6) / 1e9, 1)
            rec["frac_of_hbm_peak_at_median"] = round(rec["GBs_at_median"] / HBM_PEAK_GBS, 4)
    lines += ["", f"Kernel source hash (sha256 of gemm_qgemv_amd/csrc except probe.hip, first 16 hex): "
              f"`{src_hash}`.", "", "```json", json.dumps(rec), "```", ""]
    return "\n".join(lines)


def counter_summary(csv_paths, workload, src_hash, commands):
    """Markdown summary of rocprofv3 --pmc counter runs of one workload: per
    counter the average value per dispatch of the dominant kernel (the
    library kernel with the largest GRBM_GUI_ACTIVE), and the derived
    fractions with their formulas, plus a JSON line."""
    import csv
    from gemm_qgemv_amd import synth
    vals, meta = {}, {}
    for path in csv_paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                k = row["Kernel_Name"]
                if "qg::" not in k:
                    continue
                vals.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                meta[k] = {"grid": int(row["Grid_Size"]), "workgroup": int(row["Workgroup_Size"]),
                           "lds": int(row["LDS_Block_Size"]), "vgpr": int(row["VGPR_Count"]),
                           "agpr": int(row.get("Accum_VGPR_Count") or 0)}
    if not vals:
        raise SystemExit("no library kernel in the counter files")
    kern = max(vals, key=lambda k: sum(vals[k].get("GRBM_GUI_ACTIVE", [0])) / max(1, len(vals[k].get("GRBM_GUI_ACTIVE", [1]))))
    avg = {c: sum(v) / len(v) for c, v in vals[kern].items()}
    names = WORKLOADS.get(workload, [workload])
    case = synth.CASES_BY_NAME[names[0]] if len(names) == 1 else None
    simds, xcds = 1024, 8
    # GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles of the dispatch = sum / 8
    cycles = avg.get("GRBM_GUI_ACTIVE", 0.0) / xcds
    d = {}
    if cycles > 0:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            d["mfma_busy_frac"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * simds)
        if "SQ_INSTS_VALU" in avg:
            valu = avg["SQ_INSTS_VALU"] - avg.get("SQ_INSTS_MFMA", 0.0)
            d["valu_busy_frac"] = 4.0 * valu / (cycles * simds)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            d["valu_mfma_coexec_frac"] = avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cycles * simds)
    if "SQ_WAIT_INST_ANY" in avg and "SQ_WAVE_CYCLES" in avg and avg["SQ_WAVE_CYCLES"] > 0:
        d["wave_wait_frac"] = avg["SQ_WAIT_INST_ANY"] / avg["SQ_WAVE_CYCLES"]
    if case is not None and "SQ_INSTS_VALU" in avg:
        weights = case.M * case.K
        lane_ops = 64.0 * (avg["SQ_INSTS_VALU"] - avg.get("SQ_INSTS_MFMA", 0.0))
        if case.op == "gemm":
            d["valu_lane_ops_per_mac"] = lane_ops / (weights * case.rows)
        else:
            d["valu_lane_ops_per_weight"] = lane_ops / weights
    if case is not None and "SQ_INSTS_MFMA" in avg and avg["SQ_INSTS_MFMA"] > 0:
        d["mfma_instructions"] = avg["SQ_INSTS_MFMA"]
        d["mfma_flops_over_algorithmic"] = avg["SQ_INSTS_MFMA"] * 16 * 16 * 32 * 2 / case.flops
    lines = [f"# Counters: workload {workload} ({', '.join(names)})", "",
             "Commands (repository root, one MI355X; one counter set per run):", "", "```"] + \
        list(commands) + ["```", "",
             f"Kernel: `{kern}` (grid {meta[kern]['grid']}, workgroup {meta[kern]['workgroup']}, "
             f"LDS {meta[kern]['lds']} B, {meta[kern]['vgpr']} VGPRs, {meta[kern]['agpr']} AGPRs).", "",
             "| counter | average per dispatch |", "|---|---|"]
    for c in sorted(avg):
        lines.append(f"| {c} | {avg[c]:.4g} |")
    lines += ["", "Derived (GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the dispatch's cycles are "
              "its value / 8; 1024 SIMDs; a 64-lane VALU instruction occupies a 16-lane SIMD for 4 "
              "cycles; a 16x16x32 bf16 MFMA is 16384 flops):", "",
              "| quantity | value | formula |", "|---|---|---|"]
    formulas = {
        "mfma_busy_frac": "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024)",
        "valu_busy_frac": "4 (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (cycles x 1024)",
        "valu_mfma_coexec_frac": "SQ_VALU_MFMA_COEXEC_CYCLES / (cycles x 1024)",
        "wave_wait_frac": "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
        "valu_lane_ops_per_weight": "64 (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (M K)",
        "valu_lane_ops_per_mac": "64 (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (M K N)",
        "mfma_instructions": "SQ_INSTS_MFMA",
        "mfma_flops_over_algorithmic": "SQ_INSTS_MFMA x 16384 / (2 M K N)",
    }
    for k, v in d.items():
        lines.append(f"| {k} | {v:.4g} | {formulas[k]} |")
    rec = {"workload": workload, "kernel": kern, "kernel_source_hash": src_hash,
           **{k: round(v, 5) for k, v in d.items()}}
    lines += ["", f"Kernel source hash (sha256 of gemm_qgemv_amd/csrc except probe.hip, first 16 hex): "
              f"`{src_hash}`.", "", "```json", json.dumps(rec), "```", ""]
    return "\n".join(lines)


def traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload, src_hash,
                    commands):
    """HBM traffic per launch of the workload's library kernel from
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), each scaled
    by what the same counter reads for the copy probe of known size
    (`bench.py --probe copy`: 256 MiB read and 256 MiB written per
    dispatch). Writes profiles/traffic_<workload>.{md,json} content:
    returns (markdown, record)."""
    import csv

    def per_dispatch(path, kernel_filter):
        v = []
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if kernel_filter(row["Kernel_Name"]):
                    v.append(float(row["Counter_Value"]))
        return v

    lib = lambda k: "qg::" in k
    probe = lambda k: "qg_probe_copy" in k
    fe, wr = per_dispatch(fetch_csv, lib), per_dispatch(write_csv, lib)
    cf, cw = per_dispatch(copy_fetch_csv, probe), per_dispatch(copy_write_csv, probe)
    kib = 256 * 1024
    ff, wf = kib / (sum(cf) / len(cf)), kib / (sum(cw) / len(cw))
    fa, wa = sum(fe) / len(fe), sum(wr) / len(wr)
    rec = {"workload": workload, "kernel_source_hash": src_hash,
           "fetch_size_kib_per_dispatch": round(fa, 3), "write_size_kib_per_dispatch": round(wa, 3),
           "dispatches": [len(fe), len(wr)], "copy_probe_kib": kib,
           "copy_fetch_size_kib": round(sum(cf) / len(cf), 3),
           "copy_write_size_kib": round(sum(cw) / len(cw), 3),
           "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
           "hbm_read_bytes_per_launch": int(fa * ff * 1024),
           "hbm_write_bytes_per_launch": int(wa * wf * 1024)}
    rec["traffic_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    names = WORKLOADS.get(workload, [workload])
    lines = [f"# HBM traffic per launch: workload {workload} ({', '.join(names)})", "",
             "Commands (repository root, one MI355X), each counter in its own run:", "", "```"] + \
        list(commands) + ["```", "",
             f"Calibration: the copy probe moves 256 MiB in and 256 MiB out per dispatch; FETCH_SIZE "
             f"reads {rec['copy_fetch_size_kib']} KiB and WRITE_SIZE {rec['copy_write_size_kib']} KiB "
             f"for it, so the factors are {ff:.4f} (fetch) and {wf:.4f} (write).", "",
             "| counter | KiB per dispatch | dispatches | scaled bytes per launch |", "|---|---|---|---|",
             f"| FETCH_SIZE | {fa:.1f} | {len(fe)} | {rec['hbm_read_bytes_per_launch']:,} |",
             f"| WRITE_SIZE | {wa:.1f} | {len(wr)} | {rec['hbm_write_bytes_per_launch']:,} |",
             f"| total | | | {rec['traffic_bytes_per_launch']:,} |", "",
             f"Kernel source hash (sha256 of gemm_qgemv_amd/csrc except probe.hip, first 16 hex): "
             f"`{src_hash}`.", ""]
    return "\n".join(lines), rec


def load_trace(workload, src_hash):
    """The committed kernel-trace summary of this workload, if it was taken
    from the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"trace_{workload}.md")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if rec.get("kernel_source_hash") != src_hash:
        return None
    rec["file"] = os.path.relpath(p, ROOT)
    return rec


def load_traffic(workload, src_hash):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (default: about 2000 launches)")
    ap.add_argument("--warmup", type=int, default=0)
    ap.add_argument("--workload", default="c2b1")
    ap.add_argument("--rotate-mib", type=int, default=640)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--launch-only", action="store_true",
                    help="only run the warmup and the steps, eagerly, and print nothing else "
                         "(for counter collection under rocprofv3 --pmc)")
    ap.add_argument("--vendor", action="store_true",
                    help="prefill workloads: also time the vendor FP32 GEMM on weights dequantized "
                         "once (benchmark-only comparison, reported as vendor_ceiling)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarize a rocprofv3 kernel-trace CSV of this workload (markdown with a "
                         "JSON line, as committed under profiles/trace_<workload>.md) and exit")
    ap.add_argument("--trace-command", default="",
                    help="the command that produced the trace, quoted in the summary")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="summarize rocprofv3 --pmc counter CSVs of this workload (markdown with a "
                         "JSON line, as committed under profiles/counters_<workload>.md) and exit; "
                         "--trace-command may be given once per run")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.md and .json from rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE runs of the workload and of --probe copy, and exit")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip timing the streaming-read ceiling over the step's weight bytes")
    ap.add_argument("--probe", choices=["copy", "read"],
                    help="run only a measurement probe: 'copy' copies 256 MiB 8 times (a kernel of "
                         "known traffic, to calibrate FETCH_SIZE / WRITE_SIZE); 'read' times cold "
                         "streaming reads of the workload's weight size (two read kernels, four "
                         "grid sizes, best reported)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the kernels work on one "
              "GPU's share of the matrix; there is no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.workload, kernel_source_hash(),
                            args.trace_command))
        return
    if args.traffic_summary:
        md, rec = traffic_summary(*args.traffic_summary, args.workload, kernel_source_hash(),
                                  args.trace_command.split(" ;; ") if args.trace_command else [])
        with open(os.path.join(ROOT, "profiles", f"traffic_{args.workload}.md"), "w") as f:
            f.write(md)
        with open(os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(md)
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary, args.workload, kernel_source_hash(),
                              args.trace_command.split(" ;; ") if args.trace_command else []))
        return

    import torch

    import gemm_qgemv_amd as q
    from gemm_qgemv_amd import synth, tensors

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.probe:
        run_probe(args, torch, synth)
        return
    names = WORKLOADS.get(args.workload, [args.workload])
    cases = [synth.CASES_BY_NAME[n] for n in names]
    gemm = cases[0].op == "gemm"
    log(f"workload {args.workload}: {names}")
    launches = [Launch(c, args.rotate_mib << 20, torch, q, synth, tensors) for c in cases]
    rot = max(L.copies for L in launches)
    log(f"weight copies rotated: {[L.copies for L in launches]}")

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def step(i, s):
        for L in launches:
            L(i, s)

    per_step_launch_target = 2000 // len(launches) if not gemm else 20
    steps = args.steps or max(rot, per_step_launch_target)
    warmup = args.warmup or max(rot, 20 if not gemm else 3)
    # one HIP graph of all the timed steps (step i reads weight copy
    # i mod copies), so the host's graph launch is paid once, not per step
    chunk = steps

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i, sh)
    torch.cuda.synchronize()
    if args.launch_only:
        with torch.cuda.stream(stream):
            for i in range(steps):
                step(i, sh)
        torch.cuda.synchronize()
        log(f"launched {warmup} + {steps} steps of {args.workload}")
        return

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(chunk):
                step(i, stream.cuda_stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    state_before = gpu_state(torch)
    # ---- timed region -------------------------------------------------
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record()
        if graph is not None:
            for _ in range(steps // chunk):
                graph.replay()
        else:
            for i in range(steps):
                step(i, sh)
        ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / steps
    log(f"timed {steps} steps: {ms_total:.3f} ms on the stream, {wall * 1e3:.3f} ms wall")

    state_after = gpu_state(torch)

    # ---- per-call durations ---------------------------------------------
    # A step of one call: the call's duration is the timed region's step
    # time. A step of several calls: each call timed alone the same way (a
    # HIP graph of one pass over its weight copies, replayed, between HIP
    # events on the stream the kernels run on).
    per_case = []
    if len(launches) == 1:
        per_case.append((launches[0], ms_per_step))
    else:
        for L in launches:
            n = L.copies if not gemm else 4
            per_case.append((L, per_launch_ms(torch, L, stream, n,
                                              reps=max(1, 400 // n) if not gemm else 5)))
    for L, avg in per_case:
        unit = L.weight_bytes / (avg * 1e-3) / 1e9
        log(f"  {L.case.name}: {avg * 1e3:.2f} us per call, {unit:.1f} GB/s weight"
            + (f", {L.case.flops / (avg * 1e-3) / 1e12:.2f} TFLOP/s"
               if gemm or (L.case.rows > 1 and L.case.op != "embed") else ""))

    src_hash = kernel_source_hash()
    traffic = load_traffic(args.workload, src_hash)
    trace = load_trace(args.workload, src_hash)
    dom = max(per_case, key=lambda t: t[1])
    if gemm:
        flops = sum(L.case.flops for L in launches)
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = dom[0].case.flops / (dom[1] * 1e-3) / 1e12
        # the products run on bf16 MFMA (three exact passes per algorithmic
        # multiply-add), so the bf16 dense peak is the ceiling
        roof = {"bound": "mfma", "achieved": round(ach, 3), "peak": BF16_MATRIX_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_MATRIX_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel_call": dom[0].case.name,
                "us_per_call": round(dom[1] * 1e3, 3), "mfma_passes_per_mac": 3,
                "frac_of_fp32_matrix_peak": round(ach / FP32_MATRIX_PEAK_TFLOPS, 4)}
        dtype = "f32"
    else:
        wbytes = sum(L.weight_bytes for L in launches)
        value = wbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        ach = dom[0].weight_bytes / (dom[1] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel_call": dom[0].case.name, "us_per_call": round(dom[1] * 1e3, 3),
                "algorithmic_bytes_per_call": dom[0].weight_bytes}
        dtype = "f32"
    roof["timing"] = ("timed region (the step is this one call)" if len(launches) == 1 else
                      "this call alone, timed like the step")
    if trace is not None:
        roof["trace"] = trace

    embed = cases[0].op == "embed"
    out = {
        "metric": EMBED_METRIC if embed else METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "cases": names,
                   "shapes_MxK": [[c.M, c.K] for c in cases], "rows": [c.rows for c in cases],
                   "format": synth.FORMAT_NAMES[cases[0].fmt],
                   "weights": "cache-cold rotation" if not gemm else "resident",
                   "weight_copies": [L.copies for L in launches],
                   "launch": "hip graph" if graph is not None else "eager"},
        "roofline": roof,
    }
    out["gpu_state"] = {"before": state_before, "after": state_after}
    if not gemm:
        out["pct_of_hbm_peak"] = round(100 * value / HBM_PEAK_GBS, 2)
        if not args.no_read_ceiling and cases[0].op != "embed":
            rc, how = read_ceiling(torch, dom[0].weight_bytes, args.rotate_mib)
            if rc is not None:
                out["read_ceiling"] = {"GB/s": round(rc, 1), "how": how,
                                       "pct_of_ceiling": round(100 * ach / rc, 2)}
    if not gemm and not embed:
        out["tok_s_equiv"] = round(value * 1e9 / BYTES_PER_TOKEN[cases[0].fmt], 1)
    if gemm and args.vendor:
        out["vendor_ceiling"] = vendor_ceiling(launches, torch, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(launches, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
