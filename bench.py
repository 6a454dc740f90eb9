#!/usr/bin/env python3
"""Benchmark of the swizzled GEMM on one MI355X.

A step is one call of the hot path on one batch of synthetic input that is
already resident in HBM.  The default workload is the dense 8192^3 bf16 GEMM
D = A*B + C (A and B K-major, C bf16, bf16 output, fp32 accumulation); the
other workloads (--workload) are the grouped 16 x 4096^2 GEMM, the MXFP8,
MXFP6 (e2m3, or e3m2 as mxfp6_e3m2) and MXFP4 8192^3 GEMMs, the 1024^3 and
the 128x128x32 single-tile GEMMs.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value          whole-job TFLOP/s = 2*M*N*K / (measured seconds per step)
  roofline       the dominant kernel against MI355X's published dense MFMA
                 peak for its dtype (bf16/fp16 2516.6, fp8 5033.2, fp6 and fp4
                 10066.4 TFLOP/s);
                 achieved = algorithmic FLOP per launch / mean launch time
                 from two HIP events on the launch stream around the K
                 timed launches
  cpu_baseline   the CPU oracle (fp64 triple loop, all host cores) timed on a
                 bounded row sample of the same workload, in TFLOP/s
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e2m1": 10066.4,
               "e2m3": 10066.4, "e3m2": 10066.4}
HBM_PEAK_GBS = 8000.0
SPEC_GHZ = 2.4   # the clock MI355X's published MFMA peaks are quoted at
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
SIMDS = 1024        # 256 CUs x 4 SIMDs
CLOCK_LAUNCHES = 10  # launches in each clock-trace window (before, after the timed ones)


def _code_only(text: str) -> str:
    """C/C++ source with comments and blank lines removed (string literals in
    these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 of the kernel sources and the C header, comments left out: HBM
    traffic measured with rocprofv3 is reported only while it still
    describes this code."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_swizzled_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    with open(os.path.join(ROOT, "include", "swizzled_gemm.h"), encoding="utf-8") as f:
        h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_counters(workload: str):
    """The committed rocprofv3 counters of `workload` (profiles/counters.json,
    written by --profile), or None when they were taken on other kernel
    sources."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_workload(name: str, dev, layout=None):
    """Returns (run callable, flops per step, dtype, config dict, oracle
    sample callable(rows) -> seconds, rows_total)."""
    import torch

    import dense_gemm_swizzled_amd as sg
    import synth_inputs as si

    if name in ("dense_8192", "dense_1024", "single_tile"):
        case = {"dense_8192": si.dense_8192, "dense_1024": si.dense_1024,
                "single_tile": si.single_tile}[name]()
        A, B = case.A.to(dev), case.B.to(dev)
        C = case.C.to(dev) if case.C is not None else None
        dt = {"f32": torch.float32, "bf16": torch.bfloat16}[case.d_dtype]
        D = torch.empty(case.M, case.N, dtype=dt, device=dev)

        if layout is None:
            # The call's arguments are marshalled once: at 1024^3 and below the
            # kernel is shorter than a Python-level call.
            run = sg.gemm_plan(A, B, a_major=case.a_major, b_major=case.b_major, C=C, out=D)
        elif layout[0] == "io":
            if case.ab_dtype != "bf16" or case.a_major != "k" or case.b_major != "k" \
                    or case.d_dtype != "bf16":
                raise SystemExit("--layout-io needs a bf16 workload with K-major A and B and "
                                 "a bf16 D")
            _, ops, outs = layout

            def run():
                sg.gemm_layout_io(A, B, ops, outs, C=C, out=D)
        else:
            if case.ab_dtype != "bf16" or case.a_major != "k" or case.b_major != "k":
                raise SystemExit("--layout needs a bf16 workload with K-major A and B")

            kernel, lay = layout

            def run():
                if kernel == 256:
                    sg.gemm_layout(A, B, lay, C=C, out=D)
                else:
                    sg.gemm_layout128(A, B, lay, C=C, out=D)

        flops = 2.0 * case.M * case.N * case.K
        cfg = {"workload": case.name, "M": case.M, "N": case.N, "K": case.K,
               "a_major": case.a_major, "b_major": case.b_major,
               "ab_dtype": case.ab_dtype, "c": case.c_dtype, "d_dtype": case.d_dtype}
        if layout is not None and layout[0] == "io":
            cfg["lds_layout"] = {16: "xor_256B_lines", 0: "none"}[layout[1]]
            cfg["output_staging"] = "xor" if layout[2] else "none"
            cfg["tile"] = "256x256"
        elif layout is not None:
            cfg["lds_layout"] = {16: "xor_256B_lines", 8: "xor_128B_lines", 0: "none",
                                 sg.SG_LAYOUT_PAD16: "padded_16B"}[layout[1]]
            cfg["tile"] = f"{layout[0]}x{layout[0]}"

        def oracle_sample(rows):
            import oracle
            a = case.A[:rows] if case.a_major == "k" else case.A[:, :rows].contiguous()
            c = case.C[:rows] if case.C is not None else None
            t0 = time.perf_counter()
            oracle.gemm(rows, case.N, case.K, a, case.a_major, case.B, case.b_major,
                        case.ab_dtype, c, case.c_dtype, with_bound=False)
            return time.perf_counter() - t0, 2.0 * rows * case.N * case.K

        return run, flops, case.ab_dtype, cfg, oracle_sample, case.M

    if name == "grouped":
        case = si.grouped()
        A, B = case.A.to(dev), case.B.to(dev)
        D = torch.empty(case.A.shape[0], case.N, dtype=torch.bfloat16, device=dev)

        def run():
            sg.grouped_gemm(A, B, case.m_offsets, out=D)

        flops = 2.0 * case.m_offsets[-1] * case.N * case.K
        cfg = {"workload": case.name, "G": case.G, "m_sizes": case.m_sizes,
               "N": case.N, "K": case.K, "ab_dtype": "bf16", "d_dtype": "bf16"}

        def oracle_sample(rows):
            import oracle
            Bn = case.B.reshape(case.G, case.N, case.K)
            t0 = time.perf_counter()
            oracle.gemm(rows, case.N, case.K, case.A[:rows], "k", Bn[0], "k", "bf16",
                        with_bound=False)
            return time.perf_counter() - t0, 2.0 * rows * case.N * case.K

        return run, flops, "bf16", cfg, oracle_sample, case.m_sizes[0]

    if name in ("mxfp8", "mxfp4", "mxfp6", "mxfp6_e3m2"):
        case = {"mxfp8": lambda: si.mxfp8(), "mxfp4": lambda: si.mxfp4(),
                "mxfp6": lambda: si.mxfp6(),
                "mxfp6_e3m2": lambda: si.mxfp6(fmt="e3m2")}[name]()
        A, SFA, B, SFB = (t.to(dev) for t in (case.A, case.SFA, case.B, case.SFB))
        D = torch.empty(case.M, case.N, dtype=torch.bfloat16, device=dev)
        # A step takes the scales as they come, [rows][K/32], and rearranges
        # them into the 64-row blocks the GEMM reads one KiB at a time
        # (mx_scales_to_blocks), then runs the GEMM on them.
        sfa_b = torch.empty(sg.mx_scales_blocks_bytes(case.M, case.K), dtype=torch.uint8,
                            device=dev)
        sfb_b = torch.empty(sg.mx_scales_blocks_bytes(case.N, case.K), dtype=torch.uint8,
                            device=dev)
        code = {"e4m3": sg.SG_E4M3, "e2m1": sg.SG_E2M1, "e2m3": sg.SG_E2M3,
                "e3m2": sg.SG_E3M2}[case.fmt]
        st = torch.cuda.current_stream(dev).cuda_stream
        # The closure holds the tensors themselves: their raw pointers alone
        # would let torch's allocator hand the memory to later tensors.
        tensors = (A, SFA, B, SFB, D, sfa_b, sfb_b)

        def run():
            a, sa, b, sb, d, sab, sbb = (t.data_ptr() for t in tensors)
            rc = (sg.mx_scales_to_blocks(sa, case.M, case.K, sab, st)
                  or sg.mx_scales_to_blocks(sb, case.N, case.K, sbb, st)
                  or sg.mx_gemm_blocks_run(code, case.M, case.N, case.K, a, sab, b, sbb, d,
                                           sg.SG_BF16, st))
            if rc:
                raise RuntimeError(sg.gemm_last_error())

        flops = 2.0 * case.M * case.N * case.K
        cfg = {"workload": case.name, "M": case.M, "N": case.N, "K": case.K,
               "block": 32, "ab_dtype": case.fmt, "scale": "e8m0",
               "scale_layout": "[rows][K/32], rearranged into 64-row blocks in the step",
               "d_dtype": "bf16"}

        def oracle_sample(rows):
            import oracle
            t0 = time.perf_counter()
            oracle.mx_gemm(rows, case.N, case.K, case.A[:rows], case.SFA[:rows], case.B,
                           case.SFB, with_bound=False, fmt=case.fmt)
            return time.perf_counter() - t0, 2.0 * rows * case.N * case.K

        return run, flops, case.fmt, cfg, oracle_sample, case.M

    if name == "copy":
        # A plain device copy of known size: the reference for scaling the
        # FETCH_SIZE / WRITE_SIZE counters into bytes.
        n = 256 << 20
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)

        def run():
            dst.copy_(src)

        cfg = {"workload": "copy_1GiB_f32", "bytes_read": 4 * n, "bytes_written": 4 * n}
        return run, 0.0, "bf16", cfg, None, 0

    raise SystemExit(f"unknown workload {name}")


def prewarm(run, stream, min_s=0.5, max_s=4.0, tol=0.01):
    """Launches the step until the GPU has run it for at least min_s seconds
    and two successive windows of launches agree on the mean launch time
    within tol (or max_s seconds have passed).  The MI355X's clock takes
    tens of launches of a long GEMM to settle (at 8192^3 the early launches
    run 10-35% slower than the settled ones), so a short warmup alone would
    time the ramp.  Returns (launches, GPU seconds, last window's mean ms)."""
    import torch
    total_s, launches, prev, window = 0.0, 0, None, 8
    while True:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(window):
            run()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / window
        total_s += ms * window / 1e3
        launches += window
        if total_s >= max_s or (total_s >= min_s and prev is not None
                                and abs(ms - prev) <= tol * prev):
            return launches, total_s, ms
        prev = ms
        # windows of about 20 ms of GPU time
        window = int(min(5000, max(8, 20.0 / max(ms, 1e-3))))


class ClockWindow:
    """The clock the dominant kernel ran at over `launches` back-to-back
    launches: the library's per-workgroup clock trace (shader-clock and
    real-time counters at the start and end of every workgroup), each launch
    into its own part of the trace buffer (the clock moves over a few
    milliseconds, so one launch alone is not representative).

    The buffer is allocated when the window is made and the records are read
    only in result(), so that running the window (enqueue only) leaves the
    GPU no idle time: after a few milliseconds of idle the clock drops and
    the next launches run slower while it ramps back."""

    SLOTS = 1 << 13          # per launch; every grid here is smaller

    def __init__(self, dev, launches):
        import torch
        self.launches = launches
        self.buf = torch.full((launches, 4 * self.SLOTS), -1, dtype=torch.int64, device=dev)
        self.khz = 0

    def run(self, run):
        import dense_gemm_swizzled_amd as sg
        try:
            for i in range(self.launches):
                self.khz = sg.gemm_clock_trace(self.buf[i].data_ptr(), self.SLOTS)
                run()
        finally:
            sg.gemm_clock_trace(None, 0)

    def result(self):
        """(GHz, workgroups one launch ran, mean launch span in seconds), the
        span being first workgroup start to last workgroup end on the
        real-time counter; or (None, 0, None) if nothing was recorded."""
        import numpy as np
        raw = self.buf.view(self.launches, self.SLOTS, 4).cpu().numpy()
        written = (raw != -1).any(axis=2)
        per_launch = int(written.sum(axis=1).max())
        v = raw[written].astype(np.float64)
        ok = (v[:, 1] > v[:, 0]) & (v[:, 3] > v[:, 2])
        log(f"[bench] clock trace: {per_launch} workgroups a launch over {self.launches} "
            f"launches, {int(ok.sum())} records with increasing counters")
        if not ok.any() or self.khz <= 0:
            return None, 0, None
        spans = []
        for i in range(self.launches):
            r = raw[i][written[i]].astype(np.float64)
            r = r[(r[:, 1] > r[:, 0]) & (r[:, 3] > r[:, 2])]
            if len(r):
                spans.append((r[:, 3].max() - r[:, 2].min()) / (self.khz * 1e3))
        v = v[ok]
        return (float((v[:, 1] - v[:, 0]).sum() / (v[:, 3] - v[:, 2]).sum() * self.khz / 1e6),
                per_launch, float(np.mean(spans)) if spans else None)


def probe_clock(dev, iters=10000):
    """The MFMA clock probe: the two waves on every SIMD each issue 8 * iters
    independent 16-cycle bf16 MFMAs.  Per CU (eight waves), the clock from
    the MFMA count is 16 * 2 * 8 * iters cycles over the real-time span of
    its waves, and the shader-clock counter's span over the same real-time
    span is the counter's rate; they agree when the counter counts core
    clocks and the MFMA pipes were kept busy.  Returns both, in GHz,
    averaged over the CUs."""
    import numpy as np
    import torch

    import dense_gemm_swizzled_amd as sg
    khz = sg.gemm_clock_trace(None, 0)
    waves = sg.gemm_clock_probe_waves()
    out = torch.zeros(5 * waves, dtype=torch.int64, device=dev)
    rc = sg.gemm_clock_probe(iters, out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    if rc != sg.SG_OK:
        raise sg.GemmError(rc, sg.gemm_last_error())
    torch.cuda.synchronize()
    return probe_ghz(out[:4 * waves].view(-1, 8, 4).cpu().numpy(), iters, khz)


def probe_ghz(v, iters, khz):
    """(MFMA-count GHz, counter GHz) from the probe's [CU][wave][4] counters."""
    import numpy as np
    v = v.astype(np.float64)
    span_rt = (v[:, :, 3].max(axis=1) - v[:, :, 2].min(axis=1)) / (khz * 1e3)
    span_t = v[:, :, 1].max(axis=1) - v[:, :, 0].min(axis=1)
    mfma_cycles = 16.0 * 2 * 8 * iters
    return float(np.mean(mfma_cycles / span_rt) / 1e9), float(np.mean(span_t / span_rt) / 1e9)


# ------------------------------------------------------------------ profiling
#
# bench.py --profile OUTDIR runs the bench of each selected workload under
# rocprofv3 as child processes (this process never touches the GPU), one pass
# per counter group the hardware can collect at once, and writes
# OUTDIR/<kernel>__<workload>.md plus OUTDIR/counters.json, the file the
# normal run reads its traffic and counters from (copied to profiles/).

PMC_PASSES = [
    ("sq", ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
            "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_WAVES",
            "GRBM_GUI_ACTIVE"]),
    ("fetch", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
]
MOPS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
        "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4"]


def profile_key(workload: str, layout) -> str:
    """The counters.json key of a bench configuration."""
    if layout is None:
        return workload
    if layout[0] == "io":
        return f"{workload}@io{layout[1]}_{layout[2]}"
    return f"{workload}@layout{layout[0]}_{layout[1]}"


def _csv_rows(outdir: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _rocprof(tool_args, bench_args, outdir, tag, timeout_s=300):
    """One rocprofv3 pass over `bench.py bench_args`; returns (stdout, outdir
    of the pass)."""
    import subprocess
    d = os.path.join(outdir, "raw", tag)
    os.makedirs(d, exist_ok=True)
    cmd = ["rocprofv3", *tool_args, "-d", d, "-o", tag, "--output-format", "csv", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    log(f"[profile] {tag}: {' '.join(cmd)}")
    r = subprocess.run(cmd, cwd="/tmp", env={**os.environ, "TMPDIR": "/tmp"},
                       capture_output=True, text=True, timeout=timeout_s)
    with open(os.path.join(d, "bench.err"), "w") as f:
        f.write(r.stderr)
    if r.returncode != 0 and not r.stdout.strip():
        raise SystemExit(f"[profile] {tag} failed ({r.returncode}):\n{r.stderr[-2000:]}")
    log(f"[profile] {tag}: done")
    return r.stdout, d, cmd


def _dominant(trace_rows):
    """(name, [durations ns in launch order]) of the kernel with the most GPU
    time."""
    by = {}
    for r in trace_rows:
        name = r["Kernel_Name"]
        by.setdefault(name, []).append(
            (int(r.get("Dispatch_Id") or 0), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    name = max(by, key=lambda n: sum(d for _, d in by[n]))
    return name, [d for _, d in sorted(by[name])]


def _counter_means(rows, kernel, first, count):
    """Per counter, the mean over dispatches [first, first + count) of
    `kernel` (values of one dispatch summed over their dimensions)."""
    per = {}
    for r in rows:
        if r["Kernel_Name"] != kernel:
            continue
        did = int(r["Dispatch_Id"])
        per.setdefault(did, {})
        name = r["Counter_Name"]
        per[did][name] = per[did].get(name, 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[first:first + count]
    out = {}
    for did in ids:
        for k, v in per[did].items():
            out[k] = out.get(k, 0.0) + v / len(ids)
    return out


def _short(kernel: str) -> str:
    """'void sg::deep_gemm_kernel<64, ...>(...)' -> 'deep_gemm_kernel'."""
    k = kernel.split("(")[0]
    k = k.split("<")[0]
    k = k.split("::")[-1].replace("void ", "").strip()
    return k.removeprefix("__amd_rocclr_") or "kernel"


def profile(args, layout_args):
    outdir = os.path.abspath(args.profile)
    os.makedirs(outdir, exist_ok=True)
    # Start from what is already measured on these sources: the committed
    # file, then earlier runs into the same OUTDIR.
    base = {"workloads": {}}
    for path in (COUNTERS_FILE, os.path.join(outdir, "counters.json")):
        try:
            with open(path) as f:
                t = json.load(f)
        except (OSError, ValueError):
            continue
        if t.get("kernel_source_hash") == kernel_source_hash():
            base["workloads"].update(t.get("workloads", {}))
            for k in ("fetch_factor", "write_factor"):
                if t.get(k):
                    base[k] = t[k]
    result = {"kernel_source_hash": kernel_source_hash(),
              "note": "per launch: kernel_ns (mean of the timed launches, kernel trace), "
                      "clock_ghz (the kernel's own clock trace, mean of the windows before "
                      "and after the timed launches), clock_windows (each window's clock and "
                      "its launches' mean time), mfma_busy (per window, mean), counters (mean "
                      "of the timed launches of a --pmc pass); bytes = FETCH_SIZE[KiB]*1024*fetch_factor + "
                      "WRITE_SIZE[KiB]*1024*write_factor, factors from a 1 GiB device copy",
              "fetch_factor": base.get("fetch_factor"), "write_factor": base.get("write_factor"),
              "workloads": dict(base.get("workloads", {}))}
    workloads = args.workload.split(",")
    if "copy" in workloads:
        workloads = ["copy"] + [w for w in workloads if w != "copy"]
    for w in workloads:
        key = profile_key(w, _layout_tuple(args))
        common = ["--workload", w, "--no-cpu-baseline", *layout_args]
        trace_args = common + ["--steps", str(args.steps), "--warmup", str(args.warmup)]
        pmc_args = common + ["--steps", "10", "--warmup", "3", "--no-prewarm", "--no-clock"]
        stdout, d, cmd_trace = _rocprof(["--kernel-trace", "--stats"], trace_args, outdir,
                                        f"{w}_trace")
        line = json.loads(stdout.strip().splitlines()[-1])
        name, durs = _dominant(_csv_rows(d, "kernel_trace.csv"))
        # Launch order of the bench: warmup, prewarm, the clock window
        # before, the timed launches, the clock window after.
        ck = line.get("clock") or {}
        nb, na = int(ck.get("launches_before") or 0), int(ck.get("launches_after") or 0)
        first = args.warmup + int(line.get("prewarm_launches") or 0) + nb
        if len(durs) != first + args.steps + na:
            log(f"[profile] {w}: {len(durs)} launches of {name} in the trace, expected "
                f"{first + args.steps + na}; averaging all of them")
            first, nb, na = 0, 0, 0
            timed = durs
        else:
            timed = durs[first:first + args.steps]
        kernel_ns = sum(timed) / len(timed)
        clock = ck.get("gemm_ghz")
        # Each clock window with its own launches' mean duration.
        windows = []
        for ghz, seg in ((ck.get("gemm_ghz_before"), durs[first - nb:first] if nb else []),
                         (ck.get("gemm_ghz_after"),
                          durs[first + args.steps:first + args.steps + na] if na else [])):
            if ghz and seg:
                windows.append((ghz, sum(seg) / len(seg)))
        counters, cmds = {}, [cmd_trace]
        passes = PMC_PASSES if w != "copy" else [p for p in PMC_PASSES if p[0] != "sq"]
        for tag, names in passes:
            _, d2, cmd = _rocprof(["--pmc", *names], pmc_args, outdir, f"{w}_{tag}")
            cmds.append(cmd)
            rows = _csv_rows(d2, "counter_collection.csv")
            counters.update(_counter_means(rows, name, 3, 10))
        flops = _flops_of(line)
        entry = {"kernel": name, "kernel_ns": round(kernel_ns, 1), "launches_averaged": len(timed),
                 "clock_ghz": clock,
                 "clock_windows": [{"ghz": g, "kernel_ns": round(t, 1)} for g, t in windows],
                 "counters": {k: round(v, 3) for k, v in counters.items()}}
        if w == "copy":
            n = line["config"]["bytes_read"]
            result["fetch_factor"] = n / (counters["FETCH_SIZE"] * 1024)
            result["write_factor"] = line["config"]["bytes_written"] / (counters["WRITE_SIZE"] * 1024)
        if "FETCH_SIZE" in counters and result["fetch_factor"]:
            entry["fetch_kib"] = counters["FETCH_SIZE"]
            entry["write_kib"] = counters["WRITE_SIZE"]
            entry["bytes"] = (counters["FETCH_SIZE"] * 1024 * result["fetch_factor"]
                              + counters["WRITE_SIZE"] * 1024 * result["write_factor"])
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            mops = sum(counters.get(m, 0.0) for m in MOPS)
            entry["mops_x512"] = mops * 512
            entry["flops"] = flops
            entry["mops_x512_equals_2mnk"] = abs(mops * 512 - flops) < 0.5
            entry["lds_bank_conflict_cycles"] = counters["SQ_LDS_BANK_CONFLICT"]
            entry["lds_idx_active_cycles"] = counters["SQ_LDS_IDX_ACTIVE"]
            if windows:
                # Busy cycles over the SIMD cycles of a launch, each clock
                # window's clock with that window's own launch time (the
                # clock drifts; a clock from one window with the time of
                # another would mix two operating points).
                b = [counters["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * g * t) for g, t in windows]
                entry["mfma_busy"] = round(sum(b) / len(b), 4)
        result["workloads"][key] = entry
        _write_summary(outdir, w, key, line, entry, cmds, result)
        with open(os.path.join(outdir, "counters.json"), "w") as f:
            json.dump(result, f, indent=1, sort_keys=True)
        log(f"[profile] {key}: {json.dumps(entry)}")


def _flops_of(line) -> float:
    c = line["config"]
    if "m_sizes" in c:
        return 2.0 * sum(c["m_sizes"]) * c["N"] * c["K"]
    if "M" in c:
        return 2.0 * c["M"] * c["N"] * c["K"]
    return 0.0


def _layout_tuple(args):
    if args.layout is not None:
        return (256, args.layout)
    if args.layout_io is not None:
        ops, outs = (int(x) for x in args.layout_io.split(","))
        return ("io", ops, outs)
    if args.layout128 is not None:
        return (128, -1 if args.layout128 == "pad" else int(args.layout128))
    return None


def _write_summary(outdir, w, key, line, e, cmds, result):
    name = f"{_short(e['kernel'])}__{key.replace('@', '_')}.md"
    peak = PEAK_TFLOPS.get(line.get("dtype"), 0)
    L = [f"# {_short(e['kernel'])} -- {key}", "",
         f"Workload: `{json.dumps(line['config'])}`.", f"Kernel: `{e['kernel']}`.", "",
         "Made by `python bench.py --profile <outdir> --workload " + w + "` (from the repository "
         "root), which ran these passes (each its own process):", ""]
    L += ["    " + " ".join(c).replace(ROOT, "$REPO") for c in cmds]
    L += ["", "| quantity | value |", "|---|---|",
          f"| kernel time (mean of {e['launches_averaged']} timed launches, kernel trace) | "
          f"{e['kernel_ns'] / 1e3:.3f} us |",
          f"| clock the kernel held (its own clock trace, mean of the windows of "
          f"{CLOCK_LAUNCHES} launches before and after the timed ones) | {e['clock_ghz']} GHz |"]
    for tag, cw in zip(("before", "after"), e.get("clock_windows") or []):
        L.append(f"| clock window {tag}: clock, mean kernel time (kernel trace) | "
                 f"{cw['ghz']} GHz, {cw['kernel_ns'] / 1e3:.3f} us |")
    for k, v in sorted(e["counters"].items()):
        L.append(f"| {k} (mean per timed launch) | {v:g} |")
    if "flops" in e and e["flops"]:
        t = e["kernel_ns"] * 1e-9
        ach = e["flops"] / t / 1e12
        L += [f"| algorithmic FLOP per launch | {e['flops']:.6g} |",
              f"| MFMA MOPS x 512 | {e['mops_x512']:.6g} "
              f"({'equal' if e['mops_x512_equals_2mnk'] else 'DIFFERENT'}) |",
              f"| achieved | {ach:.1f} TFLOP/s = {100 * ach / peak:.1f}% of {peak} |"
              if peak else ""]
        if e.get("mfma_busy") is not None:
            L.append(f"| MFMA busy = BUSY_CYCLES / (1024 SIMDs x clock x time), per clock window, mean | "
                     f"{100 * e['mfma_busy']:.1f}% |")
        L.append(f"| LDS bank-conflict cycles | {e['lds_bank_conflict_cycles']:g} |")
    if "bytes" in e:
        L.append(f"| HBM-side bytes (FETCH x {result['fetch_factor']:.4f} + WRITE x "
                 f"{result['write_factor']:.4f}) | {e['bytes'] / 1e6:.1f} MB |")
    L += ["", "Bench line of the kernel-trace pass:", "", "    " + json.dumps(line)]
    with open(os.path.join(outdir, name), "w") as f:
        f.write("\n".join(x for x in L if x is not None) + "\n")


def cpu_baseline(oracle_sample, rows_total, target_s=12.0):
    """Times the oracle on a row sample sized for about target_s seconds."""
    import oracle
    cores = oracle.default_threads()
    rows = min(32, rows_total)
    t, fl = oracle_sample(rows)
    # Small samples under-use the threads, so the first estimate runs short:
    # grow the sample until it takes at least ~2/3 of the target.
    for _ in range(4):
        if t >= 0.66 * target_s or rows >= rows_total:
            break
        rows2 = int(min(rows_total, max(2 * rows, rows * target_s / max(t, 1e-3))))
        rows2 = max(cores, rows2 - rows2 % cores) if rows2 >= cores else rows2
        t, fl = oracle_sample(rows2)
        rows = rows2
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of {rows_total} output rows (all columns, full K), "
                      f"{t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="dense_8192",
                    help="dense_8192 (default), grouped, mxfp8, mxfp4, mxfp6, mxfp6_e3m2, "
                         "dense_1024, single_tile or copy (traffic calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prewarm", action="store_true",
                    help="time right after the --warmup launches, without running until "
                         "the launch time has settled")
    ap.add_argument("--layout", type=int, choices=[16, 8, 0], default=None,
                    help="run the dense workload through gemm_layout_run with this LDS "
                         "layout (16 = the library's XOR swizzle over 256-byte lines, "
                         "8 = over 128-byte lines, 0 = none) on the 256x256 ping-pong kernel")
    ap.add_argument("--layout-io", choices=["16,1", "16,0", "0,1", "0,0"], default=None,
                    help="run the dense workload through gemm_layout_io_run on the library's "
                         "256x256 kernel: operand layout (16 = XOR swizzle, 0 = none), then "
                         "the epilogue's C/D staging (1 = swizzled, 0 = not)")
    ap.add_argument("--layout128", choices=["16", "8", "0", "pad"], default=None,
                    help="the same through gemm_layout128_run on 128x128 tiles, where 'pad' "
                         "(rows padded by 16 bytes) also fits")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock-trace windows before and after the timed region and "
                         "the MFMA clock probe")
    ap.add_argument("--profile", metavar="OUTDIR", default=None,
                    help="run rocprofv3 passes (kernel trace, SQ counters, FETCH_SIZE, "
                         "WRITE_SIZE) over this bench for the --workload list (comma "
                         "separated; include 'copy' for the byte calibration) and write "
                         "summaries and counters.json to OUTDIR")
    args = ap.parse_args()
    if args.profile:
        layout_args = []
        for flag in ("layout", "layout_io", "layout128"):
            v = getattr(args, flag)
            if v is not None:
                layout_args += ["--" + flag.replace("_", "-"), str(v)]
        profile(args, layout_args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    log(f"[bench] workload {args.workload}: generating inputs")
    layout = None
    if args.layout is not None:
        layout = (256, args.layout)
    elif args.layout_io is not None:
        ops, outs = (int(x) for x in args.layout_io.split(","))
        layout = ("io", ops, outs)
    elif args.layout128 is not None:
        import dense_gemm_swizzled_amd as sg
        layout = (128, sg.SG_LAYOUT_PAD16 if args.layout128 == "pad" else int(args.layout128))
    run, flops, dtype, cfg, oracle_sample, rows_total = build_workload(args.workload, dev, layout)
    stream = torch.cuda.current_stream(dev)

    # The clock is traced over a window of launches right before the timed
    # region and one right after it (never inside): the clock drifts slowly,
    # and the two windows bracket the timed one.  Nothing between the prewarm,
    # the windows and the timed region leaves the GPU idle for longer than a
    # synchronisation.
    traced = flops > 0 and not args.no_clock
    if traced:
        win_before = ClockWindow(dev, CLOCK_LAUNCHES)
        win_after = ClockWindow(dev, CLOCK_LAUNCHES)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    pw_launches, pw_s, pw_ms = (0, 0.0, None) if args.no_prewarm else prewarm(run, stream)
    if traced:
        win_before.run(run)

    # Two HIP events on the launch stream (the library launches on torch's
    # current stream) bracket the K timed steps: their elapsed time over K is
    # the mean launch duration.  Events around every launch would add their
    # own commands between the kernels (measured: 9.8 -> 17.4 us per step at
    # 1024^3), so there are none inside the region.  The wall clock around
    # the same region gives the step time.
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        run()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if traced:
        win_after.run(run)
        torch.cuda.synchronize()
    log(f"[bench] prewarm: {pw_launches} more launches, {pw_s:.2f} s of GPU time, last "
        f"window {pw_ms} ms per launch")
    mean_ms = e_start.elapsed_time(e_end) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (mean_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    log(f"[bench] {cfg['workload']}: {ms_per_step:.4f} ms/step wall, kernel mean "
        f"{mean_ms:.4f} ms -> {achieved:.1f} TFLOP/s "
        f"({100 * achieved / peak:.1f}% of {peak} TFLOP/s)")

    clock, workgroups = None, 0
    if traced:
        ghz_before, _, span_before = win_before.result()
        ghz_after, workgroups, span_after = win_after.result()
        gemm_ghz = (None if ghz_after is None or ghz_before is None
                    else 0.5 * (ghz_before + ghz_after))
        probe_mfma, probe_ctr = probe_clock(dev)

        def r(x, n=4):
            return None if x is None else round(x, n)
        clock = {"gemm_ghz": r(gemm_ghz),
                 "gemm_ghz_before": r(ghz_before), "gemm_ghz_after": r(ghz_after),
                 "span_us_before": r(None if span_before is None else span_before * 1e6, 3),
                 "span_us_after": r(None if span_after is None else span_after * 1e6, 3),
                 "launches_before": CLOCK_LAUNCHES, "launches_after": CLOCK_LAUNCHES,
                 "workgroups": workgroups,
                 "probe_mfma_ghz": round(probe_mfma, 4),
                 "probe_counter_ghz": round(probe_ctr, 4), "spec_ghz": SPEC_GHZ}
        log(f"[bench] clock: {clock}")

    counters = measured_counters(profile_key(args.workload, layout))

    cpu = None
    if not args.no_cpu_baseline and oracle_sample is not None:
        log("[bench] timing the CPU oracle on a row sample")
        cpu = cpu_baseline(oracle_sample, rows_total)
        log(f"[bench] cpu oracle: {cpu}")

    out = {
        "metric": "GEMM TFLOP/s and % of bf16 MFMA peak at 8192^3 on 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": cfg,
        "pct_of_bf16_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": (counters or {}).get("bytes"),
                     "traffic_unit": "bytes per launch (HBM side)",
                     "kernel_ms_mean": round(mean_ms, 5)},
        "cpu_baseline": cpu,
        "prewarm_launches": pw_launches,
        "prewarm_s": round(pw_s, 3),
        "clock": clock,
    }
    if counters is not None:
        # From the committed rocprofv3 passes over this same code (bench.py
        # --profile): MFMA utilisation against the clock the kernel held, the
        # LDS bank-conflict cycles, and whether the MFMAs did exactly 2MNK.
        out["counters"] = {k: counters.get(k) for k in (
            "mfma_busy", "lds_bank_conflict_cycles", "lds_idx_active_cycles",
            "mops_x512_equals_2mnk", "kernel_ns", "clock_ghz")}
        out["counters"]["source"] = "profiles/counters.json"
    if clock is not None and clock["gemm_ghz"]:
        # The MFMA peak at the clock the kernel held (the published peak is
        # quoted at 2.4 GHz), and the fraction of it the kernel reached.  The
        # clock drifts between the windows, so each window's fraction takes
        # that window's own clock and launch span; the two are averaged.
        adj = peak * clock["gemm_ghz"] / SPEC_GHZ
        out["roofline"]["clock_adjusted_peak"] = round(adj, 1)
        fr = [flops / span / 1e12 / (peak * ghz / SPEC_GHZ)
              for ghz, span in ((ghz_before, span_before), (ghz_after, span_after))
              if ghz and span]
        if fr:
            out["roofline"]["frac_of_clock_adjusted_peak"] = round(sum(fr) / len(fr), 4)
    if args.workload == "grouped":
        # Per group the kernel can go no faster than its MFMA time or the HBM
        # time of its own bytes (A_g, B_g, D_g), whichever is longer.
        floor_s = 0.0
        for m in cfg["m_sizes"]:
            f_g = 2.0 * m * cfg["N"] * cfg["K"]
            b_g = 2.0 * (m * cfg["K"] + cfg["N"] * cfg["K"] + m * cfg["N"])
            floor_s += max(f_g / (peak * 1e12), b_g / (HBM_PEAK_GBS * 1e9))
        out["roofline"]["attainable_ms"] = round(floor_s * 1e3, 5)
        out["roofline"]["frac_of_attainable"] = round(floor_s * 1e3 / mean_ms, 4)
    if args.workload == "single_tile" and workgroups > 0:
        # A handful of workgroups, each on a CU of its own: the share of the
        # peak of the CUs the launch occupied.
        cu_peak = peak / 256 * workgroups
        out["roofline"]["occupied_cus"] = workgroups
        out["roofline"]["occupied_cu_peak"] = round(cu_peak, 3)
        out["roofline"]["frac_of_occupied_cus"] = round(achieved / cu_peak, 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
