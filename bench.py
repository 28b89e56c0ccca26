#!/usr/bin/env python3
"""Benchmark: attention forward TFLOP/s and fraction of the MFMA peak.

One step = one forward pass (attn_fwd) over the whole workload, inputs
already resident in HBM.  Default workload: bf16, causal, B=1, H=32,
S_q=S_k=16384, D_qk=D_v=128 (the headline configuration).

Prints ONE JSON line.  FLOPs per step follow the metric's count:
2*B*H*S_q*S_k*(D_qk+D_v), halved for causal.  `roofline.achieved` divides
that count (or, for an HBM-bound launch, its algorithmic bytes) by the
attention kernel's average launch duration: `steps` launches back to back
after the timed steps, between two HIP events recorded on the stream the
kernel runs on (torch's current stream, which is the stream the binding
passes to the library).  `cpu_baseline` times the fp64 CPU oracle on a
bounded row sample of the same workload.

Before the warm-up steps the step runs back to back for --settle-s seconds
(default 1): an idle MI355X starts at a low engine clock and needs tens of
launches of the headline size to reach the clock it holds under this load,
so a handful of warm-up steps alone leaves the ramp inside the timed steps.
The timed region is exactly --steps steps either way, with nothing else
enqueued between its launches; a second pass of the same steps, with a HIP
event before every launch, gives how a step divides between its launches
(`attn_ms_in_step`, and `merge_ms` for split-KV).

--power-s S (off by default) adds `power`: the GPU's socket power, its
power limit and the graphics clock, read in-process through amdsmi while
the step runs back to back for S seconds after the measurements.

--workload also selects the extended entry points' workloads (key offset,
sliding window, split-KV with its merge, grouped K/V heads); their FLOPs
count 2*(D_qk+D_v) per visible (query, key) pair, and a split-KV step is
the chunked attention launch followed by the merge launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X dense peaks (TFLOP/s) by compute dtype, and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "fp8_e4m3": 5033.2}
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "tiled_scaled_dot_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: headline)")
    ap.add_argument("--n-splits", type=int, default=None,
                    help="key chunks of a split-KV workload (default: the workload's)")
    ap.add_argument("--cpu-row-stride", type=int, default=2,
                    help="oracle sample: every N-th query row of every head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="before the warm-up steps, run the step back to back for this long "
                         "so that the engine clock has left its idle state")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run --steps launches of a plain device "
                         "copy of this many MiB (counter calibration for HBM traffic)")
    ap.add_argument("--gemm-probe", type=int, default=0, metavar="N",
                    help="instead of the benchmark, run --steps bf16 N x N x N matrix products "
                         "(torch.matmul, the platform's GEMM library) after the clock settle "
                         "and print their rate: the MFMA rate a plain dense contraction "
                         "sustains on this GPU, for comparison")
    ap.add_argument("--power-s", type=float, default=0.0,
                    help="after the timed steps (or the --gemm-probe launches), run the step back "
                         "to back for this many seconds while a thread reads the GPU's socket "
                         "power, power limit and graphics clock in-process (amdsmi) every 10 ms; "
                         "report their means as `power` (off by default)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("ATTN_FETCH", "ATTN_WRITE",
                                                          "COPY_FETCH", "COPY_WRITE"),
                    help="write the HBM traffic per launch into the stored traffic record "
                         "from four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of this benchmark, then of --copy-probe-mib)")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size the --copy-probe-mib run used (for --record-traffic)")
    ap.add_argument("--counter-summary", metavar="FOLDER",
                    help="instead of the benchmark, summarise a rocprofv3 --pmc folder: per "
                         "kernel, the shader clock from GRBM_COUNT, the MFMA pipe's busy "
                         "fraction and the rate against the peak at that clock")
    ap.add_argument("--skip-dispatches", type=int, default=0,
                    help="--counter-summary: leave out the first N dispatches (clock ramp)")
    ap.add_argument("--trace-summary", metavar="FOLDER",
                    help="instead of the benchmark, summarise a rocprofv3 --kernel-trace folder: "
                         "per kernel, the dispatch count and the mean duration over all "
                         "dispatches and over the last --last (the back-to-back block)")
    ap.add_argument("--last", type=int, default=50,
                    help="--trace-summary: dispatches at the end of the trace to average")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel source with comments and blank space
    removed, so that a traffic record survives edits of comments only."""
    import re

    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def copy_probe(mib: int, launches: int) -> int:
    """Launch a plain strided device copy of `mib` MiB `launches` times.

    The source is the left half of a wider f32 matrix, so the copy runs as an
    element-wise kernel (a contiguous copy would go to the DMA engines): it
    reads exactly `mib` MiB and writes `mib` MiB, rows aligned to 256 bytes.
    Its FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    import torch

    cols = 16384
    rows = mib * (1 << 20) // (4 * cols)
    dev = torch.device("cuda:0")
    src = torch.empty((rows, 2 * cols), dtype=torch.float32, device=dev)
    dst = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    for _ in range(launches):
        dst.copy_(src[:, :cols])
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": rows * cols * 4, "launches": launches}), flush=True)
    return 0


class PowerReader:
    """Socket power and graphics clock of the GPU torch uses as cuda:0, read
    in-process through amdsmi (no child process) by a thread every 10 ms
    while `run(step, seconds)` launches the step back to back.  The first
    quarter of the samples (the ramp) is left out of the means."""

    def __init__(self):
        import amdsmi
        import torch

        self.smi = amdsmi
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        handles = amdsmi.amdsmi_get_processor_handles()
        self.h = handles[0]
        for h in handles:
            if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                self.h = h
        self.bdf = amdsmi.amdsmi_get_gpu_device_bdf(self.h)

    def run(self, step, seconds: float) -> dict:
        import threading

        import torch

        smi, samples, stop = self.smi, [], threading.Event()

        def sample():
            while not stop.is_set():
                p = smi.amdsmi_get_power_info(self.h)
                c = smi.amdsmi_get_clock_info(self.h, smi.AmdSmiClkType.GFX)
                samples.append((float(p["current_socket_power"]), float(p["power_limit"]) / 1e6,
                                float(c["clk"])))
                time.sleep(0.01)

        th = threading.Thread(target=sample, daemon=True)
        t0 = time.perf_counter()
        launches = 0
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                step()
            launches += 4
            torch.cuda.synchronize()
        stop.set()
        th.join()
        kept = samples[len(samples) // 4:]
        if not kept:
            return {"error": "no samples"}
        mean = lambda i: sum(x[i] for x in kept) / len(kept)
        return {"socket_w_mean": round(mean(0), 1), "socket_w_max": max(x[0] for x in kept),
                "power_limit_w": round(kept[-1][1], 1), "gfx_mhz_mean": round(mean(2), 1),
                "samples": len(kept), "seconds": round(time.perf_counter() - t0, 2),
                "launches": launches, "device_bdf": self.bdf, "source": "amdsmi, in-process"}


def power_reading(step, seconds: float) -> dict:
    """PowerReader().run(step, seconds), or the reason it could not run."""
    try:
        return PowerReader().run(step, seconds)
    except Exception as e:   # amdsmi missing or not permitted here
        return {"error": f"{type(e).__name__}: {e}"}


def gemm_probe(n: int, launches: int, settle_s: float, power_s: float = 0.0) -> int:
    """Time `launches` bf16 n x n x n products C = A B (torch.matmul, which
    calls the platform GEMM library) back to back between two events, after
    running them for `settle_s` seconds; print the rate and its fraction of
    the dense bf16 peak."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    a = torch.randn((n, n), generator=g).to(dev, torch.bfloat16)
    b = torch.randn((n, n), generator=g).to(dev, torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    out = {"gemm_probe": f"bf16 {n}x{n}x{n}", "launches": launches, "ms": round(ms, 4),
           "tflops": round(tflops, 1),
           "frac_of_dense_bf16_peak": round(tflops / PEAK_TFLOPS["bf16"], 4)}
    if power_s > 0:
        out["power"] = power_reading(lambda: torch.matmul(a, b, out=c), power_s)
    print(json.dumps(out), flush=True)
    return 0


def pmc_per_dispatch(folder: str, counter: str, name_filter) -> float:
    """Mean of one counter over the dispatches whose kernel name passes the
    filter, from a rocprofv3 --pmc --output-format csv folder (KiB for the
    *_SIZE counters)."""
    import csv
    import glob

    vals = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and name_filter(row["Kernel_Name"]):
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows in {folder}")
    return sum(vals) / len(vals)


def record_traffic(args) -> int:
    """Scale the attention kernel's FETCH_SIZE and WRITE_SIZE by what the same
    counters read for the copy probe (bytes known exactly) and store the
    result, keyed by workload and kernel source hash."""
    from tiled_scaled_dot_amd.workloads import ALL_WORKLOADS, HEADLINE

    name = args.workload or HEADLINE
    w = ALL_WORKLOADS[name]
    a_fetch, a_write, c_fetch, c_write = args.record_traffic
    is_attn = lambda k: "attn_fwd" in k
    is_copy = lambda k: "attn_fwd" not in k
    copy_bytes = (args.copy_mib << 20) // (4 * 16384) * 16384 * 4
    fetch_kib = pmc_per_dispatch(a_fetch, "FETCH_SIZE", is_attn)
    write_kib = pmc_per_dispatch(a_write, "WRITE_SIZE", is_attn)
    cf_kib = pmc_per_dispatch(c_fetch, "FETCH_SIZE", is_copy)
    cw_kib = pmc_per_dispatch(c_write, "WRITE_SIZE", is_copy)
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[name] = {
        "kernel_source_sha256_16": kernel_source_hash(),
        "hbm_bytes_per_launch": round(read_b + write_b),
        "read_bytes": round(read_b),
        "write_bytes": round(write_b),
        "min_bytes_of_step": w.min_bytes(),
        "fetch_size_kib": fetch_kib,
        "write_size_kib": write_kib,
        "copy_probe_bytes": copy_bytes,
        "copy_fetch_size_kib": cf_kib,
        "copy_write_size_kib": cw_kib,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec[name]))
    return 0


def counter_summary(folder: str, skip: int = 0) -> int:
    """Per kernel of a rocprofv3 --pmc folder (csv output), averaged over the
    dispatches after the first `skip`:
      clock_mhz        GRBM_COUNT / XCDs / duration: GRBM_COUNT counts the
                       engine clock on every XCD and rocprofv3 sums the XCDs
      gui_active       GRBM_GUI_ACTIVE / GRBM_COUNT (busy fraction)
      mfma_busy        SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x clock cycles)
      sq_busy          SQ_BUSY_CYCLES / (shader arrays x clock cycles)
      mfma_tflops      SQ_INSTS_VALU_MFMA_MOPS_<dtype> x 512 FLOP / duration
      pct_peak_at_clock  that rate against the dense peak of the dtype at
                       the measured clock (peak x clock / 2400 MHz)
    Counters missing from the folder leave their fields out."""
    import csv
    import glob

    agent = {}
    for path in glob.glob(os.path.join(folder, "**", "*agent_info.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Agent_Type") == "GPU":
                    agent = row
    xcc = int(agent.get("Num_Xcc", 8))
    simds = int(agent.get("Simd_Count", 1024))
    arrays = int(agent.get("Array_Count", 32))
    disp = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                d = disp.setdefault(int(row["Dispatch_Id"]), {
                    "kernel": row["Kernel_Name"],
                    "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
                d[row["Counter_Name"]] = float(row["Counter_Value"])
    if not disp:
        raise SystemExit(f"no counter rows in {folder}")
    out = {}
    for did in sorted(disp)[skip:]:
        d = disp[did]
        out.setdefault(d["kernel"], []).append(d)
    mops_peak = {"BF16": PEAK_TFLOPS["bf16"], "F16": PEAK_TFLOPS["f16"],
                 "F8": PEAK_TFLOPS["fp8_e4m3"], "F32": PEAK_TFLOPS["f32"]}
    result = {}
    for kernel, ds in out.items():
        ns = sum(d["ns"] for d in ds) / len(ds)
        r = {"dispatches": len(ds), "mean_ns": round(ns)}

        def mean(counter):
            vals = [d[counter] for d in ds if counter in d]
            return sum(vals) / len(vals) if vals else None

        cnt = mean("GRBM_COUNT")
        if cnt:
            mhz = cnt / xcc / ns * 1e3
            cycles = cnt / xcc
            r["clock_mhz"] = round(mhz, 1)
            if mean("GRBM_GUI_ACTIVE") is not None:
                r["gui_active"] = round(mean("GRBM_GUI_ACTIVE") / cnt, 4)
            if mean("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
                r["mfma_busy"] = round(mean("SQ_VALU_MFMA_BUSY_CYCLES") / (simds * cycles), 4)
            if mean("SQ_BUSY_CYCLES") is not None:
                r["sq_busy"] = round(mean("SQ_BUSY_CYCLES") / (arrays * cycles), 4)
        for tag, peak in mops_peak.items():
            mops = mean(f"SQ_INSTS_VALU_MFMA_MOPS_{tag}")
            if mops:
                tf = mops * 512.0 / (ns * 1e-9) / 1e12
                r[f"mfma_tflops_{tag.lower()}"] = round(tf, 1)
                r[f"pct_of_{tag.lower()}_peak"] = round(100.0 * tf / peak, 2)
                if cnt:
                    r[f"pct_of_{tag.lower()}_peak_at_clock"] = round(
                        100.0 * tf / (peak * r["clock_mhz"] / 2400.0), 2)
        result[kernel] = r
    print(json.dumps(result, indent=1))
    return 0


def trace_summary(folder: str, last: int) -> int:
    """Per kernel of a rocprofv3 --kernel-trace folder (csv output): the
    dispatch count, mean / min / max duration over all dispatches, and the
    mean over the last `last` dispatches, which for a bench.py run are the
    back-to-back block it times for the roofline."""
    import csv
    import glob

    per = {}
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                per.setdefault(row["Kernel_Name"], []).append(
                    (int(row["Start_Timestamp"]), int(row["End_Timestamp"]) - int(row["Start_Timestamp"]),
                     int(row.get("Grid_Size_X", row.get("Grid_Size", 0)) or 0),
                     int(row.get("Workgroup_Size_X", row.get("Workgroup_Size", 0)) or 0)))
    if not per:
        raise SystemExit(f"no kernel trace rows in {folder}")
    result = {}
    for kernel, ds in per.items():
        ds.sort()
        ns = [d[1] for d in ds]
        tail = ns[-last:] if last > 0 else ns
        result[kernel] = {"dispatches": len(ns), "mean_ns": round(sum(ns) / len(ns)),
                          "min_ns": min(ns), "max_ns": max(ns),
                          f"mean_ns_last_{len(tail)}": round(sum(tail) / len(tail)),
                          "workgroups": ds[0][2] // max(ds[0][3], 1), "threads": ds[0][3]}
    print(json.dumps(result, indent=1))
    return 0


def cpu_baseline(w, q, k, v, stride: int, scales=None):
    import numpy as np

    import oracle

    rows = list(range(stride - 1, w.S_q, stride)) or [0]
    qd = q.double().numpy()
    kd = k.double().numpy()
    vd = v.double().numpy()
    threads = oracle.default_threads()
    ext = getattr(w, "entry", "fwd") in ("ext", "splitkv")
    t0 = time.perf_counter()
    if scales is not None:
        oracle.attn_ref_scaled(qd, kd, vd, scales[0].double().numpy(),
                               scales[1].double().numpy(), w.q_block, w.k_block, w.causal,
                               rows=rows, nthreads=threads)
    elif ext:
        oracle.attn_ref_ext(qd, kd, vd, w.scale, w.causal, causal_offset=w.causal_offset,
                            window=w.window, rows=rows, nthreads=threads)
    else:
        oracle.attn_ref(qd, kd, vd, w.scale, w.causal, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    if ext:
        lo, hi = w.row_ranges()
        pairs = int(sum(hi[r] - lo[r] for r in rows)) * w.B * w.H
    else:
        pairs = sum((min(r + 1, w.S_k) if w.causal else w.S_k) for r in rows) * w.B * w.H
    flops = 2.0 * pairs * (w.D_qk + w.D_v)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"query rows i = {rows[0] % stride} mod {stride} of all {w.B * w.H} slices "
                   f"({len(rows)} rows/slice, {flops / 1e9:.1f} GFLOP of visible pairs, "
                   f"{dt:.1f} s, fp64, {cpu_model or platform.processor()})"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards per (batch, head) slice with no exchange, but no multi-GPU "
              "run is part of it.", file=sys.stderr)
        return 2

    if args.record_traffic:
        return record_traffic(args)
    if args.counter_summary:
        return counter_summary(args.counter_summary, args.skip_dispatches)
    if args.trace_summary:
        return trace_summary(args.trace_summary, args.last)
    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib, args.steps)
    if args.gemm_probe:
        return gemm_probe(args.gemm_probe, args.steps, args.settle_s, args.power_s)

    import torch

    import tiled_scaled_dot_amd as tsd
    from tiled_scaled_dot_amd.workloads import ALL_WORKLOADS, HEADLINE, make_inputs

    name = args.workload or HEADLINE
    w = ALL_WORKLOADS[name]
    entry = getattr(w, "entry", "fwd")
    if args.n_splits is not None:
        if getattr(w, "entry", "fwd") != "splitkv":
            raise SystemExit("--n-splits applies to split-KV workloads only")
        w = w.with_(n_splits=args.n_splits)
    dev = torch.device("cuda:0")
    if entry == "scaled":
        from tiled_scaled_dot_amd.workloads import scaled_inputs

        q, k, v, q_sc, k_sc = scaled_inputs(w.B, w.H, w.S_q, w.S_k, w.D_qk, w.D_v, w.q_block,
                                            w.k_block, w.qk_dtype, w.dtype, w.seed)
        qsd, ksd = q_sc.to(dev), k_sc.to(dev)
    else:
        q, k, v = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty(w.shape_o, dtype=vd.dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.S_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = w.metric_flops()
    min_bytes = w.min_bytes()
    extra = {}

    # A step is a list of launches; the first is the attention kernel (the
    # dominant one, the roofline's subject), with its algorithmic FLOPs and
    # bytes per launch.
    if entry == "fwd":
        phases = [lambda: tsd.attn_fwd(qd, kd, vd, scale=w.scale, causal=w.causal, out=o,
                                       lse=lse, stream=stream)]
        attn_bytes = min_bytes
    elif entry == "scaled":
        phases = [lambda: tsd.attn_fwd_scaled(qd, kd, vd, qsd, ksd, w.q_block, w.k_block,
                                              causal=w.causal, out=o, lse=lse, stream=stream)]
        attn_bytes = min_bytes
    elif entry == "ext":
        phases = [lambda: tsd.attn_fwd_ext(qd, kd, vd, scale=w.scale, causal=w.causal,
                                           causal_offset=w.causal_offset, window=w.window,
                                           out=o, lse=lse, stream=stream)]
        attn_bytes = min_bytes
    else:   # splitkv: partial results over key chunks, then the merge
        mask = tsd.make_mask(w.S_k, w.causal_offset, w.window)
        n, split_len, _ = tsd.attn_splitkv_plan(w.B, w.H, w.S_q, w.S_k, w.D_qk, w.D_v,
                                                w.causal, w.dtype, mask, w.n_splits,
                                                H_kv=w.kv_heads)
        o_parts = torch.empty((n, w.B, w.H, w.S_q, w.D_v), dtype=torch.float32, device=dev)
        l_parts = torch.empty((n, w.B, w.H, w.S_q), dtype=torch.float32, device=dev)
        phases = [
            lambda: tsd.attn_fwd_partial(qd, kd, vd, n, split_len, scale=w.scale,
                                         causal=w.causal, causal_offset=w.causal_offset,
                                         window=w.window, o_parts=o_parts,
                                         lse_parts=l_parts, stream=stream),
            lambda: tsd.attn_merge(o_parts, l_parts, dtype=qd.dtype, out=o, lse=lse,
                                   stream=stream),
        ]
        rows = w.B * w.H * w.S_q
        elt = qd.element_size()
        part_bytes = n * rows * (w.D_v * 4 + 4)
        # each chunk reads Q again and writes f32 partials instead of O
        attn_bytes = (min_bytes - rows * (w.D_v * elt + 4) + (n - 1) * rows * w.D_qk * elt
                      + part_bytes)
        extra = {"n_splits": n, "split_len": split_len,
                 "merge_bytes_per_launch": part_bytes + rows * (w.D_v * elt + 4)}

    def step():
        for ph in phases:
            ph()

    # Clock settle: an idle GPU starts at a low engine clock and needs tens
    # of launches of this size to reach the clock it holds under load.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(4):
            step()
        settle_steps += 4
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps: nothing but the launches between the two
    # synchronisations (an event recorded between launches is a marker
    # packet of its own, which would count in the step time).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The same steps again with events before every launch and after the
    # last: how the step divides between its launches.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
          for _ in range(args.steps)]
    for i in range(args.steps):
        for j, ph in enumerate(phases):
            ev[i][j].record(stream)
            ph()
        ev[i][-1].record(stream)
    torch.cuda.synchronize()
    launch_ms = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / args.steps
                 for j in range(len(phases))]
    # The attention launch alone, `steps` times back to back between two
    # events: the per-launch events above also count each launch's dispatch
    # gap, which is not small next to a launch of tens of microseconds.
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.steps):
        phases[0]()
    a1.record(stream)
    torch.cuda.synchronize()
    kernel_ms = a0.elapsed_time(a1) / args.steps
    extra["attn_ms_in_step"] = round(launch_ms[0], 4)
    power = power_reading(step, args.power_s) if args.power_s > 0 else None

    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if entry == "scaled" and w.qk_dtype != w.dtype:
        # Q K^T at the Q/K dtype's peak, P V at V's: the peak of the mix
        f_qk, f_pv = w.D_qk / (w.D_qk + w.D_v), w.D_v / (w.D_qk + w.D_v)
        peak = round(1.0 / (f_qk / PEAK_TFLOPS[w.qk_dtype] + f_pv / PEAK_TFLOPS[w.dtype]), 1)
    traffic = stored_traffic(name)
    # Roofline of the attention launch: MFMA when its FLOPs per algorithmic
    # byte exceed the ridge (peak / HBM bandwidth), else HBM.
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / attn_bytes >= ridge:
        bound, unit, roof_peak = "mfma", "TFLOP/s", peak
        achieved = flops / (kernel_ms * 1e-3) / 1e12
    else:
        bound, unit, roof_peak = "hbm", "GB/s", PEAK_HBM_GBS
        achieved = attn_bytes / (kernel_ms * 1e-3) / 1e9
    if len(phases) > 1:
        extra["merge_ms"] = round(launch_ms[1], 4)
        extra["merge_gbs"] = round(extra["merge_bytes_per_launch"] / (launch_ms[1] * 1e-3) / 1e9,
                                   1)
    if entry == "scaled":
        extra.update(entry=entry, qk_dtype=w.qk_dtype, q_block=w.q_block, k_block=w.k_block,
                     mfma_peak_of_the_mix=peak)
    elif entry != "fwd":
        extra.update(entry=entry, H_kv=w.kv_heads, causal_offset=w.causal_offset,
                     window=w.window, visible_pairs_per_slice=w.visible_pairs())

    result = {
        "metric": ("attention fwd TFLOP/s and % of MFMA peak (bf16 causal, S=16k, D=128)"
                   if entry == "fwd" else
                   "attention fwd TFLOP/s, per-block scaled (metric FLOP count)"
                   if entry == "scaled" else
                   "attention fwd TFLOP/s over visible (query, key) pairs"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{w.qk_dtype}+{w.dtype}" if entry == "scaled" and w.qk_dtype != w.dtype
                  else w.dtype),
        "data": "synthetic",
        "config": {
            "workload": name,
            "B": w.B, "H": w.H, "S_q": w.S_q, "S_k": w.S_k, "D_qk": w.D_qk, "D_v": w.D_v,
            "causal": w.causal, "scale": w.scale,
            "inputs": (f"{w.dist} Q,K sigma={w.sigma_qk:.4g}, V sigma={w.sigma_v:.4g}, "
                       f"seed {w.seed}" if w.dist == "normal" else f"{w.dist}(-1,1), seed {w.seed}"),
            "flops_per_step": flops,
            "pct_of_mfma_peak": round(100.0 * (flops / (kernel_ms * 1e-3) / 1e12) / peak, 2),
            "settle_s": round(settle_s, 2),
            "settle_steps": settle_steps,
            "min_bytes_per_step": min_bytes,
            "attn_bytes_per_launch": attn_bytes,
            **extra,
            "device": torch.cuda.get_device_name(dev),
            "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
        },
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": roof_peak,
            "unit": unit,
            "frac": round(achieved / roof_peak, 4),
            "traffic": traffic,
            "kernel_ms": round(kernel_ms, 4),
        },
        "cpu_baseline": None,
    }
    if power is not None:
        result["power"] = power
    if not args.no_cpu_baseline:
        del qd, kd, vd, o, lse
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_row_stride,
                                              (q_sc, k_sc) if entry == "scaled" else None)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
