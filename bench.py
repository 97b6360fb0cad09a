"""Benchmark of the quantization hot path on one MI355X.

A step is one pass of the whole path over the 7B-shaped linear stack (32
layers x q, k, v, o, gate, up, down = 224 matrices, 6,476,005,376 fp32
weights resident in HBM): quantize and pack every matrix to int4 with group
32 (qw_quantize_pack_batched, all 224 matrices in one launch), then one M = 1
dequantizing GEMV through every matrix (qw_gemv_batched, one launch, the
codes unpacked in registers).  `value` is the step's algorithmic HBM bytes
divided by the step time.

In the same run the single-matrix decode GEMVs (4096 x 4096 int8 with one
scale per output channel at M = 1; the 7B MLP up and down matrices at int4
group 128 for M = 1, 4, 8) are timed over rotating weight copies and
reported under "decode_gemv_configs"; the prefill GEMM (qw_gemm: 2048 tokens through a 70B-style
MLP weight of 28672 x 8192, int4 group 128, bf16 matrix cores) is timed on
its own and reported under "prefill_gemm", and the CPU oracle is timed on a
bounded sample of the stack under "cpu_baseline".

The GPTQ leg ("gptq") quantizes one layer of the small model of the GPTQ
section of "Huit bits, puis quatre" (width 512, feed-forward 1368) from
synthetic calibration inputs of 65,536 tokens in 8 batches: per input the
accumulation of H (qw_gptq_hessian), the factor (qw_gptq_factor) and the
codes of every map reading that input (qw_gptq_quantize_pack).  Its value
is weights per second over the layer with the four inputs' chains on four
streams; its roofline is the fp64 MFMA accumulation of H for the
1368-input map; the oracle runs the same layer on one core.  `--only-gptq`
runs that leg alone (for profiling).

Prints ONE JSON line.  `--gpus N` with N > 1 exits: the library and this
benchmark run on one GPU.

HBM traffic ("roofline.traffic"): two rocprofv3 counter runs of this script
with `--calib-copy-mib 1024` (FETCH_SIZE, then WRITE_SIZE) are reduced by
`--pmc-summary FETCH_DIR WRITE_DIR` into profiles/pmc_traffic_c4_c5_gptq_layer.md; each
counter is scaled by what it reads for a plain device copy of known size.
The benchmark reports a kernel's traffic only while its source file (and the
shared internal header) still hash to the values recorded there (null
otherwise).
"""

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int4/int8 dequant-GEMV weight GB/s (% HBM peak); prefill GEMM TFLOPS"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ClockSampler:
    """Samples the GPU's graphics clock (each XCD's current value, averaged)
    and its socket power through amdsmi in a background thread, and reports
    their medians over the samples taken after the first `skip_s` seconds.
    The device refreshes these figures every few tens of milliseconds, so
    they describe a sustained load, not a single short kernel.  Reports None
    where amdsmi is missing or returns nothing."""

    def __init__(self, enabled=True, interval_s=0.005, skip_s=0.4):
        self.enabled, self.interval, self.skip = enabled, interval_s, skip_s
        self.samples = []   # (seconds since start, MHz or None, W or None)
        self._stop = None

    def __enter__(self):
        if not self.enabled:
            return self
        try:
            import threading
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as exc:  # no amdsmi, no device: no clock figure
            log(f"clock sampling off: {exc}")
            self.enabled = False
            return self
        self._stop = threading.Event()
        t0 = time.perf_counter()

        def run():
            while not self._stop.is_set():
                try:
                    m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                    clks = [c for c in m.get("current_gfxclks", [])
                            if isinstance(c, int) and 0 < c < 65535]
                    pw = m.get("current_socket_power")
                    self.samples.append((time.perf_counter() - t0,
                                         sum(clks) / len(clks) if clks else None,
                                         pw if isinstance(pw, (int, float)) else None))
                except Exception:
                    pass
                self._stop.wait(self.interval)

        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        if self._stop is not None:
            self._stop.set()
            self._t.join()
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self):
        kept = [(c, w) for t, c, w in self.samples if t >= self.skip]
        c = [v for v, _ in kept if v is not None]
        w = [v for _, v in kept if v is not None]
        if not c:
            return None
        return {"gfx_mhz_median": round(statistics.median(c)), "gfx_mhz_min": round(min(c)),
                "gfx_mhz_max": round(max(c)),
                "socket_w_median": round(statistics.median(w)) if w else None,
                "samples": len(c),
                "source": "amdsmi current_gfxclks (mean over XCDs) and current_socket_power"}


def sustained_clock(args, fn, seconds=3.0):
    """Clock and power while `fn` (one enqueue of the timed work) runs back to
    back for `seconds`, after the timed region and outside it."""
    import torch
    if args.no_clock:
        return None
    with ClockSampler(skip_s=1.5) as c:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
    return c.summary()


def prewarm(args, fn):
    """Runs `fn` (one enqueue of the timed work) back to back, untimed, for
    --prewarm-s seconds.  From idle, the GPU's clock and power controller
    overshoots for the first few milliseconds to a quarter second of load
    (launch durations up to 30% above their sustained value); the timed
    region that follows then sees the sustained state."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.prewarm_s:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--gemm-reps", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed back-to-back runs before each leg's warm-up "
                         "(0: time from a cold start)")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=32, help="layers of the stack (default: all 32)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB on the device "
                         "(the known-size kernel that calibrates the HBM byte counters)")
    ap.add_argument("--pmc-table", nargs="+", metavar="DIR",
                    help="print the activity-counter table of rocprofv3 --pmc CSV runs and exit")
    ap.add_argument("--trace-table", metavar="DIR",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace CSV run and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--no-gptq", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context legs (device copy and read, torch.matmul bf16)")
    ap.add_argument("--only-gptq", action="store_true",
                    help="run only the GPTQ leg and print its JSON object (for profiling)")
    ap.add_argument("--gptq-reps", type=int, default=3)
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the GPU clock and power during the timed regions")
    ap.add_argument("--cpu-protocol", metavar="OUT_MD",
                    help="run only the oracle timing protocol in full (the page's 20 warm-ups + "
                         "101 reps on c1-c3, the whole stack and the whole GEMM, both modes); "
                         "write its table to OUT_MD and print the JSON")
    ap.add_argument("--cpu-worker", help=argparse.SUPPRESS)
    ap.add_argument("--gptq-cpu-sample-worker", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


# ------------------------------------------------------- HBM traffic (PMC)

CSRC = os.path.join(ROOT, "int8_int4_dequant_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_c4_c5_gptq_layer.md")
# kernel-name fragment -> (label, source file whose hash pins the measurement,
# grid size in threads or None): the benchmark's own launches -- the c5 GEMM is
# the 262144-thread grid of gemm_kernel<4> (the M sweep launches it too), the
# decode pass the 5439488-thread grid of gemv8_kernel<4, 1, 16, 256>
PMC_KERNELS = {
    "quant_subgroup_batched_kernel": ("quantize_pack_batched", "quantize.hip", None),
    # the whole-stack pass (the chained pass launches the same kernel per stage)
    "gemv8_kernel<4, 1, 16, 256>": ("gemv_batched_m1", "gemv.hip", 5439488),
    "gemm_kernel<4>": ("gemm", "gemm.hip", 262144),
    # the GPTQ leg's H accumulation over the 1368-input map (the only launch
    # of the 128-wide fp32-operand shape)
    "gemm64_kernel<float, float, 4": ("gptq_hessian_k1368", "gptq.hip", None),
}
COPY_KERNEL = "neg_kernel"  # the calibration copy (torch.neg over a known-size buffer)


def source_hashes():
    import hashlib
    out = {}
    for f in sorted({v[1] for v in PMC_KERNELS.values()} | {"qw_internal.h"}):
        with open(os.path.join(CSRC, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()[:16]
    return out


def pmc_means(d, counter):
    """Mean counter value (KiB per dispatch) per kernel-name fragment."""
    import csv
    import glob
    sums, cnt = {}, {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            for frag in list(PMC_KERNELS) + [COPY_KERNEL]:
                grid = PMC_KERNELS[frag][2] if frag in PMC_KERNELS else None
                if grid is not None and int(r["Grid_Size"]) != grid:
                    continue
                if frag in r["Kernel_Name"]:
                    sums[frag] = sums.get(frag, 0.0) + float(r["Counter_Value"])
                    cnt[frag] = cnt.get(frag, 0) + 1
    return {k: sums[k] / cnt[k] for k in sums}, cnt


def pmc_summary(fetch_dir, write_dir, copy_mib):
    f, fc = pmc_means(fetch_dir, "FETCH_SIZE")
    w, wc = pmc_means(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    ff = copy_kib / f[COPY_KERNEL]   # true KiB per counted KiB
    wf = copy_kib / w[COPY_KERNEL]
    kernels = {}
    for frag, (label, _, _) in PMC_KERNELS.items():
        if frag in f and frag in w:
            kernels[label] = {"fetch_kib_raw": round(f[frag], 1), "write_kib_raw": round(w[frag], 1),
                              "dispatches": [fc[frag], wc[frag]],
                              "traffic_bytes": round((f[frag] * ff + w[frag] * wf) * 1024)}
    return {"copy_mib": copy_mib, "copy_fetch_kib_raw": round(f[COPY_KERNEL], 1),
            "copy_write_kib_raw": round(w[COPY_KERNEL], 1),
            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
            "kernels": kernels, "source_sha256": source_hashes()}


# Launches whose activity counters `--pmc-table` reports: (label, kernel-name
# fragment, grid size in threads or None).
PMC_TABLE_KERNELS = [
    ("c4 decode pass (qw_gemv_batched, M=1, 224 matrices)", "gemv8_kernel<4, 1, 16, 256>",
     21248 * 256),
    ("c3 up 11008x4096 M=1 (qw_gemv)", "gemv8_split_kernel<4, 1, 4, 1>", 2752 * 256),
    ("c3 up 11008x4096 M=4 (matrix cores)", "gemv_mfma_kernel<4, 4, 1, 8, 2, 1>",
     688 * 512),
    ("c3 down 4096x11008 M=4 (matrix cores)", "gemv_mfma_kernel<4, 4, 1, 16, 2, 1>",
     256 * 1024),
    ("c3 up 11008x4096 M=8 (matrix cores)", "gemv_mfma_kernel<4, 8, 1, 8, 2, 1>", 688 * 512),
    ("c3 down 4096x11008 M=8 (matrix cores)", "gemv_mfma_kernel<4, 8, 1, 16, 2, 1>",
     256 * 1024),
    ("c4 decode pass at M=8 (qw_gemv_batched, matrix cores, groups of 32)",
     "gemv_mfma_batched_kernel<4, 8, 2, 4, 2, 4, 256>", None),
    ("c5 prefill GEMM 2048x28672x8192", "gemm_kernel<4>", 262144),
    ("c4 quantize pass (qw_quantize_pack_batched)", "quant_subgroup_batched_kernel<4, 8>", None),
]
SIMDS = 1024   # 256 compute units x 4
XCDS = 8


def pmc_table(dirs):
    """Markdown table of the activity counters of PMC_TABLE_KERNELS from
    rocprofv3 --pmc CSV runs (one counter set per directory): the mean per
    dispatch of each counter, and derived ratios."""
    import csv
    import glob
    vals = {}   # label -> counter -> [values]
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                for label, frag, grid in PMC_TABLE_KERNELS:
                    if frag in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid):
                        vals.setdefault(label, {}).setdefault(r["Counter_Name"], []).append(
                            float(r["Counter_Value"]))
    mean = {lb: {c: sum(v) / len(v) for c, v in cs.items()} for lb, cs in vals.items()}
    counters = sorted({c for cs in mean.values() for c in cs})
    labels = [lb for lb, _, _ in PMC_TABLE_KERNELS if lb in mean]
    lines = ["| counter (mean per dispatch) | " + " | ".join(labels) + " |",
             "|---|" + "---:|" * len(labels)]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(
            f"{mean[lb][c]:,.0f}" if c in mean[lb] else "" for lb in labels) + " |")

    def ratio(lb, a, b, scale=1.0):
        m = mean[lb]
        return f"{scale * m[a] / m[b]:.3f}" if a in m and b in m and m[b] else ""
    derived = [
        ("VALU instructions issued per SIMD per cycle (SQ_INSTS_VALU / (GRBM_GUI_ACTIVE / 8 "
         "XCDs) / 1024 SIMDs)", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE", XCDS / SIMDS),
        ("share of wave cycles issuing VALU (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES)",
         "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", 1.0),
        ("share of wave cycles waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", "SQ_WAIT_ANY",
         "SQ_WAVE_CYCLES", 1.0),
        ("share of wave cycles waiting on an instruction (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
         "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", 1.0),
        ("resident waves per SIMD (SQ_WAVE_CYCLES / (GRBM_GUI_ACTIVE / 8) / 1024)",
         "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE", XCDS / SIMDS),
        ("matrix-core busy share of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
         "8) / 1024)", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", XCDS / SIMDS),
        ("vector memory instructions per wave (SQ_INSTS_VMEM_RD / SQ_WAVES)", "SQ_INSTS_VMEM_RD",
         "SQ_WAVES", 1.0),
        ("mean vector memory instructions in flight per wave (SQ_INST_LEVEL_VMEM / "
         "SQ_WAVE_CYCLES)", "SQ_INST_LEVEL_VMEM", "SQ_WAVE_CYCLES", 1.0),
        ("L2 hit share (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum))", "TCC_HIT_sum",
         "TCC_REQ_EST", 1.0),
        ("mean L1->L2 read latency, cycles (TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum)",
         "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", 1.0),
    ]
    for m in mean.values():
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
            m["TCC_REQ_EST"] = m["TCC_HIT_sum"] + m["TCC_MISS_sum"]
    lines += ["", "| derived | " + " | ".join(labels) + " |", "|---|" + "---:|" * len(labels)]
    for name, a, b, sc in derived:
        lines.append(f"| {name} | " + " | ".join(ratio(lb, a, b, sc) for lb in labels) + " |")
    n = {lb: max(len(v) for v in vals[lb].values()) for lb in labels}
    lines += ["", "Dispatches averaged: " + ", ".join(f"{lb}: {n[lb]}" for lb in labels) + "."]
    return "\n".join(lines)


def trace_table(d, top=40):
    """Markdown table of a rocprofv3 --kernel-trace CSV run: one row per
    (kernel, grid, block) with call count and duration statistics in
    microseconds, and the register, LDS and scratch figures the trace records,
    sorted by total time."""
    import csv
    import glob

    def num(r, *names):
        for n in names:
            if r.get(n) not in (None, ""):
                return int(float(r[n]))
        return 0
    def short(name):
        # drop the trailing parameter list, the return type and the library's
        # own namespace
        name = name.strip()
        if name.endswith(")"):
            depth = 0
            for i in range(len(name) - 1, -1, -1):
                depth += {")": 1, "(": -1}.get(name[i], 0)
                if depth == 0:
                    name = name[:i]
                    break
        if name.startswith("void "):
            name = name[5:]
        return name.replace("qw::(anonymous namespace)::", "")[:120]

    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            gx = num(r, "Grid_Size_X", "Grid_Size")
            gz = num(r, "Grid_Size_Z")
            name = short(r["Kernel_Name"])
            if gz > 1:
                name += f" (grid z {gz})"
            key = (name, gx, num(r, "Workgroup_Size_X", "Workgroup_Size"))
            e = rows.setdefault(key, {"us": [], "vgpr": num(r, "VGPR_Count", "Arch_VGPR_Count"),
                                      "agpr": num(r, "Accum_VGPR_Count"),
                                      "lds": num(r, "LDS_Block_Size", "Group_Segment_Size"),
                                      "scratch": num(r, "Scratch_Size", "Private_Segment_Size")})
            e["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    order = sorted(rows.items(), key=lambda kv: -sum(kv[1]["us"]))
    lines = ["| kernel | grid threads | block | calls | avg us | median us | min us | max us | "
             "VGPR (alloc) | AGPR | LDS B | scratch B |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, gx, bx), e in order[:top]:
        us = e["us"]
        lines.append(f"| `{name}` | {gx} | {bx} | {len(us)} | {sum(us) / len(us):.2f} | "
                     f"{statistics.median(us):.2f} | {min(us):.2f} | {max(us):.2f} | "
                     f"{e['vgpr']} | {e['agpr']} | {e['lds']} | {e['scratch']} |")
    return "\n".join(lines)


def measured_traffic(label):
    """HBM bytes per launch of `label` from the committed counter summary, or
    None when the summary is missing or the kernel sources changed since."""
    try:
        txt = open(TRAFFIC_FILE).read()
        blob = json.loads(txt.split("```json")[1].split("```")[0])
    except (OSError, IndexError, ValueError):
        return None
    # only the measured kernel's own source and the shared header matter
    src = {v[0]: v[1] for v in PMC_KERNELS.values()}.get(label)
    now, then = source_hashes(), blob.get("source_sha256", {})
    if src is None or any(then.get(f) != now[f] for f in (src, "qw_internal.h")):
        return None
    k = blob.get("kernels", {}).get(label)
    return None if k is None else k["traffic_bytes"]


# ---------------------------------------------------------------- CPU leg
#
# The oracle on this machine's host cores, timed the way the 量化推理 page's
# script times its CPU paths (function `benchmark`: warm-up calls, then timed
# calls, median and p90 of the per-call times), in two modes:
#   one thread -- BLAS / OpenMP threads pinned to 1, as that script pins them;
#   all cores  -- each call split into row blocks (a group never crosses a
#                 row) over a pool of one process per host core, one BLAS
#                 thread each; weights, payload and scales sit in shared
#                 memory, so no timed call ships them between processes.
# The default run stays bounded (~20 s of CPU work per mode): the page's 20
# warm-ups + 101 reps on the tiny config, fewer on the 4096 and MLP matrices
# (the counts are reported with each figure), layer 0 of the 7B stack, and a
# 256-row block of the 70B GEMM.  `--cpu-protocol` runs 20 + 101 on c1-c3,
# the whole stack streamed one matrix at a time (3 reps) and the whole GEMM
# (3 reps), with the one-thread legs in separate processes on separate cores.

CPU_DEFAULT = {"c1": (20, 101), "c2": (2, 5), "c3": (1, 2), "c4": (0, 3), "c5": (1, 3),
               "c4_layers": 1, "c5_rows": 256}
CPU_FULL = {"c1": (20, 101), "c2": (20, 101), "c3": (20, 101), "c4": (0, 3), "c5": (0, 3),
            "c4_layers": 32, "c5_rows": 28672}


def _stats(ts_ns):
    t = sorted(ts_ns)
    return {"median_us": round(statistics.median(t) / 1e3, 1),
            "p90_us": round(t[-(-9 * len(t) // 10) - 1] / 1e3, 1)}


def _entry(cfg, op, ts_ns, warm, nbytes=None, flops=None, **extra):
    e = {"config": cfg, "op": op, "warmups": warm, "reps": len(ts_ns), **_stats(ts_ns), **extra}
    med_s = statistics.median(ts_ns) * 1e-9
    if nbytes is not None:
        e["bytes"] = nbytes
        e["GB/s"] = round(nbytes / med_s / 1e9, 4)
    if flops is not None:
        e["flops"] = flops
        e["TFLOP/s"] = round(flops / med_s / 1e12, 5)
    return e


def _timed(fn, warm, reps, what=None):
    """Per-call times (ns) of `reps` calls after `warm` untimed ones; with
    `what`, one progress line per call that takes over 10 s."""
    for _ in range(warm):
        fn()
    ts = []
    for r in range(reps):
        t0 = time.perf_counter_ns()
        fn()
        ts.append(time.perf_counter_ns() - t0)
        if what is not None and ts[-1] > 10e9:
            log(f"[oracle timing] {what}: rep {r + 1}/{reps} {ts[-1] / 1e9:.1f} s")
    return ts


class _Runner:
    """Runs oracle calls on row blocks: in this process (one thread) or over
    a process pool with the arrays in shared memory (all cores)."""

    def __init__(self, pool=None, folder=None):
        self.pool, self.folder, self.n = pool, folder, 0

    def share(self, a):
        """The array as the workers will see it (a memmap path or itself)."""
        if self.pool is None:
            return a
        self.n += 1
        path = os.path.join(self.folder, f"a{self.n}.npy")
        np = __import__("numpy")
        mm = np.lib.format.open_memmap(path, mode="w+", dtype=a.dtype, shape=a.shape)
        mm[...] = a
        mm.flush()
        return path

    def out(self, dtype, shape):
        np = __import__("numpy")
        if self.pool is None:
            return np.empty(shape, dtype)
        self.n += 1
        path = os.path.join(self.folder, f"a{self.n}.npy")
        np.lib.format.open_memmap(path, mode="w+", dtype=dtype, shape=shape).flush()
        return path

    def release(self):
        """Delete the shared arrays made so far (all-cores mode)."""
        if self.pool is None:
            return
        for f in os.listdir(self.folder):
            os.remove(os.path.join(self.folder, f))

    def call(self, op, n, **kw):
        """op over rows [0, n): inline, or as row blocks over the pool."""
        if self.pool is None:
            _cpu_block((op, 0, n, kw))
            return
        parts = max(1, min(n, self.pool._max_workers))
        step = -(-n // parts)
        list(self.pool.map(_cpu_block, [(op, r, min(n, r + step), kw)
                                        for r in range(0, n, step)]))


def _arr(a, mode="r"):
    np = __import__("numpy")
    return np.load(a, mmap_mode=mode) if isinstance(a, str) else a


def _cpu_block(task):
    """One row block [r0, r1) of an oracle call (weights [n][k], groups
    inside rows): quantize_pack, unpack, gemv (x fp32) or gemm (x bf16)."""
    import numpy as np

    import oracle

    op, r0, r1, kw = task
    bits, group, k = kw["bits"], kw["group"], kw["k"]
    pb, sg = k * bits // 8, k // group
    if op == "quantize_pack":
        w = _arr(kw["w"])
        rec = oracle.quantize_pack(np.asarray(w[r0:r1]), bits, group)
        _arr(kw["payload"], "r+")[r0 * pb:r1 * pb] = rec["payload"]
        _arr(kw["scales"], "r+")[r0 * sg:r1 * sg] = rec["scales"]
        return
    rec = dict(bits=bits, group=group, shape=[r1 - r0, k],
               payload=np.asarray(_arr(kw["payload"])[r0 * pb:r1 * pb]),
               scales=np.asarray(_arr(kw["scales"])[r0 * sg:r1 * sg]))
    if op == "unpack":
        _arr(kw["out"], "r+")[r0:r1] = oracle.unpack(rec)
    elif op == "gemv":
        _arr(kw["out"], "r+")[:, r0:r1] = oracle.gemv_ref(rec, _arr(kw["x"]))
    else:
        _arr(kw["out"], "r+")[:, r0:r1] = oracle.gemm_ref(rec, _arr(kw["x"]))


def _qbytes(n, k, bits, group):
    return n * k * 4 + n * k * bits // 8 + 4 * (n * k // group)


def _ubytes(n, k, bits, group):
    return n * k * bits // 8 + 4 * (n * k // group) + 4 * n * k


def _gbytes(n, k, bits, group, m):
    return n * k * bits // 8 + 4 * (n * k // group) + 4 * m * k + 4 * m * n


def _matrix_legs(run, cfg, w, bits, group, reps, ms, x_of, tag=""):
    """quantize_pack, unpack and the GEMV at every m of one matrix."""
    n, k = w.shape
    warm, nrep = reps
    kw = dict(bits=bits, group=group, k=k, w=run.share(w))
    kw["payload"] = run.out("uint8", (n * k * bits // 8,))
    kw["scales"] = run.out("float32", (n * k // group,))
    out = [_entry(cfg, f"quantize_pack{tag}", _timed(lambda: run.call("quantize_pack", n, **kw),
                                                     warm, nrep), warm, _qbytes(n, k, bits, group))]
    _progress(out[-1])
    kw["out"] = run.out("float32", (n, k))
    out.append(_entry(cfg, f"unpack{tag}", _timed(lambda: run.call("unpack", n, **kw), warm, nrep),
                      warm, _ubytes(n, k, bits, group)))
    _progress(out[-1])
    for m in ms:
        kg = dict(kw, x=run.share(x_of(m)), out=run.out("float64", (m, n)))
        out.append(_entry(cfg, f"gemv_m{m}{tag}", _timed(lambda: run.call("gemv", n, **kg), warm,
                                                        nrep), warm, _gbytes(n, k, bits, group, m),
                          2 * m * n * k))
        _progress(out[-1])
    return out


def _progress(e):
    log(f"[oracle timing] {e['config']} {e['op']}: {e['warmups']}+{e['reps']} calls, "
        f"median {e['median_us']:.0f} us")


def cpu_legs(mode, plan, legs):
    """The oracle legs `legs` (c1 .. c5) in this process, one thread or all
    cores; returns a list of entries."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import tempfile

    from int8_int4_dequant_amd import inputs

    pool, tmp = None, None
    if mode == "all_cores":
        cores = len(os.sched_getaffinity(0))
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            os.environ[v] = "1"
        pool = cf.ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn"))
        tmp = tempfile.TemporaryDirectory(dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    run = _Runner(pool, tmp.name if tmp else None)
    out = []
    try:
        if pool is not None:  # start every worker (imports) outside the timing
            list(pool.map(time.sleep, [0.2] * (2 * pool._max_workers)))
        if "c1" in legs:
            w, x = inputs.c1_weight(), inputs.c1_x()
            for bits in (8, 4):
                out += _matrix_legs(run, "c1", w, bits, 32, plan["c1"], [1], lambda m: x,
                                    f"_int{bits}")
        if "c2" in legs:
            out += _matrix_legs(run, "c2", inputs.c2_weight(), 8, 4096, plan["c2"], [1],
                                lambda m: inputs.c2_x())
        for j, mat in enumerate(inputs.C3["mats"]):
            if f"c3_{mat['tag']}" in legs or "c3" in legs:
                out += _matrix_legs(run, "c3", inputs.c3_weight(j), 4, 128, plan["c3"],
                                    inputs.C3["ms"], lambda m, j=j: inputs.c3_x(j, m),
                                    f"_{mat['tag']}")
        for leg in legs:
            if leg.startswith("c4"):
                out.append(_c4_leg(run, plan, leg))
        if "c5" in legs:
            out.append(_c5_leg(run, plan))
    finally:
        if pool is not None:
            pool.shutdown()
        if tmp is not None:
            tmp.cleanup()
    return out


def _c4_leg(run, plan, leg):
    """The step's work on the stack (quantize_pack then the M = 1 GEMV of
    every matrix), one matrix at a time, weights generated outside the
    timing; `leg` = "c4" or "c4:i/s" (shard i of s of the matrices)."""
    from int8_int4_dequant_amd import inputs

    mats = [m for m in inputs.c4_matrices() if m[0] < plan["c4_layers"]]
    if ":" in leg:
        i, s = map(int, leg.split(":")[1].split("/"))
        mats = mats[i::s]
    warm, nrep = plan["c4"]
    reps, nbytes = [0] * nrep, 0
    for j, (layer, tag, n, k, seed) in enumerate(mats):
        w = inputs.weight(seed, n, k, inputs.C4["sigma"])
        kw = dict(bits=4, group=32, k=k, w=run.share(w), x=run.share(inputs.c4_x(k)))
        kw["payload"] = run.out("uint8", (n * k // 2,))
        kw["scales"] = run.out("float32", (n * k // 32,))
        kw["out"] = run.out("float64", (1, n))

        def step():
            run.call("quantize_pack", n, **kw)
            run.call("gemv", n, **kw)
        for r, t in enumerate(_timed(step, warm, nrep)):
            reps[r] += t
        nbytes += _qbytes(n, k, 4, 32) + _gbytes(n, k, 4, 32, 1)
        run.release()
        if j % 8 == 7 or j == len(mats) - 1:
            log(f"[oracle timing] {leg}: {j + 1}/{len(mats)} matrices")
    return _entry("c4", f"quantize_pack+gemv_m1 ({len(mats)} matrices)", reps, warm, nbytes,
                  matrices=len(mats), rep_us=[round(t / 1e3, 1) for t in reps])


def _c5_leg(run, plan):
    """The prefill GEMM's oracle (fp64 product of the 2048 bf16 rows with the
    dequantized weight) on the first `c5_rows` weight rows, plus their
    quantize_pack outside the timing; TFLOP/s of that block."""
    from int8_int4_dequant_amd import inputs

    c = inputs.C5
    rows = plan["c5_rows"]
    w = inputs.c5_weight()[:rows]
    xb = inputs.c5_x_bf16()
    kw = dict(bits=4, group=128, k=c["k"], w=run.share(w), x=run.share(xb))
    kw["payload"] = run.out("uint8", (rows * c["k"] // 2,))
    kw["scales"] = run.out("float32", (rows * c["k"] // 128,))
    kw["out"] = run.out("float64", (c["m"], rows))
    run.call("quantize_pack", rows, **kw)
    warm, nrep = plan["c5"]
    ts = _timed(lambda: run.call("gemm", rows, **kw), warm, nrep, what=f"c5 gemm, {rows} rows")
    return _entry("c5", f"gemm ({c['m']} x {rows} x {c['k']}, fp64)", ts, warm,
                  flops=2 * c["m"] * rows * c["k"], rows=rows)


def cpu_worker(spec):
    """Child-process entry: spec = {mode, plan, legs}; prints the entries."""
    d = json.loads(spec)
    print(json.dumps(cpu_legs(d["mode"], d["plan"], d["legs"])))


def _run_cpu_child(mode, plan, legs, core=None, timeout=3600):
    env = dict(os.environ)
    if mode == "one_thread":
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                  "VECLIB_MAXIMUM_THREADS"):
            env[v] = "1"
    spec = json.dumps({"mode": mode, "plan": plan, "legs": legs})
    pre = (lambda: os.sched_setaffinity(0, {core})) if core is not None else None
    # the child's progress lines go straight to this process's stderr
    return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker", spec],
                            stdout=subprocess.PIPE, stderr=None, text=True, env=env,
                            preexec_fn=pre)


def _collect(procs, timeout=3600):
    out = []
    for p in procs:
        so, _ = p.communicate(timeout=timeout)
        if p.returncode != 0:
            raise RuntimeError(f"oracle timing child failed (exit {p.returncode})")
        out += json.loads(so.strip().splitlines()[-1])
    return out


def cpu_baselines(full=False):
    """Both modes over every config; returns (cpu_baseline, all_cores,
    configs).  The default plan runs each mode in one child process; the
    full protocol runs the one-thread legs in parallel children, one core
    each (reported), then the all-cores legs."""
    plan = CPU_FULL if full else CPU_DEFAULT
    cores = sorted(os.sched_getaffinity(0))
    if full:
        shards = max(1, min(8, len(cores) - 5))
        legs = [["c1", "c2"], ["c3_up"], ["c3_down"], ["c5"]] + \
            [[f"c4:{i}/{shards}"] for i in range(shards)]
        procs = [_run_cpu_child("one_thread", plan, lg, cores[i % len(cores)])
                 for i, lg in enumerate(legs)]
        one = _collect(procs)
        # the c4 shards of each rep add up to the stack's rep
        c4 = [e for e in one if e["config"] == "c4"]
        if c4:
            one = [e for e in one if e["config"] != "c4"] + [_merge_c4(c4)]
        concurrent = len(legs)
    else:
        one = _collect([_run_cpu_child("one_thread", plan, ["c1", "c2", "c3", "c4", "c5"])])
        concurrent = 1
    # (the 256 x 256 matrix is too small to split: its calls would time the
    # pool's dispatch, so it runs in the one-thread mode only)
    allc = _collect([_run_cpu_child("all_cores", plan, ["c2", "c3", "c4", "c5"])])
    c4a = next(e for e in one if e["config"] == "c4")
    c4b = next(e for e in allc if e["config"] == "c4")
    def sample(e):
        return (f"{e['op']} of the 7B stack "
                f"({'all 32 layers' if plan['c4_layers'] == 32 else 'layer 0'}), "
                f"weights generated outside the timing; median of {e['reps']} reps")
    one_thread = {"value": c4a["GB/s"], "unit": "GB/s", "cores": 1, "kind": "oracle",
                  "sample": sample(c4a), "median_us": c4a["median_us"], "p90_us": c4a["p90_us"]}
    all_cores = {"value": c4b["GB/s"], "unit": "GB/s", "cores": len(cores), "kind": "oracle",
                 "sample": sample(c4b) + "; row blocks over one process per core",
                 "median_us": c4b["median_us"], "p90_us": c4b["p90_us"]}
    configs = {"protocol": "full (the page's 20 warm-ups + 101 reps on c1-c3)" if full
               else "bounded (reps per entry)",
               "host_cores": len(cores), "one_thread_processes_at_once": concurrent,
               "one_thread": one, "all_cores": allc}
    return one_thread, all_cores, configs


def _merge_c4(parts):
    """The stack's reps from its shards' reps (each shard timed one thread,
    on its own core): rep r of the stack = the sum of the shards' rep r."""
    reps = [sum(p["rep_us"][r] for p in parts) * 1e3 for r in range(len(parts[0]["rep_us"]))]
    matrices = sum(p["matrices"] for p in parts)
    return _entry("c4", f"quantize_pack+gemv_m1 ({matrices} matrices; {len(parts)} shards "
                        f"timed on separate cores, reps summed)", reps, parts[0]["warmups"],
                  sum(p["bytes"] for p in parts), matrices=matrices,
                  rep_us=[round(t / 1e3, 1) for t in reps])


def cpu_protocol_summary(res):
    """Markdown table of a --cpu-protocol run."""
    one, allc, cfgs = res
    lines = [f"Host cores: {cfgs['host_cores']}; one-thread legs run "
             f"{cfgs['one_thread_processes_at_once']} processes at once, one core each.", "",
             "| mode | config | op | warm-ups | reps | median µs | p90 µs | GB/s | TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for mode in ("one_thread", "all_cores"):
        for e in cfgs[mode]:
            lines.append(f"| {mode} | {e['config']} | {e['op']} | {e['warmups']} | {e['reps']} | "
                         f"{e['median_us']} | {e['p90_us']} | {e.get('GB/s', '')} | "
                         f"{e.get('TFLOP/s', '')} |")
    return "\n".join(lines)


# ------------------------------------------------------------ accounting


def quant_bytes(n, k, bits=4, group=32):
    return n * k * 4 + n * k * bits // 8 + 4 * (n * k // group)


def gemv_bytes(n, k, m=1, bits=4, group=32):
    return n * k * bits // 8 + 4 * (n * k // group) + 4 * m * k + 4 * m * n


# ----------------------------------------------------------------- main


def main():
    args = parse()
    if args.cpu_worker:
        cpu_worker(args.cpu_worker)
        return
    if args.cpu_protocol:
        res = cpu_baselines(full=True)
        with open(args.cpu_protocol, "w") as f:
            f.write(cpu_protocol_summary(res) + "\n")
        print(json.dumps({"cpu_baseline": res[0], "cpu_baseline_all_cores": res[1],
                          "cpu_baseline_configs": res[2]}), flush=True)
        return
    if args.gptq_cpu_sample_worker:
        gptq_cpu_sample_worker()
        return
    if args.pmc_table:
        print(pmc_table(args.pmc_table))
        return
    if args.trace_table:
        print(trace_table(args.trace_table))
        return
    if args.pmc_summary:
        print("```json\n" + json.dumps(pmc_summary(*args.pmc_summary, copy_mib=1024), indent=1)
              + "\n```")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from int8_int4_dequant_amd import inputs, qw

    qw.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    L = qw.lib()

    if args.only_gptq:
        print(json.dumps(bench_gptq(args, L, stream)), flush=True)
        return

    # ---- setup: the stack's fp32 weights resident in HBM, outputs allocated
    mats = [m for m in inputs.c4_matrices() if m[0] < args.layers]
    W, P, S, Y = [], [], [], []
    xs = {k: torch.from_numpy(inputs.c4_x(k)).to(dev) for k in (4096, 11008)}
    t0 = time.time()

    def upload(i, layer, tag, w):
        n, k = w.shape
        W.append(torch.from_numpy(w).to(dev))
        P.append(torch.empty(n * k // 2, dtype=torch.uint8, device=dev))
        S.append(torch.empty(n * k // 32, dtype=torch.float32, device=dev))
        Y.append(torch.empty((1, n), dtype=torch.float32, device=dev))
        if (i + 1) % 28 == 0:
            log(f"setup: {i + 1} matrices resident ({time.time() - t0:.1f} s)")

    if args.layers == 32:
        inputs.c4_weights_parallel(upload)
    else:
        for i, (layer, tag, n, k, seed) in enumerate(mats):
            upload(i, layer, tag, inputs.weight(seed, n, k, inputs.C4["sigma"]))
    torch.cuda.synchronize()
    log(f"setup: {len(W)} matrices uploaded in {time.time() - t0:.1f} s")

    shapes = [(m[2], m[3]) for m in mats]
    qbytes = sum(quant_bytes(n, k) for n, k in shapes)
    gbytes = sum(gemv_bytes(n, k) for n, k in shapes)
    weights = sum(n * k for n, k in shapes)

    # quantize/pack every matrix, then the decode pass: one batched call each
    # (a few large launches instead of one per matrix)
    qdescs, nq = qw.make_quant_descs(
        (4, 32, n, k, W[i], P[i], S[i]) for i, (n, k) in enumerate(shapes))
    descs, ndesc = qw.make_gemv_descs(
        (4, 32, n, k, P[i], S[i], xs[k], Y[i]) for i, (n, k) in enumerate(shapes))
    quant_launches = (nq + qw.BATCH_PER_LAUNCH - 1) // qw.BATCH_PER_LAUNCH
    gemv_launches = (ndesc + qw.BATCH_PER_LAUNCH - 1) // qw.BATCH_PER_LAUNCH

    def run_step(ev=None):
        if ev is not None:
            ev[0][0].record(stream)
        st = L.qw_quantize_pack_batched(nq, qdescs, sptr)
        if ev is not None:
            ev[1][0].record(stream)
        if st:
            raise RuntimeError(f"qw_quantize_pack_batched failed: {st}")
        if ev is not None:
            ev[2][0].record(stream)
        st = L.qw_gemv_batched(ndesc, descs, 1, sptr)
        if ev is not None:
            ev[3][0].record(stream)
        if st:
            raise RuntimeError(f"qw_gemv_batched failed: {st}")

    def single_quant_pass():
        for i, (n, k) in enumerate(shapes):
            st = L.qw_quantize_pack(4, 32, n, k, W[i].data_ptr(), P[i].data_ptr(),
                                    S[i].data_ptr(), sptr)
            if st:
                raise RuntimeError(f"qw_quantize_pack failed: {st}")

    def single_gemv_pass(sp=None):
        for i, (n, k) in enumerate(shapes):
            st = L.qw_gemv(4, 32, n, k, P[i].data_ptr(), S[i].data_ptr(), 1,
                           xs[k].data_ptr(), Y[i].data_ptr(), sptr if sp is None else sp)
            if st:
                raise RuntimeError(f"qw_gemv failed: {st}")

    prewarm(args, run_step)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, per-launch HIP events on the launch stream
    evs = [[[torch.cuda.Event(enable_timing=True)] for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        run_step(evs[s])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    # the clock the step runs at (a sustained run after the timed one)
    step_clock = sustained_clock(args, run_step)

    q_ms = sum(evs[s][0][0].elapsed_time(evs[s][1][0]) for s in range(args.steps))
    g_ms = sum(evs[s][2][0].elapsed_time(evs[s][3][0]) for s in range(args.steps))
    q_avg_us = 1e3 * q_ms / (args.steps * quant_launches)
    g_avg_us = 1e3 * g_ms / (args.steps * gemv_launches)
    # per-step spread (GPU time between the events of each step)
    def med_p90_us(pairs):
        t = sorted(1e3 * e0.elapsed_time(e1) for e0, e1 in pairs)
        return {"median_us": round(statistics.median(t), 1),
                "p90_us": round(t[-(-9 * len(t) // 10) - 1], 1)}

    q_spread = med_p90_us([(evs[s][0][0], evs[s][1][0]) for s in range(args.steps)])
    g_spread = med_p90_us([(evs[s][2][0], evs[s][3][0]) for s in range(args.steps)])
    step_spread = med_p90_us([(evs[s][0][0], evs[s][3][0]) for s in range(args.steps)])

    # for comparison (not part of the step): the same passes as one launch per matrix
    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps

    single_us = timed(single_gemv_pass)
    single_q_us = timed(single_quant_pass)
    # the same one-launch-per-matrix pass replayed from a HIP graph (every
    # replay checked against the eager outputs)
    single_graph_us = None
    try:
        ref = [y.clone() for y in Y]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            single_gemv_pass(side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            single_gemv_pass(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for _ in range(3):
            for y in Y:
                y.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(ref, Y)):
                raise RuntimeError("graph replay differs from the eager pass")
        single_graph_us = timed(g.replay)
        del g
    except RuntimeError as exc:
        log(f"graph replay of the per-matrix pass skipped: {exc}")

    # unpack (a5 on its own): every matrix back to fp32, as one batched call
    # (qw_unpack_batched, distinct outputs) and as one call per matrix
    wouts = [torch.empty(n * k, dtype=torch.float32, device=dev) for n, k in shapes]
    udescs, und = qw.make_unpack_descs((4, 32, n, k, P[i], S[i], wouts[i])
                                       for i, (n, k) in enumerate(shapes))

    def unpack_pass():
        st = L.qw_unpack_batched(und, udescs, sptr)
        if st:
            raise RuntimeError(f"qw_unpack_batched failed: {st}")

    def unpack_single_pass():
        for i, (n, k) in enumerate(shapes):
            st = L.qw_unpack(4, 32, n, k, P[i].data_ptr(), S[i].data_ptr(), wouts[i].data_ptr(),
                             sptr)
            if st:
                raise RuntimeError(f"qw_unpack failed: {st}")

    unpack_us = timed(unpack_pass)
    unpack_single_us = timed(unpack_single_pass)

    # the same decode pass at 8 rows of x (several sequences at once): one
    # batched call, which takes the matrix-core kernel
    x8 = {k: torch.from_numpy(inputs.c4_x8(k)).to(dev) for k in (4096, 11008)}
    Y8 = [torch.empty((8, n), dtype=torch.float32, device=dev) for n, k in shapes]
    d8, n8 = qw.make_gemv_descs(
        (4, 32, n, k, P[i], S[i], x8[k], Y8[i]) for i, (n, k) in enumerate(shapes))

    def m8_pass():
        st = L.qw_gemv_batched(n8, d8, 8, sptr)
        if st:
            raise RuntimeError(f"qw_gemv_batched (m = 8) failed: {st}")

    prewarm(args, m8_pass)
    m8_us = timed(m8_pass)
    gbytes8 = sum(gemv_bytes(n, k, m=8) for n, k in shapes)
    del Y8, d8
    ubytes = sum(n * k * 4 + n * k // 2 + 4 * (n * k // 32) for n, k in shapes)
    del wouts, udescs
    q_gbs = qbytes * args.steps / (q_ms * 1e-3) / 1e9
    g_gbs = gbytes * args.steps / (g_ms * 1e-3) / 1e9
    ms_per_step = 1e3 * t_total / args.steps
    value = (qbytes + gbytes) / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step:.3f} ms; quantize {q_gbs:.0f} GB/s ({quant_launches} launches, avg "
        f"{q_avg_us:.1f} us); one quantize launch per matrix: {single_q_us:.1f} us; "
        f"gemv pass {g_gbs:.0f} GB/s ({1e3 * g_ms / args.steps:.1f} us, {gemv_launches} launches); "
        f"one launch per matrix: {single_us:.1f} us (graph replay "
        f"{single_graph_us if single_graph_us is None else round(single_graph_us, 1)} us); "
        f"unpack pass {unpack_us:.1f} us "
        f"({ubytes / (unpack_us * 1e-6) / 1e9:.0f} GB/s, 1 batched call; one launch per matrix: "
        f"{unpack_single_us:.1f} us); pass at 8 rows of x {m8_us:.1f} us")

    chain = bench_chain(args, L, stream, mats, shapes, P, S, xs, gbytes)

    dominant = "quantize_pack" if q_ms >= g_ms else "gemv"
    if dominant == "quantize_pack":
        ach, per_launch = q_gbs, qbytes / quant_launches
    else:
        ach, per_launch = g_gbs, gbytes / gemv_launches
    traffic = measured_traffic("quantize_pack_batched" if dominant == "quantize_pack"
                               else "gemv_batched_m1")
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("qw_quantize_pack_batched" if dominant == "quantize_pack"
                           else "qw_gemv_batched") + " (int4 g32, 224 matrices per step)",
                "algorithmic_bytes_per_launch": round(per_launch),
                "avg_launch_us": round(q_avg_us if dominant == "quantize_pack" else g_avg_us, 3)}
    roofline_gemv = {"bound": "hbm", "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemv_batched_m1"),
                     "kernel": "qw_gemv_batched M=1 (int4 g32, 224 matrices per launch)",
                     "algorithmic_bytes_per_launch": round(gbytes / gemv_launches),
                     "avg_launch_us": round(g_avg_us, 3)}
    parts = {
        "quantize_pack": {"GB/s": round(q_gbs, 1), "frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
                          "entry": "qw_quantize_pack_batched", "launches_per_pass": quant_launches,
                          "avg_launch_us": round(q_avg_us, 3), "bytes_per_step": qbytes,
                          "pass_us": round(1e3 * q_ms / args.steps, 1), **q_spread},
        "quantize_pack_one_launch_per_matrix": {
            "pass_us": round(single_q_us, 1),
            "GB/s": round(qbytes / (single_q_us * 1e-6) / 1e9, 1)},
        "decode_gemv_m1": {"GB/s": round(g_gbs, 1), "frac_hbm": round(g_gbs / HBM_PEAK_GBS, 4),
                           "entry": "qw_gemv_batched", "launches_per_pass": gemv_launches,
                           "avg_launch_us": round(g_avg_us, 3), "bytes_per_step": gbytes,
                           "traffic_per_launch": measured_traffic("gemv_batched_m1"),
                           "pass_us": round(1e3 * g_ms / args.steps, 1), **g_spread},
        "step": {"entries": "qw_quantize_pack_batched then qw_gemv_batched", **step_spread,
                 "gpu_clock_sustained": step_clock},
        "unpack": {"GB/s": round(ubytes / (unpack_us * 1e-6) / 1e9, 1),
                   "frac_hbm": round(ubytes / (unpack_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "entry": "qw_unpack_batched", "launches_per_pass": 1,
                   "pass_us": round(unpack_us, 1), "bytes_per_pass": ubytes},
        "unpack_one_launch_per_matrix": {
            "pass_us": round(unpack_single_us, 1),
            "GB/s": round(ubytes / (unpack_single_us * 1e-6) / 1e9, 1)},
        "decode_chain_m1": chain,
        "decode_gemv_m8": {"entry": "qw_gemv_batched (matrix cores)", "m": 8,
                           "pass_us": round(m8_us, 1), "bytes_per_pass": gbytes8,
                           "GB/s": round(gbytes8 / (m8_us * 1e-6) / 1e9, 1),
                           "TFLOP/s": round(2.0 * 8 * weights / (m8_us * 1e-6) / 1e12, 2)},
        "decode_gemv_m1_one_launch_per_matrix": {
            "pass_us": round(single_us, 1),
            "GB/s": round(gbytes / (single_us * 1e-6) / 1e9, 1),
            "graph_replay_pass_us": None if single_graph_us is None else round(single_graph_us, 1),
            "graph_replay_GB/s": None if single_graph_us is None
            else round(gbytes / (single_graph_us * 1e-6) / 1e9, 1)},
    }

    if args.calib_copy_mib:
        # known-size device copy (outside the timed region) for the byte counters
        # (an elementwise negation: fully coalesced 16-byte loads and stores per
        # lane like the kernels measured, N bytes read and N bytes written)
        nf = (args.calib_copy_mib << 20) // 4
        src = torch.empty(nf, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # free the stack before the GEMM leg
    del W, P, S, Y
    torch.cuda.empty_cache()

    gemv_cfgs = bench_gemv_configs(args, L, stream)

    gemm = None
    if not args.no_gemm:
        gemm = bench_gemm(args, L, stream)

    gptq = None if args.no_gptq else bench_gptq(args, L, stream)

    context = None if args.no_context else bench_context(args, stream)

    cpu = cpu_all = cpu_cfgs = None
    if not args.no_cpu_baseline:
        try:
            cpu, cpu_all, cpu_cfgs = cpu_baselines()
        except Exception as exc:  # a child that cannot run is reported, not fatal
            log(f"oracle baseline skipped: {exc}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) fp32 weights in place of trained 7B layers)",
        "config": {"workload": "c4: 7B-shaped linear stack, 32 layers x (4 x 4096x4096 + 2 x "
                               "11008x4096 + 4096x11008), int4 group 32. One step = quantize+pack "
                               "of all 224 matrices (one launch) then one M=1 dequant-GEMV pass "
                               "(one launch); value = (quantize bytes + GEMV bytes) / step time, "
                               "a blend of the two kernels. The GEMV pass alone: roofline_gemv "
                               "and parts.decode_gemv_m1",
                   "layers": args.layers, "matrices": len(shapes), "weights": weights,
                   "bits": 4, "group": 32, "m": 1, "bytes_per_step": qbytes + gbytes},
        "roofline": roofline, "roofline_gemv": roofline_gemv, "parts": parts,
        "decode_gemv_configs": gemv_cfgs, "context": context,
        "prefill_gemm": gemm, "gptq": gptq, "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all, "cpu_baseline_configs": cpu_cfgs,
    }
    print(json.dumps(out), flush=True)


def bench_chain(args, L, stream, mats, shapes, P, S, xs, gbytes):
    """The decode pass as a chain: in every layer q, k, v read the layer's
    input, o reads v's output, gate and up read o's, down reads up's, and the
    next layer reads down's (no attention or nonlinearity in between).  Four
    dependent stages per layer, 128 for the stack, timed as one
    qw_gemv_chain call (one launch per stage) and as those launches replayed
    from a HIP graph."""
    import torch

    from int8_int4_dequant_amd import qw

    dev = torch.device("cuda:0")
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for n, _ in shapes]
    slot_of = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}
    wiring, stages = [], []
    index = {}
    for i, (layer, tag, n, k, _seed) in enumerate(mats):
        index[(layer, tag)] = i
    for i, (layer, tag, n, k, _seed) in enumerate(mats):
        slot = slot_of[tag]
        if slot <= 2:
            x = xs[4096] if layer == 0 else ys[index[(layer - 1, "down")]]
            st = 0
        elif slot == 3:
            x, st = ys[index[(layer, "v")]], 1
        elif slot in (4, 5):
            x, st = ys[index[(layer, "o")]], 2
        else:
            x, st = ys[index[(layer, "up")]], 3
        wiring.append(x)
        stages.append(4 * layer + st)
    descs, nd = qw.make_gemv_descs((4, 32, n, k, P[i], S[i], wiring[i], ys[i])
                                   for i, (n, k) in enumerate(shapes))
    import ctypes
    stg = (ctypes.c_int32 * nd)(*stages)

    def run(sp):
        r = L.qw_gemv_chain(nd, descs, stg, 1, sp)
        if r:
            raise RuntimeError(f"qw_gemv_chain failed: {r}")

    def timed(fn, reps=max(3, args.steps)):
        prewarm(args, fn)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / reps

    sp = stream.cuda_stream
    chain_us = timed(lambda: run(sp))
    ref = [y.clone() for y in ys]
    same = True
    graph_us = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run(side.cuda_stream)   # warm-up outside capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for _ in range(3):   # every replay must reproduce the eager result
            for y in ys:
                y.zero_()
            g.replay()
            torch.cuda.synchronize()
            same = same and all(torch.equal(a, b) for a, b in zip(ref, ys))
        graph_us = timed(g.replay)
    except RuntimeError as exc:  # capture unsupported: report without it
        log(f"chain graph capture skipped: {exc}")
    gbs = lambda us: round(gbytes / (us * 1e-6) / 1e9, 1)
    log(f"chained decode pass ({len(set(stages))} stages): {chain_us:.1f} us ({gbs(chain_us)} GB/s)"
        + (f", graph replay {graph_us:.1f} us ({gbs(graph_us)} GB/s)" if graph_us else "")
        + f"; replays identical: {same}")
    return {"entry": "qw_gemv_chain", "stages": len(set(stages)), "matrices": nd,
            "bytes_per_pass": gbytes, "pass_us": round(chain_us, 1), "GB/s": gbs(chain_us),
            "frac_hbm": round(gbs(chain_us) / HBM_PEAK_GBS, 4),
            "graph_replay_us": None if graph_us is None else round(graph_us, 1),
            "graph_replay_GB/s": None if graph_us is None else gbs(graph_us),
            "graph_replays_identical": bool(same)}


def _event_us(stream, fn, reps):
    """Per-call GPU times (µs) of `fn`, each bracketed by events on `stream`."""
    import torch
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(1e3 * a.elapsed_time(b) for a, b in ev)


def bench_context(args, stream):
    """Practical ceilings of this part, timed in the same run as the
    kernels: a device copy of 2 GiB (torch: 2 GiB read + 2 GiB written), a
    read-only reduction over 4 GiB (torch.sum), and the vendor BLAS bf16
    product (torch.matmul, bf16 in and out, no dequantization) at the
    prefill shape 2048 x 28672 x 8192 on random operands, with the clock it
    sustains."""
    import torch

    dev = torch.device("cuda:0")
    out = {}
    gen = torch.Generator(device=dev).manual_seed(1234)
    n = (2 << 30) // 4
    src = torch.rand(n, dtype=torch.float32, device=dev, generator=gen)
    dst = torch.empty_like(src)
    prewarm(args, lambda: dst.copy_(src))
    t = _event_us(stream, lambda: dst.copy_(src), 10)
    med = statistics.median(t)
    out["device_copy_2GiB"] = {"bytes": 8 * n, "median_us": round(med, 1),
                               "GB/s": round(8 * n / (med * 1e-6) / 1e9, 1),
                               "frac_hbm": round(8 * n / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del dst
    big = torch.cat([src, src])
    del src
    prewarm(args, lambda: big.sum())
    t = _event_us(stream, lambda: big.sum(), 10)
    med = statistics.median(t)
    out["device_read_4GiB"] = {"bytes": 4 * big.numel(), "median_us": round(med, 1),
                               "GB/s": round(4 * big.numel() / (med * 1e-6) / 1e9, 1),
                               "frac_hbm": round(4 * big.numel() / (med * 1e-6) / 1e9
                                                 / HBM_PEAK_GBS, 4)}
    del big
    torch.cuda.empty_cache()
    m, nn, k = 2048, 28672, 8192
    x = torch.randn((m, k), dtype=torch.float32, device=dev, generator=gen).to(torch.bfloat16)
    wt = (torch.randn((k, nn), dtype=torch.float32, device=dev, generator=gen) * 0.015
          ).to(torch.bfloat16)              # the weight's transpose, contiguous
    y = torch.empty((m, nn), dtype=torch.bfloat16, device=dev)
    mm = lambda: torch.matmul(x, wt, out=y)  # noqa: E731
    prewarm(args, mm)
    t = _event_us(stream, mm, 20)
    med = statistics.median(t)
    tf = 2.0 * m * nn * k / (med * 1e-6) / 1e12
    out["torch_matmul_bf16_2048x28672x8192"] = {
        "median_us": round(med, 1), "p90_us": round(t[-(-9 * len(t) // 10) - 1], 1),
        "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
        "gpu_clock_sustained": sustained_clock(args, mm)}
    del x, wt, y
    torch.cuda.empty_cache()
    log("context: copy {GB/s} GB/s, ".format(**out["device_copy_2GiB"])
        + "read {GB/s} GB/s, ".format(**out["device_read_4GiB"])
        + "torch.matmul bf16 {median_us} us = {TFLOP/s} TFLOP/s".format(
            **out["torch_matmul_bf16_2048x28672x8192"]))
    return out


def bench_gemv_configs(args, L, stream):
    """The single-matrix decode GEMVs of the other workloads: c2 (int8, one
    scale per output channel, M = 1) and c3 (int4 group 128, MLP up and down,
    M = 1, 4, 8).  Each is timed over rotating copies of its packed weight
    totalling >= 1 GiB, so the 256 MB Infinity Cache cannot serve repeats."""
    import numpy as np
    import torch

    from int8_int4_dequant_amd import inputs

    dev = torch.device("cuda:0")
    sp = stream.cuda_stream
    out = {}

    def one(tag, w, bits, group, ms, xs_of):
        n, k = w.shape
        wd = torch.from_numpy(w).to(dev)
        p0 = torch.empty(n * k * bits // 8, dtype=torch.uint8, device=dev)
        s0 = torch.empty(n * k // group, dtype=torch.float32, device=dev)
        st = L.qw_quantize_pack(bits, group, n, k, wd.data_ptr(), p0.data_ptr(), s0.data_ptr(), sp)
        assert st == 0, st
        del wd
        wbytes = p0.numel() + 4 * s0.numel()
        copies = max(2, -(-(1 << 30) // wbytes))
        ps = [p0] + [p0.clone() for _ in range(copies - 1)]
        ss = [s0] + [s0.clone() for _ in range(copies - 1)]
        for m in ms:
            x = torch.from_numpy(xs_of(m)).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)

            def rnd():
                for c in range(copies):
                    r = L.qw_gemv(bits, group, n, k, ps[c].data_ptr(), ss[c].data_ptr(), m,
                                  x.data_ptr(), y.data_ptr(), sp)
                    if r:
                        raise RuntimeError(f"qw_gemv failed: {r}")
            prewarm(args, rnd)
            rnd()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            reps = 3
            for _ in range(reps):
                rnd()
            e1.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / (reps * copies)
            nbytes = wbytes + 4 * m * k + 4 * m * n
            gbs = nbytes / (us * 1e-6) / 1e9
            flops = 2.0 * m * n * k
            out[f"{tag}_m{m}"] = {"shape_nk": [n, k], "bits": bits, "group": group, "m": m,
                                  "us_per_call": round(us, 2), "GB/s": round(gbs, 1),
                                  "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                  "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 3),
                                  "rotating_copies": copies}
            log(f"gemv {tag} m={m}: {us:.2f} us/call, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%})")
        del ps, ss
        torch.cuda.empty_cache()

    one("c2_int8_per_channel_4096x4096", inputs.c2_weight(), 8, 4096, [1], lambda m: inputs.c2_x())
    for j, mat in enumerate(inputs.C3["mats"]):
        one(f"c3_int4_g128_{mat['tag']}_{mat['n']}x{mat['k']}", inputs.c3_weight(j), 4, 128,
            inputs.C3["ms"], lambda m, j=j: inputs.c3_x(j, m))
    return out


def bench_gemm(args, L, stream):
    import numpy as np
    import torch

    from int8_int4_dequant_amd import inputs

    dev = torch.device("cuda:0")
    c = inputs.C5
    n, k, m = c["n"], c["k"], c["m"]
    w = torch.from_numpy(inputs.c5_weight()).to(dev)
    p = torch.empty(n * k // 2, dtype=torch.uint8, device=dev)
    s = torch.empty(n * k // 128, dtype=torch.float32, device=dev)
    st = L.qw_quantize_pack(4, 128, n, k, w.data_ptr(), p.data_ptr(), s.data_ptr(), stream.cuda_stream)
    assert st == 0, st
    del w
    x = torch.from_numpy(inputs.c5_x_bf16().view(np.int16)).to(dev)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    sp = stream.cuda_stream

    def run():
        r = L.qw_gemm(4, 128, n, k, p.data_ptr(), s.data_ptr(), m, x.data_ptr(), y.data_ptr(), sp)
        if r:
            raise RuntimeError(f"qw_gemm failed: {r}")

    prewarm(args, run)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.gemm_reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in ev)
    clock = sustained_clock(args, run)
    med = times[len(times) // 2]
    flops = 2.0 * m * n * k

    # the same weight against the number of rows: qw_gemm (bf16, matrix cores)
    # and, up to 8 rows, qw_gemv (fp32) -- where one product overtakes the
    # other.  Three copies of the packed weight (372 MB) are taken in turn, so
    # the 256 MB Infinity Cache cannot serve a repeat.
    sweep = {}
    xf = torch.from_numpy(inputs.activations(7, 8, k)).to(dev)
    yv = torch.empty((8, n), dtype=torch.float32, device=dev)
    # fp32 activations for qw_matmul (QuantizedMatmul: GEMV up to
    # MATMUL_GEMV_MAX_M rows, else bf16 rounding into `mw` and the GEMM)
    xm = torch.from_numpy(inputs.activations(8, 1024, k)).to(dev)
    mw = torch.empty(max(1, L.qw_matmul_work_bytes(1024, k)), dtype=torch.uint8, device=dev)
    copies = [(p, s), (p.clone(), s.clone()), (p.clone(), s.clone())]
    for mm in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        def g(mm=mm):
            for pc, sc in copies:
                r = L.qw_gemm(4, 128, n, k, pc.data_ptr(), sc.data_ptr(), mm, x.data_ptr(),
                              y.data_ptr(), sp)
                if r:
                    raise RuntimeError(f"qw_gemm failed: {r}")

        def v(mm=mm):
            for pc, sc in copies:
                r = L.qw_gemv(4, 128, n, k, pc.data_ptr(), sc.data_ptr(), mm, xf.data_ptr(),
                              yv.data_ptr(), sp)
                if r:
                    raise RuntimeError(f"qw_gemv failed: {r}")

        def mmul(mm=mm):
            for pc, sc in copies:
                r = L.qw_matmul(4, 128, n, k, pc.data_ptr(), sc.data_ptr(), mm, xm.data_ptr(),
                                y.data_ptr(), mw.data_ptr(), mw.numel(), sp)
                if r:
                    raise RuntimeError(f"qw_matmul failed: {r}")

        row = {}
        for name, fn in (("gemm_us", g), ("gemv_us", v), ("matmul_us", mmul)):
            if name == "gemv_us" and mm > 8:
                continue
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(3):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            row[name] = round(1e3 * e0.elapsed_time(e1) / (3 * len(copies)), 2)
        row["gemm_TFLOP/s"] = round(2.0 * mm * n * k / (row["gemm_us"] * 1e-6) / 1e12, 1)
        sweep[str(mm)] = row
    del copies, xm, mw
    log("gemm/gemv against m: " + ", ".join(
        f"m={k_}: {r_['gemm_us']:.0f}" + (f"/{r_['gemv_us']:.0f}" if "gemv_us" in r_ else "") + " us"
        for k_, r_ in sweep.items()))
    log("qw_matmul against m: " + ", ".join(f"m={k_}: {r_['matmul_us']:.0f} us"
                                           for k_, r_ in sweep.items()))
    tf = flops / (med * 1e-3) / 1e12
    if clock is not None:
        # the dense bf16 peak scales with the clock (2.5 PFLOP/s at 2.4 GHz)
        clock["bf16_peak_tflops_at_median_clock"] = round(
            BF16_PEAK_TFLOPS * clock["gfx_mhz_median"] / 2400.0, 1)
    log(f"gemm: median {med * 1e3:.1f} us, {tf:.1f} TFLOP/s ({tf / BF16_PEAK_TFLOPS:.1%} of bf16 peak)"
        + ("" if clock is None else f"; clock {clock['gfx_mhz_median']} MHz, "
           f"{clock['socket_w_median']} W ({clock['samples']} samples)"))
    return {"workload": "c5: M=2048 bf16 x (28672 x 8192) int4 group 128, fp32 accumulate",
            "m_sweep_same_weight": sweep,
            "median_us": round(med * 1e3, 2), "p90_us": round(times[-(-9 * len(times) // 10) - 1] * 1e3, 2),
            "rep_us_sorted": [round(t_ * 1e3, 1) for t_ in times],
            "TFLOP/s": round(tf, 2), "gpu_clock_sustained": clock,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("gemm"),
                         "algorithmic_bytes": n * k // 2 + n * k // 128 * 4 + m * k * 2 + m * n * 4}}


# ------------------------------------------------------------------ GPTQ

FP64_PEAK_TFLOPS = 78.6
GPTQ_BATCHES = 8  # calibration batches per input (the page: 8 batches of 16 sequences)


def gptq_cpu_sample_worker():
    """Runs in a child process with one BLAS / OpenMP thread: the oracle on
    the whole layer the GPU leg times (per input: H over the 65,536
    calibration tokens in 8 batches, damping, factor, then the codes of
    every map reading that input)."""
    import numpy as np

    from oracle import gptq as G
    from int8_int4_dequant_amd import inputs

    dt = 0.0
    weights = 0
    for src in inputs.SMALLEM_INPUTS:
        x = inputs.smallem_calibration(src)
        maps = [(s, m) for s, m in enumerate(inputs.SMALLEM_LAYER) if m[3] == src]
        ws = [inputs.smallem_weight(s) for s, _ in maps]
        t0 = time.perf_counter()
        u = G.inverse_factor(G.damped(G.hessian(np.array_split(x, GPTQ_BATCHES))))
        for w in ws:
            G.quantize_pack(w, u, 4, inputs.smallem_group(w.shape[1]))
        dt += time.perf_counter() - t0
        weights += sum(w.size for w in ws)
        del x
    print(json.dumps(dict(seconds=dt, weights=weights, tokens=inputs.CALIB_TOKENS)))


def gptq_cpu_baseline():
    env = dict(os.environ)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "VECLIB_MAXIMUM_THREADS"):
        env[v] = "1"
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--gptq-cpu-sample-worker"],
                       capture_output=True, text=True, env=env, timeout=900)
    if r.returncode != 0:
        log(r.stderr[-2000:])
        return None
    d = json.loads(r.stdout.strip().splitlines()[-1])
    return {"value": round(d["weights"] / d["seconds"], 1), "unit": "weights/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the whole layer ({d['weights']} weights, 4 inputs of {d['tokens']} "
                      f"tokens in {GPTQ_BATCHES} batches): oracle H, factor and codes, "
                      f"{d['seconds']:.2f} s, one thread"}


def bench_gptq(args, L, stream):
    """GPTQ of one layer of the page's small model from its calibration
    inputs: per input, H accumulated over 8 batches (qw_gptq_hessian), the
    factor (qw_gptq_factor), then the codes of every map reading that input
    (qw_gptq_quantize_pack).  Timed with events on the launch stream."""
    import torch

    from int8_int4_dequant_amd import inputs

    dev = torch.device("cuda:0")
    sp = stream.cuda_stream
    groups = {}
    for slot, (name, n, k, src) in enumerate(inputs.SMALLEM_LAYER):
        groups.setdefault(src, []).append((slot, name, n, k))
    T = inputs.CALIB_TOKENS
    chunk = T // GPTQ_BATCHES
    data = {}
    for src, maps in groups.items():
        k = maps[0][3]
        x = torch.from_numpy(inputs.smallem_calibration(src)).to(dev)
        h = torch.empty((k, k), dtype=torch.float64, device=dev)
        u = torch.empty((k, k), dtype=torch.float64, device=dev)
        info = torch.zeros(1, dtype=torch.int32, device=dev)
        hw = L.qw_gptq_hessian_work_bytes(k, chunk)
        fw = L.qw_gptq_factor_work_bytes(k)
        # the maps reading one input share its H and U, and GPTQ treats every
        # output channel on its own: they are stacked along n into one call
        # (q, k, v: 1536 rows; gate, up: 2736), whose payload and scales are
        # the maps' own, one after the other
        g = inputs.smallem_group(k)
        n = sum(mp_[2] for mp_ in maps)
        w = torch.cat([torch.from_numpy(inputs.smallem_weight(slot)) for slot, *_ in maps]).to(dev)
        recs = [dict(name="+".join(mp_[1] for mp_ in maps), n=n, k=k, group=g, w=w,
                     p=torch.empty(n * k // 2, dtype=torch.uint8, device=dev),
                     s=torch.empty(n * k // g, dtype=torch.float32, device=dev),
                     wb=L.qw_gptq_quantize_work_bytes(n, k))]
        qwb = recs[0]["wb"]
        data[src] = dict(k=k, x=x, h=h, u=u, info=info, hw=hw, fw=fw, recs=recs,
                         hwork=torch.empty(hw, dtype=torch.uint8, device=dev),
                         fwork=torch.empty(fw, dtype=torch.uint8, device=dev),
                         qwork=torch.empty(qwb, dtype=torch.uint8, device=dev))

    def ck(r, what):
        if r:
            raise RuntimeError(f"{what} failed: {r}")

    streams = {src: torch.cuda.Stream() for src in data}  # default priority

    def run(ev=None, concurrent=False):
        # one chain per input; with `concurrent` each runs on its own stream
        # (they are independent), else all run on `stream` one after another
        if concurrent:
            start = torch.cuda.Event()
            start.record(stream)
        # the longest chain (largest k) first, so its factor and codes overlap
        # the other inputs' accumulation of H
        for src, d in sorted(data.items(), key=lambda kv: -kv[1]["k"]):
            k = d["k"]
            st = streams[src] if concurrent else stream
            sp_ = st.cuda_stream
            if concurrent:
                st.wait_event(start)
            if ev is not None:
                ev[src][0].record(st)
            with torch.cuda.stream(st):
                d["h"].zero_()
            for b in range(GPTQ_BATCHES):
                ck(L.qw_gptq_hessian(k, chunk, d["x"][b * chunk:].data_ptr(), d["h"].data_ptr(),
                                     d["hwork"].data_ptr(), d["hw"], sp_), "qw_gptq_hessian")
            if ev is not None:
                ev[src][1].record(st)
            ck(L.qw_gptq_factor(k, d["h"].data_ptr(), 0.01, d["u"].data_ptr(),
                                d["info"].data_ptr(), d["fwork"].data_ptr(), d["fw"], sp_),
               "qw_gptq_factor")
            if ev is not None:
                ev[src][2].record(st)
            for r in d["recs"]:
                ck(L.qw_gptq_quantize_pack(4, r["group"], r["n"], r["k"], r["w"].data_ptr(),
                                           d["u"].data_ptr(), r["p"].data_ptr(),
                                           r["s"].data_ptr(), d["qwork"].data_ptr(),
                                           d["qwork"].numel(), sp_), "qw_gptq_quantize_pack")
            if ev is not None:
                ev[src][3].record(st)
        if concurrent:
            for src in data:
                stream.wait_stream(streams[src])

    def outputs():
        torch.cuda.synchronize()
        for src, d in data.items():
            if int(d["info"].item()) != 0:
                raise RuntimeError(f"GPTQ factor of {src} reported a non-positive-definite H")
        return [t.clone() for d in data.values() for r in d["recs"] for t in (r["p"], r["s"])]

    run()
    one_stream = outputs()
    run(concurrent=True)
    # the chains are deterministic: four streams must give the same codes
    if not all(torch.equal(a, b) for a, b in zip(one_stream, outputs())):
        raise RuntimeError("GPTQ codes on four streams differ from those on one stream")
    # the layer with the four inputs' chains on four streams
    prewarm(args, lambda: run(concurrent=True))
    conc = []
    for _ in range(args.gptq_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(concurrent=True)
        e1.record(stream)
        torch.cuda.synchronize()
        conc.append(e0.elapsed_time(e1))
    if not all(torch.equal(a, b) for a, b in zip(one_stream, outputs())):
        raise RuntimeError("GPTQ codes of a timed four-stream pass differ from one stream")
    conc.sort()
    conc_ms = conc[len(conc) // 2]
    # per-stage times with the chains one after another on one stream
    reps = []
    for _ in range(args.gptq_reps):
        ev = {src: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for src in data}
        run(ev)
        torch.cuda.synchronize()
        reps.append({src: [e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                           e[2].elapsed_time(e[3])] for src, e in ev.items()})
    # the rep with the median layer time
    layer = sorted(reps, key=lambda r: sum(sum(v) for v in r.values()))[len(reps) // 2]
    seq_ms = sum(sum(v) for v in layer.values())
    layer_ms = min(conc_ms, seq_ms)
    weights = sum(r["n"] * r["k"] for d in data.values() for r in d["recs"])
    per_input = {}
    for src, (th, tf, tq) in layer.items():
        d = data[src]
        k = d["k"]
        flops = T * k * (k + 1)
        per_input[src] = {"k": k, "maps": [r["name"] for r in d["recs"]],
                          "hessian_us": round(th * 1e3, 1), "factor_us": round(tf * 1e3, 1),
                          "quantize_us": round(tq * 1e3, 1),
                          "hessian_TFLOP/s": round(flops / (th * 1e-3) / 1e12, 2)}
    dom = max(per_input, key=lambda s: per_input[s]["hessian_us"])
    dk = per_input[dom]["k"]
    h_us_per_launch = per_input[dom]["hessian_us"] / GPTQ_BATCHES
    tf = chunk * dk * (dk + 1) / (h_us_per_launch * 1e-6) / 1e12
    log(f"gptq layer {layer_ms:.2f} ms ({weights / (layer_ms * 1e-3) / 1e6:.1f} M weights/s; "
        f"4 streams {conc_ms:.2f} ms, one stream {seq_ms:.2f} ms); "
        + "; ".join(f"{s}: H {v['hessian_us']:.0f} us ({v['hessian_TFLOP/s']:.1f} TF), factor "
                    f"{v['factor_us']:.0f} us, codes {v['quantize_us']:.0f} us"
                    for s, v in per_input.items()))
    cpu = None if args.no_cpu_baseline else gptq_cpu_baseline()
    return {
        "workload": "GPTQ of one layer of the small model (width 512, feed-forward 1368): "
                    "q, k, v, o 512x512, gate and up 1368x512, down 512x1368, int4 group 64 "
                    "(72 for the 1368-input map); 65,536 calibration tokens per input in 8 "
                    "batches; H, damping 1%, factor, codes (maps sharing an input in one call)",
        "value": round(weights / (layer_ms * 1e-3), 1), "unit": "weights/s",
        "layer_ms": round(layer_ms, 3), "layer_ms_four_streams": round(conc_ms, 3),
        "layer_ms_one_stream": round(seq_ms, 3), "weights": weights, "reps": args.gptq_reps,
        "per_input": per_input,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP64_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / FP64_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("gptq_hessian_k1368"),
                     "kernel": f"qw_gptq_hessian (fp64 MFMA X^T X + fixed-order reduce), "
                               f"k={dk}, {chunk} tokens per launch",
                     "algorithmic_flops_per_launch": chunk * dk * (dk + 1),
                     "avg_launch_us": round(h_us_per_launch, 2)},
        "cpu_baseline": cpu,
    }


if __name__ == "__main__":
    main()
