#!/usr/bin/env python3
"""Throughput of the top-k sparse MQA hot path (forward + backward) on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input: the forward
(O, LSE), then the backward on those outputs: the Delta preprocess, the staging plan (selection
bitmap, scan, positions; on a second stream beside the forward), the dKV partials kernel writing
each pair's contribution row and the dS, dQ from that dS, and the per-row reduction that also
emits the bf16 dKV. Inputs are resident in HBM before timing starts.

Prints one JSON line. `value` is the step's algorithmic TFLOP/s: (4 + 10) * H * D flops per valid
(token, slot) pair (forward 4HD: QK^T and PV; backward 10HD: score recompute, dP, dQ, dKV) divided
by the measured step time, which is taken with events around each step only. Per-kernel times come
from as many steps again with HIP events recorded around every kernel on the stream it runs on;
the backward runs as its library steps (preprocess, prepare, partials, dq, reduce), so each kernel
is timed alone.

`roofline` is for the longest single-kernel step, with its own algorithmic flops per valid pair
(forward 4HD; dQ from the stored dS 2HD; dKV partials kernel 8HD: S and dP recompute, dS^T Q and
P^T dO). `traffic` is that kernel's HBM bytes per launch from the rocprofv3 FETCH_SIZE
and WRITE_SIZE summary under profiles/, scaled by the same counters' reading for a copy of known
size, and null once the kernel source differs from the one the counters were taken on.

Beside the headline line's warm-cache step time it reports a cold-cache step time (each step
preceded by a 1 GiB write that evicts L2 and the Infinity Cache), the rate counted over all
B*S*topk slots (nominal) next to the valid pairs, and, as `gather_bound`, the same step timed on
the batched gather workload (B=4, S=2048, S_kv=65536, uniform indices with masked slots) with each
gathering kernel's row-gather rate against the HBM peak, in the bench's schedule and with every
kernel alone on one stream (`serial`).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--calibration-copy] [--cold-steps C] [--gather-workload NAME] [--gather-steps G]
  python bench.py --summarize-pmc FETCH.csv WRITE.csv --out profiles/hbm_traffic_<workload>.md
  python bench.py --summarize-trace KERNEL_STATS.csv --out profiles/kernel_trace_<workload>.md
  python bench.py --summarize-counters PASS1.csv [PASS2.csv ...] --out profiles/counters_<workload>.md
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

METRIC = "sparse-MQA fwd/bwd TFLOP/s and % bf16 MFMA peak @ H=64 D=512 topk=2048"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
KERNELS = ("fwd", "bwd_preprocess", "bwd_dkv_prepare", "bwd_dkv_partials", "bwd_dkv_dq", "bwd_dkv_reduce")
# single-kernel steps: rocprofv3 kernel name prefix, source files, algorithmic flops per valid pair / (H*D)
SINGLE = {
    "fwd": ("smqa::fwd_", ("fwd.hip", "device_common.h"), 4),  # fwd_ws_kernel at H=64k D=512
    # bwd_dkv_ws_kernel: S and dP recompute, dS^T Q and P^T dO
    "bwd_dkv_partials": ("smqa::bwd_dkv_", ("bwd.hip", "device_common.h"), 8),
    "bwd_dkv_dq": ("smqa::bwd_dq_ds_", ("bwd.hip", "device_common.h"), 2),  # dS K from the stored dS
}
GATHER_KERNELS = ("fwd", "bwd_dkv_partials", "bwd_dkv_dq")  # each gathers one kv row per valid pair
FLUSH_BYTES = 1 << 30        # written before each cold-cache step (L2 4 MiB per XCD, Infinity Cache 256 MiB)
CALIB_BYTES = 1 << 30        # the calibration copy reads and writes this many bytes
CALIB_KERNEL = "MulFunctor"  # part of the name of the kernel torch.mul(src, 1.0, out=dst) runs
REPO = os.path.dirname(os.path.abspath(__file__))
# bench arguments of every profiled run (a short run of the one workload)
PROFILE_STEPS, PROFILE_WARMUP = 8, 2
PROFILE_ARGS = f"--steps {PROFILE_STEPS} --warmup {PROFILE_WARMUP} --no-cpu-baseline --cold-steps 0 --gather-steps 0"
# kernels the counter summary reports, in this order
COUNTER_KERNELS = ("fwd_ws_kernel", "bwd_dkv_ws_kernel", "bwd_dq_ds_kernel", "reduce_rows_kernel", "delta_kernel",
                   "mark_kernel", "position_kernel")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="causal_h64_d512_k2048")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibration-copy", action="store_true",
                   help="run one 1 GiB copy kernel before the warmup (reference for the HBM byte counters)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM traffic summary from two rocprofv3 --pmc counter_collection.csv files")
    p.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                   help="write the kernel-time summary from a rocprofv3 --kernel-trace --stats kernel_stats.csv")
    p.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                   help="write the counter summary from rocprofv3 --pmc counter_collection.csv files (one per pass)")
    p.add_argument("--out", help="output file of --summarize-*")
    p.add_argument("--serial", action="store_true",
                   help="run every kernel on one stream (default: the dKV staging plan on a side stream)")
    p.add_argument("--cold-steps", type=int, default=5,
                   help="steps timed after a cache-evicting write each (0: none)")
    p.add_argument("--gather-workload", default="gather_b4_skv64k",
                   help="workload of the gather_bound object ('none': skip it)")
    p.add_argument("--gather-steps", type=int, default=5)
    return p.parse_args()


class Step:
    """Preallocated buffers and the library calls of one fwd+bwd step (no allocation inside)."""

    def __init__(self, smqa, w, x, overlap: bool = True):
        self.lib = smqa.load_library()
        self.w = w
        dev = torch.device("cuda:0")
        self.q = x["q"].to(dev)
        self.kv = x["kv"].to(dev)
        self.sink = x["attn_sink"].to(dev)
        self.idx = x["topk_idxs"].to(dev)
        self.do = x["do"].to(dev)
        B, S, S_kv, H, D = w.B, w.S, w.S_kv, w.H, w.D
        self.o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, S, H), dtype=torch.float32, device=dev)
        self.delta = torch.empty((B, S, H), dtype=torch.float32, device=dev)
        self.dq = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
        self.dkv = torch.empty((B, S_kv, D), dtype=torch.bfloat16, device=dev)
        # one pass over all tokens (the dKV steps need it)
        self.ws_bytes = self.lib.sparse_mqa_bwd_workspace_bytes(B, S, S_kv, H, D, w.topk)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        # The dKV staging plan (prepare) reads only topk_idxs, so it runs on a second stream (default
        # priority) beside the forward, preprocess and dQ kernels; the partials wait for it.
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self.events = []  # one {kernel: (start, end)} per timed step
        self.step_events = []  # one (start, end) per timed step, on the main stream
        self.nan = float("nan")

    def _check(self, name, st):
        if st != 0:
            raise RuntimeError(f"{name}: status {st} {self.lib.sparse_mqa_status_string(st).decode()}")

    def run(self, timed: bool, step_event: bool = False):
        """One step; timed: events around every kernel and the step, step_event: around the step only."""
        w, L = self.w, self.lib
        B, S, S_kv, H, D, K = w.B, w.S, w.S_kv, w.H, w.D, w.topk
        p = lambda t: t.data_ptr()  # noqa: E731
        calls = {
            "fwd": lambda h: L.sparse_mqa_fwd(p(self.q), p(self.kv), p(self.sink), p(self.idx), p(self.o),
                                            p(self.lse), B, S, S_kv, H, D, K, self.nan, 0, h),
            "bwd_preprocess": lambda h: L.sparse_mqa_bwd_preprocess(p(self.o), p(self.do), p(self.delta), B, S, H, D, h),
            "bwd_dkv_dq": lambda h: L.sparse_mqa_bwd_dkv_dq(p(self.kv), p(self.idx), p(self.dq), p(self.ws),
                                                          self.ws_bytes, B, S, S_kv, H, D, K, self.nan, h),
            "bwd_dkv_prepare": lambda h: L.sparse_mqa_bwd_dkv_prepare(p(self.idx), p(self.ws), self.ws_bytes,
                                                                    B, S, S_kv, H, D, K, h),
            "bwd_dkv_partials": lambda h: L.sparse_mqa_bwd_dkv_partials(
                p(self.q), p(self.kv), p(self.do), p(self.idx), p(self.lse), p(self.delta), p(self.ws),
                self.ws_bytes, B, S, S_kv, H, D, K, self.nan, h),
            "bwd_dkv_reduce": lambda h: L.sparse_mqa_bwd_dkv_reduce(p(self.dkv), 0, p(self.ws), self.ws_bytes,
                                                                  B, S, S_kv, H, D, K, h),
        }
        ev = {}

        def launch(k, st):
            if timed:
                ev[k] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[k][0].record(st)
            self._check(k, calls[k](st.cuda_stream))
            if timed:
                ev[k][1].record(st)

        if timed or step_event:
            st_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            st_ev[0].record(self.stream)
        if self.side is None:
            for k in KERNELS:
                launch(k, self.stream)
        else:
            # prepare on the side stream once the previous step's dKV kernels are enqueued before it
            go = torch.cuda.Event()
            go.record(self.stream)
            self.side.wait_event(go)
            launch("bwd_dkv_prepare", self.side)
            ready = torch.cuda.Event()
            ready.record(self.side)
            for k in ("fwd", "bwd_preprocess"):
                launch(k, self.stream)
            self.stream.wait_event(ready)
            for k in ("bwd_dkv_partials", "bwd_dkv_dq", "bwd_dkv_reduce"):
                launch(k, self.stream)
        if timed or step_event:
            st_ev[1].record(self.stream)  # the side stream joined the main one before the partials
            self.step_events.append(st_ev)
        if timed:
            self.events.append(ev)

    def step_ms_median(self):
        import statistics
        return statistics.median(a.elapsed_time(b) for a, b in self.step_events)

    def kernel_ms(self):
        """Average event-timed duration of each kernel over the timed steps."""
        n = len(self.events)
        return {k: sum(e[k][0].elapsed_time(e[k][1]) for e in self.events) / n for k in KERNELS}


def source_sha256(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(REPO, "top_sparse_mqa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def summarize_pmc(fetch_csv: str, write_csv: str, out_path: str, workload: str) -> None:
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two rocprofv3 --pmc runs,
    scaled by the same counters' reading for the calibration copy (CALIB_BYTES read and written)."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.mean(v) for k, v in vals.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    calib = [k for k in fetch if CALIB_KERNEL in k]
    if not calib:
        raise SystemExit("no calibration copy kernel in the counter files (run with --calibration-copy)")
    f_scale = CALIB_BYTES / (fetch[calib[0]] * 1024.0)
    w_scale = CALIB_BYTES / (write[calib[0]] * 1024.0)
    kernels = {}
    for step, (prefix, files, _) in SINGLE.items():
        names = [k for k in fetch if k.startswith("void " + prefix) or k.startswith(prefix)]
        if not names:
            continue
        k = names[0]
        kernels[step] = {"kernel": k.split("(")[0].replace("void ", ""),
                         "fetch_bytes": round(fetch[k] * 1024.0 * f_scale),
                         "write_bytes": round(write.get(k, 0.0) * 1024.0 * w_scale),
                         "source_sha256": source_sha256(files)}
    summary = {"workload": workload, "calibration": {"bytes": CALIB_BYTES, "fetch_KiB": fetch[calib[0]],
                                                     "write_KiB": write[calib[0]], "fetch_scale": f_scale,
                                                     "write_scale": w_scale},
               "kernels": kernels}
    lines = [f"# HBM traffic per launch: {workload}", "",
             "rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), two separate runs, averaged per kernel,",
             f"each scaled by the same counter's reading for a copy kernel that reads and writes {CALIB_BYTES} bytes.",
             "", "Commands (from the repository root on one MI355X; `<out>` an output directory):", "", "```",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o pmc -- python bench.py --workload "
             f"{workload} {PROFILE_ARGS} --calibration-copy",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o pmc -- python bench.py --workload "
             f"{workload} {PROFILE_ARGS} --calibration-copy",
             "python bench.py --summarize-pmc <out>/fetch/pmc_counter_collection.csv "
             f"<out>/write/pmc_counter_collection.csv --workload {workload} --out <this file>", "```", "",
             "| step | kernel | fetch (GB) | write (GB) |", "|---|---|---|---|"]
    for step, k in kernels.items():
        lines.append(f"| {step} | `{k['kernel']}` | {k['fetch_bytes'] / 1e9:.3f} | {k['write_bytes'] / 1e9:.3f} |")
    lines += ["", f"Calibration: copy read {fetch[calib[0]]:.0f} KiB and wrote {write[calib[0]]:.0f} KiB for "
              f"{CALIB_BYTES // 1024} KiB each (scales {f_scale:.4f}, {w_scale:.4f}).", "",
              "Machine-readable (bench.py reads this block):", "", "```json", json.dumps(summary, indent=1), "```"]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def traffic_for(step: str, workload: str):
    """HBM bytes per launch of a single-kernel step from the committed summary, or None when there
    is none for this workload or the kernel source changed since the counters were taken."""
    path = os.path.join(REPO, "profiles", f"hbm_traffic_{workload}.md")
    if step not in SINGLE or not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        k = json.loads(block)["kernels"][step]
    except (IndexError, KeyError, ValueError):
        return None
    if k["source_sha256"] != source_sha256(SINGLE[step][1]):
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def summarize_trace(stats_csv: str, out_path: str, workload: str) -> None:
    """Kernel times of a rocprofv3 --kernel-trace --stats run as a table: the statistics over every
    dispatch, and, from the per-dispatch trace beside it, the mean over the last PROFILE_STEPS
    dispatches of each kernel: the steps with events around every kernel, which the bench line's
    kernel times cover."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    timed = {}
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if os.path.exists(trace_csv):
        per = {}
        for r in csv.DictReader(open(trace_csv)):
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        for k, v in per.items():
            v.sort()
            last = [d for _, d in v[-PROFILE_STEPS:]]
            timed[k] = sum(last) / len(last)
    lines = [f"# Kernel trace: {workload}", "",
             f"rocprofv3 kernel-trace statistics of a short bench run ({PROFILE_WARMUP} warmup steps, {PROFILE_STEPS} timed "
             f"steps, then {PROFILE_STEPS} steps with events around every kernel): every dispatch, and the mean over "
             "the last of these, whose times the bench line's kernel times are.", "",
             "Command (from the repository root on one MI355X; `<out>` an output directory):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o trace -- python bench.py "
             f"--workload {workload} {PROFILE_ARGS}",
             f"python bench.py --workload {workload} --summarize-trace <out>/trace_kernel_stats.csv --out <this file>",
             "```", "", "| kernel | calls | avg (us) | avg, last steps (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        t = f"{timed[r['Name']] / 1e3:.1f}" if r["Name"] in timed else ""
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {t} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += ["", "Library steps to kernels: fwd = `fwd_ws_kernel`; bwd_preprocess = `delta_kernel`;",
              "bwd_dkv_prepare = `fill_zero_kernel` + `mark_kernel` + three scan kernels + `position_kernel`;",
              "bwd_dkv_partials = `kv_row_norm_kernel` + `bwd_dkv_ws_kernel`; bwd_dkv_dq = `bwd_dq_ds_kernel`;",
              "bwd_dkv_reduce = `reduce_rows_kernel`. The staging plan (bwd_dkv_prepare) runs on a second stream",
              "beside the forward and the preprocess, so their durations include that overlap."]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counter_table(paths):
    """{kernel: {counter: mean over dispatches}} and {kernel: mean duration ns} from --pmc csv files."""
    import csv
    from collections import defaultdict

    vals = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    passes = []
    for p in paths:
        names = []
        for r in csv.DictReader(open(p)):
            k = next((k for k in COUNTER_KERNELS if k in r["Kernel_Name"]), None)
            if r["Counter_Name"] not in names:
                names.append(r["Counter_Name"])
            if k is None:
                continue
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        passes.append(names)
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    return mean, {k: sum(v) / len(v) for k, v in dur.items()}, passes


def derived_counters(a: dict, dur_ns: float) -> dict:
    """Utilisations from raw counter means of one kernel. GRBM_GUI_ACTIVE is summed over the 8 XCDs,
    so a kernel's clock count is a eighth of it; per-CU counters (TA, TD, TCP, SQ_LDS_*) are summed over
    256 CUs and SQ_VALU_MFMA_BUSY_CYCLES over their 1024 SIMDs."""
    out = {}
    if "GRBM_GUI_ACTIVE" not in a:
        return out
    cyc = a["GRBM_GUI_ACTIVE"] / 8
    out["clock_GHz"] = cyc / dur_ns
    per_cu = lambda c: a[c] / (cyc * 256)  # noqa: E731
    if "SQ_VALU_MFMA_BUSY_CYCLES" in a:
        out["mfma_busy"] = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024)
    if "VmemLatency" in a:
        out["vmem_latency_cycles"] = a["VmemLatency"]
    if "SQ_WAVE_CYCLES" in a and "SQ_WAIT_INST_ANY" in a:
        out["wave_wait_dependency"] = a["SQ_WAIT_INST_ANY"] / a["SQ_WAVE_CYCLES"]
    if "SQ_WAVE_CYCLES" in a and "SQ_ACTIVE_INST_ANY" in a:
        out["wave_issuing"] = a["SQ_ACTIVE_INST_ANY"] / a["SQ_WAVE_CYCLES"]
    for c, n in (("TA_TA_BUSY_sum", "ta_busy"), ("TA_ADDR_STALLED_BY_TC_CYCLES_sum", "ta_stalled_by_tc"),
                 ("TD_TD_BUSY_sum", "td_busy"), ("TD_TC_STALL_sum", "td_tc_stall"),
                 ("SQ_LDS_IDX_ACTIVE", "lds_active")):
        if c in a:
            out[n] = per_cu(c)
    if "TCC_HIT_sum" in a and "TCC_MISS_sum" in a:
        out["l2_hit"] = a["TCC_HIT_sum"] / max(a["TCC_HIT_sum"] + a["TCC_MISS_sum"], 1.0)
    if "SQ_LDS_BANK_CONFLICT" in a and "SQ_LDS_IDX_ACTIVE" in a:
        out["lds_bank_conflict"] = a["SQ_LDS_BANK_CONFLICT"] / max(a["SQ_LDS_IDX_ACTIVE"], 1.0)
    if "TCP_TCC_READ_REQ_LATENCY_sum" in a and "TCP_TCC_READ_REQ_sum" in a:
        out["l1_l2_read_latency_cycles"] = a["TCP_TCC_READ_REQ_LATENCY_sum"] / max(a["TCP_TCC_READ_REQ_sum"], 1.0)
    if "TCP_UTCL1_TRANSLATION_MISS_sum" in a and "TCP_UTCL1_REQUEST_sum" in a:
        out["utcl1_miss"] = a["TCP_UTCL1_TRANSLATION_MISS_sum"] / max(a["TCP_UTCL1_REQUEST_sum"], 1.0)
    return out


DERIVED_DOC = {
    "clock_GHz": "GRBM_GUI_ACTIVE / 8 over the dispatch duration",
    "mfma_busy": "SQ_VALU_MFMA_BUSY_CYCLES / (clocks x 1024 SIMDs)",
    "vmem_latency_cycles": "VmemLatency (derived: average vector-memory instruction latency)",
    "wave_wait_dependency": "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
    "wave_issuing": "SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES",
    "ta_busy": "TA_TA_BUSY_sum / (clocks x 256 CUs)",
    "ta_stalled_by_tc": "TA_ADDR_STALLED_BY_TC_CYCLES_sum / (clocks x 256)",
    "td_busy": "TD_TD_BUSY_sum / (clocks x 256)",
    "td_tc_stall": "TD_TC_STALL_sum / (clocks x 256)",
    "lds_active": "SQ_LDS_IDX_ACTIVE / (clocks x 256)",
    "lds_bank_conflict": "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
    "l2_hit": "TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)",
    "l1_l2_read_latency_cycles": "TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum",
    "utcl1_miss": "TCP_UTCL1_TRANSLATION_MISS_sum / TCP_UTCL1_REQUEST_sum",
}


def summarize_counters(paths, out_path: str, workload: str) -> None:
    """Per-kernel utilisation table from rocprofv3 --pmc passes over the same short bench run."""
    mean, dur, passes = counter_table(paths)
    lines = [f"# Hardware counters: {workload}", "",
             "rocprofv3 --pmc passes (one run each, counters averaged over every dispatch of a kernel), over the",
             "same short bench run. Commands (from the repository root on one MI355X; `<out>` an output directory):",
             "", "```"]
    for i, names in enumerate(passes):
        lines.append(f"rocprofv3 --pmc {' '.join(names)} --output-format csv -d <out>/p{i} -o pmc -- "
                     f"python bench.py --workload {workload} {PROFILE_ARGS}")
    lines.append("python bench.py --workload " + workload + " --summarize-counters "
                 + " ".join(f"<out>/p{i}/pmc_counter_collection.csv" for i in range(len(passes))) + " --out <this file>")
    lines += ["```", ""]
    table = {k: derived_counters(mean[k], dur[k]) for k in COUNTER_KERNELS if k in mean}
    cols = [c for c in DERIVED_DOC if any(c in v for v in table.values())]
    lines += ["| kernel | avg (us) | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for k, v in table.items():
        cells = [(f"{v[c]:.0f}" if c.endswith("cycles") else f"{v[c]:.3f}") if c in v else "" for c in cols]
        lines.append(f"| `{k}` | {dur[k] / 1e3:.0f} | " + " | ".join(cells) + " |")
    lines += ["", "Columns:", ""] + [f"- `{c}`: {DERIVED_DOC[c]}" for c in cols]
    lines += ["", "Raw means per dispatch:", "", "```json",
              json.dumps({k: {c: round(x, 1) for c, x in sorted(mean[k].items())} for k in table}, indent=1), "```"]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def cpu_baseline(x, w, valid_per_token):
    """The oracle as it stands, on a bounded sample of the same workload (about 10 s of CPU work at
    the headline shape): forward and dQ for all tokens (at most 4096), dKV for the first 1536 kv rows."""
    import oracle

    n_tok = min(4096, w.B * w.S)
    toks = list(range(w.B * w.S - n_tok, w.B * w.S))
    rows = list(range(0, min(1536, w.B * w.S_kv)))
    t0 = time.perf_counter()
    o, lse = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], tokens=toks)
    O = torch.zeros(w.B * w.S, w.H, w.D, dtype=torch.bfloat16)
    Ls = torch.zeros(w.B * w.S, w.H)
    O[toks] = o.to(torch.bfloat16)
    Ls[toks] = lse
    t1 = time.perf_counter()
    oracle.dq(x["q"], x["kv"], O.view(w.B, w.S, w.H, w.D), x["do"], x["topk_idxs"], Ls.view(w.B, w.S, w.H),
              tokens=toks)
    t2 = time.perf_counter()
    # dKV rows: every token referencing them needs O/LSE; the sample's LSE rows are filled only for
    # the sampled tokens, which is enough to time the arithmetic (the values are not checked here)
    oracle.dkv(x["q"], x["kv"], O.view(w.B, w.S, w.H, w.D), x["do"], x["topk_idxs"], Ls.view(w.B, w.S, w.H),
               rows=rows)
    t3 = time.perf_counter()
    pairs = int(valid_per_token[toks].sum())
    idx = x["topk_idxs"].reshape(w.B, -1).long()
    ok = (idx >= 0) & (idx < w.S_kv)
    flat = (idx + torch.arange(w.B).view(-1, 1) * w.S_kv)[ok]
    refs = int(torch.bincount(flat, minlength=w.B * w.S_kv)[rows].sum())
    flops = 4 * w.H * w.D * pairs + 6 * w.H * w.D * pairs + 10 * w.H * w.D * refs
    secs = t3 - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            **cpu_info(),
            "sample": (f"fp32 oracle: forward + dQ for the last {n_tok} tokens ({pairs} valid pairs) and dKV for "
                       f"kv rows 0..{len(rows) - 1} ({refs} references); {secs:.1f} s "
                       f"(fwd {t1 - t0:.1f} s, dQ {t2 - t1:.1f} s, dKV {t3 - t2:.1f} s)")}


def cpu_info():
    """CPU model and the cores this process may run on (its affinity mask)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = sorted(os.sched_getaffinity(0))
    return {"cpu_model": model, "affinity_cores": len(aff), "affinity": f"{aff[0]}-{aff[-1]}" if aff else ""}


def measure(smqa, w, x, steps, warmup, overlap=True, cold_steps=0, calibration_copy=False):
    """Warm step time over `steps` steps (after `warmup`), with events around each step only; then
    per-kernel event times over as many steps again (events around every kernel, which add a few
    hundredths of a millisecond per step, so they stay out of the step time); then, if cold_steps,
    the step time with a cache-evicting write before each step (outside the timed span)."""
    step = Step(smqa, w, x, overlap=overlap)
    if calibration_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(warmup):
        step.run(timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step.run(timed=False, step_event=True)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = {"ms_step": start.elapsed_time(end) / steps, "wall": wall, "ms_step_median": step.step_ms_median()}
    step.events = []
    for _ in range(steps):
        step.run(timed=True)
    torch.cuda.synchronize()
    res["ms"] = step.kernel_ms()
    if cold_steps > 0:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        tot = 0.0
        for _ in range(cold_steps):  # step times
            flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step.run(timed=False)
            b.record()
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        res["cold_ms_step"] = tot / cold_steps
        step.events = []
        for _ in range(cold_steps):  # kernel times
            flush.zero_()
            step.run(timed=True)
            torch.cuda.synchronize()
        res["cold_ms"] = step.kernel_ms()
        del flush
    del step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def gather_rates(w, n_valid, ms):
    """Row-gather rate of each gathering kernel (one D-wide bf16 kv row per valid pair) and the staging
    rows the reduce reads (D int16 values per valid pair and 64-head block), in GB/s and as a fraction
    of the HBM peak. Rows served from L2 or the Infinity Cache count the same, so a fraction above 1
    is possible."""
    row = w.D * 2
    out = {}
    for k in GATHER_KERNELS:
        gbs = n_valid * row / (ms[k] * 1e-3) / 1e9
        out[k] = {"GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    gbs = n_valid * max(1, w.H // 64) * row / (ms["bwd_dkv_reduce"] * 1e-3) / 1e9
    out["bwd_dkv_reduce"] = {"GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                             "bytes": "staging rows read"}
    return out


def algorithmic_bytes(w, n_valid):
    """HBM bytes of one step by the method's own accounting, per valid pair and per token/row: two
    row gathers (forward, backward) of 2D bytes and a 4D-byte dKV scatter per pair; per token the q
    and O streams of the forward, O and dO of the preprocess, q, dO and dQ of the backward (2HD
    bytes each), the indices (4 per slot, read by the forward and the backward); per kv row the
    accumulator's zero and postprocess (10D)."""
    tokens, HD = w.B * w.S, w.H * w.D
    return (n_valid * (2 * 2 * w.D + 4 * w.D) + tokens * 7 * 2 * HD + 2 * tokens * w.topk * 4
            + w.B * w.S_kv * 10 * w.D)


def main():
    args = parse()
    if args.summarize_pmc:
        if not args.out:
            raise SystemExit("--summarize-pmc needs --out")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.workload)
        return
    if args.summarize_trace or args.summarize_counters:
        if not args.out:
            raise SystemExit("--summarize-trace / --summarize-counters need --out")
        if args.summarize_trace:
            summarize_trace(args.summarize_trace, args.out, args.workload)
        else:
            summarize_counters(args.summarize_counters, args.out, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU (got --gpus {args.gpus}): the kernels run on a single device and "
              "no multi-GPU path exists", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import top_sparse_mqa_amd as smqa
    from top_sparse_mqa_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = syn.WORKLOADS[args.workload]
    x = syn.workload_inputs(w)
    valid = ((x["topk_idxs"] >= 0) & (x["topk_idxs"] < w.S_kv)).sum(-1).view(-1)
    n_valid = int(valid.sum())
    n_nominal = w.B * w.S * w.topk
    r = measure(smqa, w, x, args.steps, args.warmup, overlap=not args.serial, cold_steps=args.cold_steps,
                calibration_copy=args.calibration_copy)
    ms, ms_step = r["ms"], r["ms_step"]

    HD = w.H * w.D
    fl_fwd = 4 * HD * n_valid
    fl_bwd = 10 * HD * n_valid
    ms_fwd = ms["fwd"]
    ms_bwd = sum(ms[k] for k in KERNELS if k.startswith("bwd"))
    tflops = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
    dom = max(SINGLE, key=lambda k: ms[k])
    ach = SINGLE[dom][2] * HD * n_valid / (ms[dom] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(r["ms_step_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "operand_dtypes": ("bf16 inputs, outputs and MFMA operands; fp16 (hi + lo split) P and dS operands in the "
                           "dKV products; fp32 accumulation; int16 block floating point dKV staging rows"),
        "data": "synthetic",
        "config": dict(w.describe(), valid_pairs=n_valid, step="forward + backward",
                       schedule="serial" if args.serial else "dkv prepare on a side stream"),
        "flops_per_valid_pair": {"fwd": 4 * HD, "bwd": 10 * HD},
        "nominal_pairs": n_nominal,
        "nominal_tflops": round((fl_fwd + fl_bwd) / n_valid * n_nominal / (ms_step * 1e-3) / 1e12, 3),
        "fwd_ms": round(ms_fwd, 4),
        "bwd_ms": round(ms_bwd, 4),
        "fwd_tflops": round(fl_fwd / (ms_fwd * 1e-3) / 1e12, 2),
        "bwd_tflops": round(fl_bwd / (ms_bwd * 1e-3) / 1e12, 2),
        "fwd_frac_mfma_peak": round(fl_fwd / (ms_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_mfma_peak": round(fl_bwd / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_gather_GBps": round(n_valid * 2 * w.D / (ms_fwd * 1e-3) / 1e9, 1),
        "fwd_gather_frac_hbm": round(n_valid * 2 * w.D / (ms_fwd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "kernel_ms": {k: round(v, 4) for k, v in ms.items()},
        "wall_s_timed": round(r["wall"], 3),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(ach, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(dom, args.workload),
        },
    }
    if "cold_ms_step" in r:
        out["cold_cache"] = {"steps": args.cold_steps, "ms_per_step": round(r["cold_ms_step"], 4),
                             "tflops": round((fl_fwd + fl_bwd) / (r["cold_ms_step"] * 1e-3) / 1e12, 3),
                             "kernel_ms": {k: round(v, 4) for k, v in r["cold_ms"].items()},
                             "flush": f"{FLUSH_BYTES >> 20} MiB write before each step, outside the timed span"}
    # staged dKV rows written by the partials kernel: D int16 values per valid pair and head block
    out["dkv_staging_write_TBps"] = round(n_valid * (w.H // min(w.H, 64)) * 2 * w.D / (ms["bwd_dkv_partials"] * 1e-3)
                                          / 1e12, 3)
    if args.gather_workload != "none" and args.gather_steps > 0:
        wg = syn.WORKLOADS[args.gather_workload]
        xg = syn.workload_inputs(wg)
        ng = int(((xg["topk_idxs"] >= 0) & (xg["topk_idxs"] < wg.S_kv)).sum())
        rg = measure(smqa, wg, xg, args.gather_steps, 1, overlap=not args.serial)
        # the same steps on one stream: each kernel alone on the GPU (the forward's gather rate
        # without the staging plan beside it)
        rs = rg if args.serial else measure(smqa, wg, xg, args.gather_steps, 1, overlap=False)
        del xg
        HDg = wg.H * wg.D
        out["gather_bound"] = {
            "config": dict(wg.describe(), valid_pairs=ng, nominal_pairs=wg.B * wg.S * wg.topk),
            "steps": args.gather_steps, "warmup": 1,
            "ms_per_step": round(rg["ms_step"], 4),
            "tflops": round(14 * HDg * ng / (rg["ms_step"] * 1e-3) / 1e12, 3),
            "kernel_ms": {k: round(v, 4) for k, v in rg["ms"].items()},
            "gather": gather_rates(wg, ng, rg["ms"]),
            "serial": {"ms_per_step": round(rs["ms_step"], 4),
                       "kernel_ms": {k: round(v, 4) for k, v in rs["ms"].items()},
                       "gather": gather_rates(wg, ng, rs["ms"])},
            "step_algorithmic_GB": round(algorithmic_bytes(wg, ng) / 1e9, 2),
            "step_algorithmic_GBps": round(algorithmic_bytes(wg, ng) / (rg["ms_step"] * 1e-3) / 1e9, 1),
            "step_algorithmic_frac_hbm": round(algorithmic_bytes(wg, ng) / (rg["ms_step"] * 1e-3) / 1e9
                                               / PEAK_HBM_GBS, 4),
            "hbm_peak_GBps": PEAK_HBM_GBS,
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w, valid)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
