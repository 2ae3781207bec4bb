#!/usr/bin/env python3
"""Throughput of the top-k sparse MQA hot path (forward + backward) on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input: the forward
(O, LSE), then the backward on those outputs (Delta preprocess, dQ kernel, and the dKV stage:
the staging plan (selection bitmap, scan, positions), the dKV kernel writing each pair's
contribution row, and the per-row reduction that also emits the bf16 dKV). Inputs are resident in HBM before timing starts.

Prints one JSON line. `value` is the step's algorithmic TFLOP/s: (4 + 10) * H * D flops per valid
(token, slot) pair (forward 4HD: QK^T and PV; backward 10HD: score recompute, dP, dQ, dKV) divided
by the measured step time. Per-kernel times come from HIP events recorded on the stream the
kernels run on; the dKV stage runs as its three library steps (prepare, partials, reduce) so the
partials kernel is timed alone.

`roofline` is for the longest single-kernel step, with its own algorithmic flops per valid pair
(forward 4HD; dQ kernel 6HD: S and dP recompute, dQ; dKV partials kernel 8HD: S and dP recompute,
dS^T Q and P^T dO). `traffic` is that kernel's HBM bytes per launch from the rocprofv3 FETCH_SIZE
and WRITE_SIZE summary under profiles/, scaled by the same counters' reading for a copy of known
size, and null once the kernel source differs from the one the counters were taken on.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--calibration-copy]
  python bench.py --summarize-pmc FETCH.csv WRITE.csv --out profiles/hbm_traffic_<workload>.md
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
CALIB_BYTES = 1 << 30        # the calibration copy reads and writes this many bytes
CALIB_KERNEL = "MulFunctor"  # part of the name of the kernel torch.mul(src, 1.0, out=dst) runs
REPO = os.path.dirname(os.path.abspath(__file__))


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
    p.add_argument("--out", help="output file of --summarize-pmc")
    p.add_argument("--serial", action="store_true",
                   help="run every kernel on one stream (default: the dKV staging plan on a side stream)")
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
        self.nan = float("nan")

    def _check(self, name, st):
        if st != 0:
            raise RuntimeError(f"{name}: status {st} {self.lib.sparse_mqa_status_string(st).decode()}")

    def run(self, timed: bool):
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
        if timed:
            self.events.append(ev)

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
             f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --calibration-copy",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o pmc -- python bench.py --workload "
             f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --calibration-copy",
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
            "sample": (f"fp32 oracle: forward + dQ for the last {n_tok} tokens ({pairs} valid pairs) and dKV for "
                       f"kv rows 0..{len(rows) - 1} ({refs} references); {secs:.1f} s "
                       f"(fwd {t1 - t0:.1f} s, dQ {t2 - t1:.1f} s, dKV {t3 - t2:.1f} s)")}


def main():
    args = parse()
    if args.summarize_pmc:
        if not args.out:
            raise SystemExit("--summarize-pmc needs --out")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.workload)
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
    step = Step(smqa, w, x, overlap=not args.serial)
    if args.calibration_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step.run(timed=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step.run(timed=True)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    # per-kernel event times (each kernel bracketed on the stream it runs on)
    ms = step.kernel_ms()
    ms_step = total_ms / args.steps

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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(w.describe(), valid_pairs=n_valid, step="forward + backward",
                       schedule="serial" if args.serial else "dkv prepare on a side stream"),
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
        "wall_s_timed": round(wall, 3),
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
    # staged dKV rows written by the partials kernel: D fp16 values per valid pair and head block
    out["dkv_staging_write_TBps"] = round(n_valid * (w.H // min(w.H, 64)) * 2 * w.D / (ms["bwd_dkv_partials"] * 1e-3)
                                          / 1e12, 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w, valid)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
