"""Host logic of bench.py, on the CPU: the one-GPU contract and the HBM-traffic summary that feeds
the roofline object's `traffic` (counter files are synthetic here; no GPU, no profiler)."""
import csv
import json
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path):
    calib = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float> >(int)"
    dkv = "void smqa::bwd_dkv_ws_kernel<512, 4>(unsigned short const*)"
    fwd = "void smqa::fwd_ws_kernel<512>(unsigned short const*)"
    kib = bench.CALIB_BYTES / 1024
    # the copy's FETCH counter reads half its bytes (scale 2), WRITE reads them exactly (scale 1)
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(calib, kib / 2), (dkv, 1000.0), (dkv, 1002.0), (fwd, 10.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(calib, kib), (dkv, 3000.0), (fwd, 5.0)])
    out = tmp_path / "hbm.md"
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out), "some_workload")
    text = out.read_text()
    block = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert block["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert block["calibration"]["write_scale"] == pytest.approx(1.0)
    k = block["kernels"]["bwd_dkv_partials"]
    assert k["kernel"].startswith("smqa::bwd_dkv_ws_kernel")
    assert k["fetch_bytes"] == round(1001.0 * 1024 * 2.0)  # mean of the two dispatches, scaled
    assert k["write_bytes"] == round(3000.0 * 1024)
    assert block["kernels"]["fwd"]["fetch_bytes"] == round(10.0 * 1024 * 2.0)
    assert "bwd_dkv_dq" not in block["kernels"]  # no dispatch of it in the files


def test_traffic_is_null_once_the_kernel_source_changes(tmp_path, monkeypatch):
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    current = bench.source_sha256(bench.SINGLE["bwd_dkv_partials"][1])  # the kernel sources as they are
    summary = {"workload": "w", "kernels": {"bwd_dkv_partials": {
        "kernel": "k", "fetch_bytes": 7, "write_bytes": 11, "source_sha256": current}}}
    (profiles / "hbm_traffic_w.md").write_text("x\n```json\n" + json.dumps(summary) + "\n```\n")
    # the summary is read from a scratch tree; the sources still hash as they are
    monkeypatch.setattr(bench, "REPO", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha256", lambda files: current)
    assert bench.traffic_for("bwd_dkv_partials", "w") == 18
    summary["kernels"]["bwd_dkv_partials"]["source_sha256"] = "0" * 64
    (profiles / "hbm_traffic_w.md").write_text("x\n```json\n" + json.dumps(summary) + "\n```\n")
    assert bench.traffic_for("bwd_dkv_partials", "w") is None
    assert bench.traffic_for("bwd_dkv_partials", "missing_workload") is None
    assert bench.traffic_for("bwd_preprocess", "w") is None  # not a single-kernel step
