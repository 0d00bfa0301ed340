"""The profile summarizer of bench.py (CPU): rocprofv3 counter CSVs in, HBM
bytes per launch out, scaled by the copy calibration."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(dirpath, rows):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": 1, "Kernel_Name": kernel,
                        "Counter_Name": counter, "Counter_Value": value})


def test_summary_scales_by_the_copy(tmp_path):
    gib_kib = (1 << 30) / 1024
    # the copy reads 1 GiB but the counter reports half of it; writes report in full
    _csv(tmp_path / "cf", [("copy_kernel", "FETCH_SIZE", gib_kib / 2)])
    _csv(tmp_path / "cw", [("copy_kernel", "WRITE_SIZE", gib_kib)])
    _csv(tmp_path / "f", [("ikbo_attn_bf16_w8_kernel<128, 2>", "FETCH_SIZE", 100.0),
                          ("ikbo_attn_bf16_w8_kernel<128, 2>", "FETCH_SIZE", 300.0),
                          ("ikbo_merge_kernel<128>", "FETCH_SIZE", 50.0)])
    _csv(tmp_path / "w", [("ikbo_attn_bf16_w8_kernel<128, 2>", "WRITE_SIZE", 10.0),
                          ("ikbo_merge_kernel<128>", "WRITE_SIZE", 5.0)])
    out = tmp_path / "s.json"
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-pmc", "--config", "c2_typical",
                    "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--copy-fetch",
                    str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"), "--out", str(out)],
                   check=True, stdout=subprocess.DEVNULL)
    s = json.loads(out.read_text())
    attn = s["kernels"]["ikbo_attn_bf16"]
    assert attn["read_bytes"] == 200.0 * 1024 * 2 and attn["write_bytes"] == 10.0 * 1024
    assert s["hbm_bytes_per_launch"] == attn["read_bytes"] + attn["write_bytes"]
    assert s["hbm_bytes_per_step_with_merge"] == s["hbm_bytes_per_launch"] + 50.0 * 1024 * 2 + 5.0 * 1024
    assert s["copy_calibration"]["fetch_scale"] == 2.0 and s["copy_calibration"]["write_scale"] == 1.0


def test_committed_traffic_summaries_load_only_on_their_sources(monkeypatch):
    """The roofline's traffic and the measured materialised ratio come from the
    committed summaries only while the kernel sources hash as they did when the
    counters were taken."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "ikbo_materialized_c2_typical_pmc.json")) as fh:
        mat = json.load(fh)
    assert mat["hbm_bytes_per_step_with_merge"] == sum(
        k["read_bytes"] + k["write_bytes"] for k in mat["kernels"].values())
    assert mat["kernels"]["ikbo_bcast_copy_kernel"]["dispatches"][0] > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a, **k: mat["kernel_source_hash"])
    assert bench.materialized_traffic_from_profiles("c2_typical") == mat["hbm_bytes_per_step_with_merge"]
    assert bench.materialized_traffic_from_profiles("c3_skewed") is None  # no summary for it
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a, **k: "0" * 16)
    assert bench.materialized_traffic_from_profiles("c2_typical") is None
    assert bench.traffic_from_profiles("c2_typical") is None
