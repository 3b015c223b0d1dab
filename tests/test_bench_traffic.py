"""The traffic record bench.py writes from two rocprofv3 PMC runs: counter
medians per kernel, scale factors from the calibration copy, bytes per launch
of the dominant kernel.  CPU only (synthetic counter files)."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({k: "0" for k in FIELDS} | {"Dispatch_Id": str(i), "Kernel_Name": name,
                                                   "Counter_Name": counter, "Counter_Value": str(value)})


def test_write_traffic_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    os.makedirs(tmp_path / "align_moe_route_amd" / "csrc")
    (tmp_path / "align_moe_route_amd" / "csrc" / "moe_route_sort.hip").write_text("// source")
    sel = "void (anonymous namespace)::k_select<32, 28, true, 1>((anonymous namespace)::Args)"
    scat = "(anonymous namespace)::k_scatter((anonymous namespace)::Args)"
    copy = "__amd_rocclr_copyBuffer"
    calib_mb = 64.0
    calib = 64000000
    # the copy's FETCH_SIZE counts half of what it reads (scale 2), WRITE_SIZE all of it (scale 1);
    # medians must ignore the outlier dispatches
    fetch = [(copy, calib / 2 / 1024), (copy, calib / 2 / 1024), (copy, 10),
             (sel, 7000), (sel, 7400), (sel, 90000), (scat, 700)]
    write = [(copy, calib / 1024), (copy, calib / 1024), (copy, 5),
             (sel, 2400), (sel, 2432), (sel, 2432), (scat, 1100)]
    _csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    js, md = bench.write_traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "prefill_skew",
                                        calib_mb, ["cmd1", "cmd2"])
    rec = json.load(open(js))
    assert os.path.basename(js) == "traffic_k_select_prefill_skew.json"
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == round(7400 * 1024 * 2.0)
    assert rec["write_bytes"] == 2432 * 1024
    assert rec["commands"] == ["cmd1", "cmd2"] and len(rec["source_sha256"]) == 64
    text = open(md).read()
    assert "k_select<32, 28, true, 1>" in text and "k_scatter" in text and "copyBuffer" not in text.split("|", 1)[1]
    # the record is used only while the source keeps its hash
    assert bench.traffic_record("k_select", "prefill_skew")["fetch_bytes"] == rec["fetch_bytes"]
    (tmp_path / "align_moe_route_amd" / "csrc" / "moe_route_sort.hip").write_text("// changed")
    assert bench.traffic_record("k_select", "prefill_skew") is None
