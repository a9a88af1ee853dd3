"""Host-side logic of bench.py and the counter summary: the traffic figure is scaled by the copy
calibration and is only reported while the kernel sources are the ones that were measured."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dynamic_block_sparse_pool_amd import traffic  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for i, (k, c, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scales_by_copy_calibration(tmp_path, monkeypatch):
    attn = "dbsp::attn_fwd_bf16_kernel(unsigned short const*, ...)"
    write_csv(tmp_path / "f.csv", [("other", "FETCH_SIZE", 5.0), (attn, "FETCH_SIZE", 1000.0),
                                   (attn, "FETCH_SIZE", 3000.0)])
    write_csv(tmp_path / "w.csv", [(attn, "WRITE_SIZE", 64.0)])
    # the copy of 1 GiB counts half its reads and all its writes
    write_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    write_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "t.json"
    traffic.main(["--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                  "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
                  "--workload", "final_720p_clip2", "--out", str(out), "--command", "test"])
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["traffic_bytes"] == 2000 * 1024 * 2 + 64 * 1024
    assert t["source_sha256"] == bench.attn_source_hash()

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.stored_traffic("final_720p_clip2") == t["traffic_bytes"]
    assert bench.stored_traffic("dit_mass") is None
    t["source_sha256"] = "0" * 64  # taken on other kernel sources
    out.write_text(json.dumps(t))
    assert bench.stored_traffic("final_720p_clip2") is None


def test_traffic_summary_rejects_missing_kernel(tmp_path):
    write_csv(tmp_path / "f.csv", [("other", "FETCH_SIZE", 5.0)])
    with pytest.raises(SystemExit):
        traffic.mean_counter(str(tmp_path / "f.csv"), "FETCH_SIZE", traffic.KERNEL)


def test_percentiles():
    assert bench.percentiles([5.0, 1.0, 3.0, 2.0, 4.0]) == (1.0, 3.0, 5.0)
    assert bench.percentiles([7.0]) == (7.0, 7.0, 7.0)
