"""Host logic of bench.py (no GPU): turning two rocprofv3 counter runs into the
traffic record, and reporting that record only while the kernel source it was
taken on is unchanged."""
import csv
import json
import os

import bench


def write_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow([r[0], r[1], r[2], counter, r[3]])


def test_traffic_record_scales_counters_by_the_calibration_copy(tmp_path, monkeypatch):
    plan = bench._traffic_plan("gemm")
    (gemm_name, gemm_grid), (_, pgrid) = plan["parts"]
    calib = plan["calib_bytes"]
    # Fetch counters read half the bytes (a 2x scale), write counters all of them.
    # A pack dispatch of another grid (another product's) is not counted.
    fetch = [(1, pgrid, "k_pack_scales(x)", 400.0), (2, pgrid + 256, "k_pack_scales(y)", 7.0),
             (3, gemm_grid, "k_gemm_mxfp4(GParams)", 1000.0), (4, gemm_grid, "k_gemm_mxfp4(GParams)", 3000.0),
             (5, 64, "__amd_rocclr_copyBuffer", 1.0), (9, 64, "__amd_rocclr_copyBuffer", calib / 2048)]
    write = [(1, pgrid, "k_pack_scales(x)", 40.0), (2, pgrid + 256, "k_pack_scales(y)", 7.0),
             (3, gemm_grid, "k_gemm_mxfp4(GParams)", 500.0), (4, gemm_grid, "k_gemm_mxfp4(GParams)", 500.0),
             (9, 64, "__amd_rocclr_copyBuffer", calib / 1024)]
    write_csv(tmp_path / "F", "FETCH_SIZE", fetch)
    write_csv(tmp_path / "W", "WRITE_SIZE", write)
    out = tmp_path / "rec.json"
    bench.write_traffic("gemm", str(tmp_path / "F"), str(tmp_path / "W"), str(out))
    rec = json.load(open(out))
    # per launch: fetch (400 + mean(1000, 3000)) KiB x 2, write (40 + 500) KiB x 1
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (2400 * 2 + 540) * 1024
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash("gemm")
    assert os.path.exists(str(out)[:-5] + ".md")
    # read_traffic reports it while the source hash matches, and not after
    monkeypatch.setitem(bench.TRAFFIC, "gemm", (bench.TRAFFIC["gemm"][0], str(out)))
    assert bench.read_traffic("gemm") == rec["hbm_bytes_per_launch"]
    rec["kernel_source_sha256_16"] = "0" * 16
    json.dump(rec, open(out, "w"))
    assert bench.read_traffic("gemm") is None

