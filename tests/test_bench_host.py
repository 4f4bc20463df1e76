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



def test_trace_summary_takes_the_roofline_leg(tmp_path):
    """write_trace picks the leg's quantize launches (after warm-up, timed steps
    and one warm replay) and sets their kernel durations beside the events."""
    n_q = 4  # quantize launches per step: 2 tensors x (MXFP4, NVFP4)
    line = {"warmup": 1, "steps": 2, "value": 1.0, "ms_per_step": 1.0, "config": {"streams": 2},
            "roofline": {"launches": n_q, "frac": 0.5, "us_per_launch": 11.0,
                         "per_spec": {"mx32": {"us_per_launch": 10.5}, "nv16_dyn": {"us_per_launch": 11.5}}}}
    bl = tmp_path / "line.json"
    bl.write_text(json.dumps(line) + "\n")
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "bench_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writerow(["void k_quantize<0, 1, 16>(QParams)", 10, 1000, 100.0, 50, 150])
    rows, t = [], 0
    names = ["void fp4q::k_quantize_amax<0, true, true>(QParams)", "void fp4q::k_quantize<0, 1, 16>(QParams)"]
    for i in range(5 * n_q):  # warm-up, 2 timed steps, the warm replay, then the leg
        dur = (10000 if i % 2 == 0 else 11000) if 4 * n_q <= i < 5 * n_q else 99000
        rows.append([i + 1, names[i % 2], t, t + dur])
        rows.append([1000 + i, "k_finalize(StatsOut, int)", t, t + 1])
        t += dur + 10
    with open(d / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)
    out = tmp_path / "t.md"
    bench.write_trace("qwen14model", str(out), str(bl), str(d), "cmd")
    text = out.read_text()
    assert "| mx32 | 2 | 10.000 | 10.500 | +5.00 % |" in text
    assert "| nv16_dyn | 2 | 11.000 | 11.500 | +4.55 % |" in text


def test_counter_summary_per_chunk(tmp_path):
    """write_counters divides instruction counts by the layer's mean chunks per
    launch and names the counter sets it was given."""
    import fp4_workloads as wl
    chunks = sum(r * c for _, (r, c) in wl.QWEN14_PROJ) / len(wl.QWEN14_PROJ) / 512
    line = {"roofline": {"per_spec": {"mx32": {"us_per_launch": 20.0}, "nv16_dyn": {"us_per_launch": 25.0}}}}
    bl = tmp_path / "line.json"
    bl.write_text(json.dumps(line) + "\n")
    d = tmp_path / "pa"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerow([1, "void k_quantize_amax<0, true, true>(QParams)", "SQ_INSTS_VALU", 100 * chunks])
        w.writerow([2, "void k_quantize_amax<0, true, true>(QParams)", "SQ_INSTS_VALU", 140 * chunks])
        w.writerow([3, "void k_quantize<0, 1, 16, 0, true, true, false>(QParams)", "SQ_INSTS_VALU",
                    150 * chunks])
    out = tmp_path / "c.md"
    bench.write_counters("qwen14model", str(out), str(bl), [str(d)])
    text = out.read_text()
    assert "--pmc SQ_INSTS_VALU " in text
    assert f"| SQ_INSTS_VALU | {120 * chunks:,.2f} | 120.00 |" in text
    assert f"| SQ_INSTS_VALU | {150 * chunks:,.2f} | 150.00 |" in text
