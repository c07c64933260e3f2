"""Host-side check of bench.py's rocprofv3 summarizer: dispatches in
dispatch order are assigned to the profile-run manifest's workloads by their
launch counts, warm-up launches are left out, torch's own kernels are
ignored, counter runs are merged and calibrated by the copy's known bytes."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FWD = "void mxfp4::(anonymous namespace)::row_fwd_kernel<1, 32, 0, 0, 1, 64>(mxfp4::(anonymous namespace)::RowArgs)"
COPY = "void (anonymous namespace)::probe_kernel<1, false, 1>(unsigned char const*, unsigned char*, unsigned char*, long, unsigned long*)"
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(int, float)"


def manifest(tmp):
    m = {"entries": [
        {"label": "calibration: probe copy", "kernel": "probe_kernel", "launches": 2, "alg_read": 1 << 20,
         "alg_write": 1 << 20, "alg_bytes": 2 << 20, "skip": True},
        {"label": "calibration: probe copy", "kernel": "probe_kernel", "launches": 2, "alg_read": 1 << 20,
         "alg_write": 1 << 20, "alg_bytes": 2 << 20, "skip": False},
        {"label": "weight_4k forward (y + bitmap)", "kernel": "row_fwd_kernel", "launches": 1, "alg_read": 4096,
         "alg_write": 4352, "alg_bytes": 8448, "skip": True},
        {"label": "weight_4k forward (y + bitmap)", "kernel": "row_fwd_kernel", "launches": 3, "alg_read": 4096,
         "alg_write": 4352, "alg_bytes": 8448, "skip": False}]}
    p = tmp / "m.json"
    p.write_text(json.dumps(m))
    return str(p)


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary(tmp_path):
    man = manifest(tmp_path)
    rows, t = [], 1000
    for name, dur in [(COPY, 500), (TORCH, 5), (COPY, 500), (COPY, 400), (COPY, 400),
                      (FWD, 99), (FWD, 10), (TORCH, 5), (FWD, 20), (FWD, 30)]:
        rows.append([name, t, t + dur])
        t += 2000
    write_csv(str(tmp_path / "tr" / "h" / "x_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              rows)
    out = tmp_path / "t.md"
    bench.summarize("trace", str(tmp_path / "tr"), man, str(out), "cmd")
    d = json.loads((tmp_path / "t.json").read_text())
    fwd = [r for r in d["rows"] if r["label"].startswith("weight_4k")][0]
    assert abs(fwd["avg_us"] - 0.020) < 1e-9          # (10 + 20 + 30) ns / 3, warm-up 99 left out
    cal = [r for r in d["rows"] if r["label"].startswith("calibration")][0]
    assert abs(cal["avg_us"] - 0.4) < 1e-9


def test_counter_summary_and_traffic(tmp_path):
    man = manifest(tmp_path)
    # FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them (KiB)
    seq = [COPY, COPY, COPY, COPY, FWD, FWD, FWD, FWD]
    fetch = [512, 512, 512, 512, 2, 2, 2, 2]
    write = [1024, 1024, 1024, 1024, 4.25, 4.25, 4.25, 4.25]
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(str(tmp_path / "f" / "a" / "r_counter_collection.csv"), hdr,
              [[i + 1, k, "FETCH_SIZE", v] for i, (k, v) in enumerate(zip(seq, fetch))] + [[99, TORCH, "FETCH_SIZE", 7]])
    write_csv(str(tmp_path / "w" / "a" / "r_counter_collection.csv"), hdr,
              [[i + 1, k, "WRITE_SIZE", v] for i, (k, v) in enumerate(zip(seq, write))])
    out = tmp_path / "c.md"
    bench.summarize("pmc", f"{tmp_path / 'f'},{tmp_path / 'w'}", man, str(out), "cmd")
    d = json.loads((tmp_path / "c.json").read_text())
    fwd = [r for r in d["rows"] if r["label"].startswith("weight_4k")][0]
    assert abs(fwd["fetch_scale"] - 2.0) < 1e-12 and abs(fwd["write_scale"] - 1.0) < 1e-12
    assert abs(fwd["read_bytes"] - 4096) < 1e-6 and abs(fwd["write_bytes"] - 4352) < 1e-6
    assert abs(fwd["traffic_over_alg"] - 1.0) < 1e-12
    bench.traffic_json(str(tmp_path / "c.json"), str(tmp_path / "traffic.json"))
    t = json.loads((tmp_path / "traffic.json").read_text())
    assert t["traffic_bytes_per_launch"] == 8448 and t["kernel_source_sha"] == bench.kernel_source_sha()


def test_bench_trace_summary(tmp_path):
    """The plain bench command's trace: this library's launches grouped by
    kernel and launch size (torch's left out), with the bench line's own
    roofline timing quoted beside them."""
    rows, t = [], 1000
    for name, grid, wg, dur in [(FWD, 2097152, 64, 12000), (TORCH, 64, 64, 5), (FWD, 2097152, 64, 14000),
                                (FWD, 29360128, 64, 145000), (COPY, 256, 256, 700)]:
        rows.append([name, grid, wg, t, t + dur])
        t += 200000
    write_csv(str(tmp_path / "tr" / "h" / "x_kernel_trace.csv"),
              ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"], rows)
    line = {"value": 5400.0, "unit": "GB/s", "ms_per_step": 0.0254,
            "roofline": {"kernel": "row_fwd", "achieved": 5300.0, "alg_bytes_per_launch": 69206016.0,
                         "frac": 0.6625}}
    (tmp_path / "b.json").write_text("warm-up text\n" + json.dumps(line) + "\n")
    out = tmp_path / "bt.md"
    bench.summarize_bench_trace(str(tmp_path / "tr"), str(tmp_path / "b.json"), str(out), "cmd")
    d = json.loads((tmp_path / "bt.json").read_text())
    by = {(r["kernel"], r["grid"]): r for r in d["rows"]}
    assert len(by) == 3                                   # two sizes of the forward, the probe; no torch
    small = by[("row_fwd_kernel<1, 32, 0, 0, 1, 64>", 2097152)]
    assert small["launches"] == 2 and abs(small["avg_us"] - 13.0) < 1e-9
    assert "13.06 us per launch by HIP events" in out.read_text()   # 69206016 B / 5300 GB/s
