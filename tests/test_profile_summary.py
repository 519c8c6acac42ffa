"""bench.py --summarize-profile on synthetic rocprofv3 CSVs (CPU only): the
copy-kernel calibration, the per-launch HBM bytes, the algorithmic bytes and
the written summaries."""
import csv
import json
import os

import bench
import workloads


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


BWD = "void mn::kern::bwd_kernel<0, 0, 0, 0, 512, 8, 1, 3, 512, 1, 3>(mn::BwdArgs)"
FWD = "void mn::kern::fwd_kernel<0, 0, 256, 8, 2, 1, 256, 0, 3>(mn::FwdArgs)"
RED = "void mn::kern::reduce_kernel<16>(mn::ReduceArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_summary_of_synthetic_counters(tmp_path):
    wl = "rms_16384x4096"
    w = workloads.WORKLOADS[wl]
    nd2 = w.N * w.D * 2
    pre = str(tmp_path / "prof")
    _write(f"{pre}_trace/host/1_trace_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"],
           [[BWD, 10, 670000, 67000.0, 60.0, 66000, 68000, 1.0],
            [FWD, 10, 440000, 44000.0, 39.0, 43000, 45000, 1.0],
            [RED, 10, 45000, 4500.0, 1.0, 4000, 5000, 1.0],
            [COPY, 3, 150000, 50000.0, 0.5, 49000, 51000, 1.0]])
    _write(f"{pre}_trace/host/1_trace_kernel_trace.csv",
           ["Kind", "Kernel_Name", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Grid_Size_X"],
           [["KERNEL_DISPATCH", BWD, 192, 0, 144, 0, 56, 512, 131072],
            ["KERNEL_DISPATCH", FWD, 32, 0, 40, 0, 40, 256, 4194304]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the copy reads half its bytes in FETCH_SIZE KiB, writes all of them
    _write(f"{pre}_fetch/fetch_counter_collection.csv", hdr,
           [[COPY, "FETCH_SIZE", nd2 / 2048.0], [COPY, "FETCH_SIZE", 10.0],
            [BWD, "FETCH_SIZE", 2 * nd2 / 2048.0], [FWD, "FETCH_SIZE", nd2 / 2048.0]])
    _write(f"{pre}_write/write_counter_collection.csv", hdr,
           [[COPY, "WRITE_SIZE", nd2 / 1024.0], [BWD, "WRITE_SIZE", (nd2 + (4 << 20)) / 1024.0],
            [FWD, "WRITE_SIZE", nd2 / 1024.0]])
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profile(wl, pre, out_dir=str(out))
    t = json.loads((out / f"traffic_{wl}.json").read_text())
    assert abs(t["calibration"]["fetch_scale"] - 2.0) < 1e-12
    assert abs(t["calibration"]["write_scale"] - 1.0) < 1e-12
    b = t["kernels"]["backward_rows"]
    fb, bb = bench.alg_bytes("rms", w.N, w.D)
    assert b["algorithmic_bytes_per_launch"] == bb
    assert b["fetch_bytes_per_launch"] == 2 * nd2
    assert b["write_bytes_per_launch"] == nd2 + (4 << 20)
    assert abs(b["algorithmic_GBps_at_avg"] - bb / 67000e-9 / 1e9) < 1e-6
    assert b["resources"]["Workgroup_Size_X"] == "512"
    assert t["kernels"]["forward"]["hbm_bytes_per_launch"] == 2 * nd2
    assert "reduce_partials" in t["kernels"]
    assert t["kernel_source_sha256_16"] == bench.kernel_hash("rms")
    md = (out / f"{wl}_trace_and_traffic.md").read_text()
    assert "rocprofv3 --pmc FETCH_SIZE" in md and "--summarize-profile" in md
    assert "| backward_rows |" in md
    # bench's roofline reads the measured traffic back while the source hash matches
    assert bench.measured_traffic.__code__.co_argcount == 2


def test_multi_kernel_groupnorm_backward_traffic():
    """A GroupNorm backward that runs as sums, merge and apply kernels plus the
    column reduce (the channels-last layout, and slices beyond one workgroup)
    reports the summed counter bytes of all four in its roofline; a one-kernel
    backward reports its row kernel's."""
    for wl in ("gn_nlc_32x4096x320_g32", "gn_32x320x16384_g32"):
        labels = bench.backward_traffic_labels(wl)
        assert labels == bench.GN_MULTI_BACKWARD, wl
        with open(os.path.join(bench.ROOT, "profiles", f"traffic_{wl}.json")) as f:
            ks = json.load(f)["kernels"]
        want = sum(ks[k]["hbm_bytes_per_launch"] for k in labels)
        assert bench.measured_traffic(wl, labels) == want
        # X and dY are fetched twice, dX written once
        w = workloads.WORKLOADS[wl]
        assert want > 1.5 * bench.alg_bytes("gn", w.N, w.D, C=w.channels, G=w.groups)[1]
    assert bench.backward_traffic_labels("gn_32x320x4096_g32") == "backward_rows"
    assert bench.backward_traffic_labels("rms_16384x4096") == "backward_rows"
