"""CPU checks of bench.py's rocprofv3 summary arithmetic on synthetic counter
files shaped like rocprofv3's csv output: HBM traffic per launch scaled by a
plain copy's counter readings, MFMA-busy as busy cycles over per-XCD active
cycles times SIMDs, the shader clock, and the rule that a summary taken from
other kernel sources reads as absent."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FWD = "void mxgg::grouped_fwd_kernel<mxgg::TileCfg<256, 256, 2, 4, 128, 4, 0, 1, 7, 1> >(mxgg::RowsGemmParams)"
DGRAD = "void mxgg::grouped_dgrad_kernel<mxgg::TileCfg<256, 256, 2, 4, 128, 4, 0, 1, 7, 1> >(mxgg::RowsGemmParams)"
WGRAD = "void mxgg::grouped_wgrad_kernel<mxgg::TileCfg<256, 256, 2, 2, 128, 4, 0, 1, 7, 1> >(mxgg::WgradParams)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda>"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_mfma_busy_and_clock(tmp_path):
    # fwd (dispatch 1) and dgrad (dispatch 2) are separate kernel symbols; busy
    # is one row per dispatch, GRBM_GUI_ACTIVE the sum over 8 XCDs
    rows = [
        (1, FWD, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 400, 0, 500),
        (1, FWD, "GRBM_GUI_ACTIVE", 8 * 1000, 0, 500),
        (2, DGRAD, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250, 1000, 2000),
        (2, DGRAD, "GRBM_GUI_ACTIVE", 8 * 2000, 1000, 2000),
        (3, WGRAD, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 100, 3000, 3400),
        (3, WGRAD, "GRBM_GUI_ACTIVE", 8 * 800, 3000, 3400),
    ]
    pmc = tmp_path / "run_counter_collection.csv"
    _write(pmc, rows)
    with open(tmp_path / "run_agent_info.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Agent_Type", "Num_Xcc", "Simd_Count"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Num_Xcc": 1, "Simd_Count": 0})
        w.writerow({"Agent_Type": "GPU", "Num_Xcc": 8, "Simd_Count": 1024})
    kv = {}
    for line in bench.summarize_mfma(str(pmc)).splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert float(kv["fwd_mfma_busy_pct_median"]) == pytest.approx(40.0)      # 400 / 1000
    assert float(kv["dgrad_mfma_busy_pct_median"]) == pytest.approx(12.5)    # 250 / 2000
    assert float(kv["wgrad_mfma_busy_pct_median"]) == pytest.approx(12.5)    # 100 / 800
    assert float(kv["fwd_sclk_ghz_median"]) == pytest.approx(2.0)            # 1000 cycles / 500 ns
    assert float(kv["wgrad_sclk_ghz_median"]) == pytest.approx(2.0)


def test_traffic_scaled_by_copy_calibration(tmp_path):
    kib = 1024
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": WGRAD, "Calls": 1, "AverageNs": 700000, "MinNs": 690000, "MaxNs": 710000})
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # the wgrad dispatch counts 1000 KiB fetched and 3000 KiB written; the
    # 1 GiB copy reads as half its size fetched (x2) and its full size written
    _write(fetch, [(7, WGRAD, "FETCH_SIZE", 600, 0, 1), (7, WGRAD, "FETCH_SIZE", 400, 0, 1)])
    _write(write, [(7, WGRAD, "WRITE_SIZE", 3000, 0, 1)])
    _write(cfetch, [(1, COPY, "FETCH_SIZE", bench.COPY_BYTES / kib / 2, 0, 1)])
    _write(cwrite, [(1, COPY, "WRITE_SIZE", bench.COPY_BYTES / kib, 0, 1)])
    kv = {}
    for line in bench.summarize("wgrad", str(stats), str(fetch), str(write), str(cfetch), str(cwrite)).splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["hbm_fetch_bytes_per_launch"]) == pytest.approx(1000 * kib * 2)
    assert float(kv["hbm_write_bytes_per_launch"]) == pytest.approx(3000 * kib)
    assert kv["source_sha256_16"] == bench.source_hash("wgrad")


def test_stale_summaries_read_as_absent(tmp_path, monkeypatch):
    good = tmp_path / "gemm_fc1_mfma_busy.txt"
    good.write_text(f"wgrad_source_sha256_16: {bench.source_hash('wgrad')}\nwgrad_mfma_busy_pct_median: 12.00\n")
    monkeypatch.setattr(bench, "mfma_summary_path", lambda: str(good))
    assert bench.read_mfma_busy("wgrad") == pytest.approx(12.0)
    good.write_text("wgrad_source_sha256_16: 0000000000000000\nwgrad_mfma_busy_pct_median: 12.00\n")
    assert bench.read_mfma_busy("wgrad") is None
    traffic = tmp_path / "wgrad_fc1_traffic.txt"
    traffic.write_text("source_sha256_16: 0000000000000000\nhbm_fetch_bytes_per_launch: 1\n"
                       "hbm_write_bytes_per_launch: 2\n")
    monkeypatch.setattr(bench, "traffic_summary_path", lambda k, w="fc1": str(traffic))
    assert bench.read_traffic("wgrad") is None


def test_traffic_summary_names_its_workload(tmp_path):
    # a summary of another workload's kernel carries that workload's title and
    # commands, and is found under its own file name
    kib = 1024
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": WGRAD, "Calls": 1, "AverageNs": 2000000, "MinNs": 1, "MaxNs": 2})
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    _write(fetch, [(7, WGRAD, "FETCH_SIZE", 10, 0, 1)])
    _write(write, [(7, WGRAD, "WRITE_SIZE", 20, 0, 1)])
    _write(cfetch, [(1, COPY, "FETCH_SIZE", bench.COPY_BYTES / kib, 0, 1)])
    _write(cwrite, [(1, COPY, "WRITE_SIZE", bench.COPY_BYTES / kib, 0, 1)])
    text = bench.summarize("wgrad", str(stats), str(fetch), str(write), str(cfetch), str(cwrite),
                           workload="blockwise")
    assert bench.WORKLOAD_TITLES["blockwise"] in text
    assert "bench.py --workload blockwise --steps 3" in text
    assert bench.traffic_summary_path("wgrad", "blockwise").endswith("wgrad_blockwise_traffic.txt")



def test_fwd_and_dgrad_summaries_read_their_own_kernel(tmp_path):
    # the two passes have their own kernel symbols: each summary takes its
    # own stats row and its own dispatches' counters
    kib = 1024
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": DGRAD, "Calls": 5, "AverageNs": 300000, "MinNs": 290000, "MaxNs": 310000})
        w.writerow({"Name": FWD, "Calls": 5, "AverageNs": 270000, "MinNs": 260000, "MaxNs": 280000})
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    _write(fetch, [(1, FWD, "FETCH_SIZE", 100, 0, 1), (2, DGRAD, "FETCH_SIZE", 900, 0, 1),
                   (3, FWD, "FETCH_SIZE", 100, 0, 1), (4, DGRAD, "FETCH_SIZE", 900, 0, 1)])
    _write(write, [(1, FWD, "WRITE_SIZE", 10, 0, 1), (2, DGRAD, "WRITE_SIZE", 90, 0, 1)])
    _write(cfetch, [(1, COPY, "FETCH_SIZE", bench.COPY_BYTES / kib, 0, 1)])
    _write(cwrite, [(1, COPY, "WRITE_SIZE", bench.COPY_BYTES / kib, 0, 1)])

    def kv_of(kernel):
        out = {}
        for line in bench.summarize(kernel, str(stats), str(fetch), str(write), str(cfetch),
                                    str(cwrite)).splitlines():
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
        return out
    f, d = kv_of("fwd"), kv_of("dgrad")
    assert f["stats_average_ns"] == "270000" and d["stats_average_ns"] == "300000"
    assert float(f["hbm_fetch_bytes_per_launch"]) == pytest.approx(100 * kib)
    assert float(d["hbm_fetch_bytes_per_launch"]) == pytest.approx(900 * kib)
    assert float(d["hbm_write_bytes_per_launch"]) == pytest.approx(90 * kib)
