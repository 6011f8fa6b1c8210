"""CPU checks of the profiling helpers behind bench.py's roofline.traffic:
the copy calibration, the per-pass sum over the phase schedule's kernels,
the single-kernel summary, and the digest guard that withholds a record
once the measured sources change.  The inputs are small synthetic rocprofv3
CSV files with known counter values, so every expected byte count follows
from the calibration by hand."""
import csv
import json

import pytest

from combine_wave_level_amd import profiling

MIB = 1 << 20


def _pmc_csv(path, rows):
    """rows: (kernel name, counter, value) -> a counter-collection CSV."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    return str(path)


@pytest.fixture
def calib(tmp_path):
    # a 1024 MiB copy: FETCH_SIZE reads half of the bytes moved, WRITE_SIZE all of them
    cf = _pmc_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512 * 1024)] * 2)
    cw = _pmc_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024 * 1024)] * 2)
    return cf, cw


def test_step_traffic_sums_the_calibrated_kernels(tmp_path, calib):
    cf, cw = calib
    fetch = _pmc_csv(tmp_path / "f.csv", [
        ("void moe::gemm1_phase_kernel<FfnLarge, true>(...)", "FETCH_SIZE", 100 * 1024),
        ("void moe::gemm1_phase_kernel<FfnLarge, true>(...)", "FETCH_SIZE", 300 * 1024),  # mean 200 MiB
        ("void moe::gemm2_phase_kernel<FfnLarge>(...)", "FETCH_SIZE", 50 * 1024),
        ("void moe::combine_kernel<true>(...)", "FETCH_SIZE", 10 * 1024),
        ("router_logits_mfma_kernel", "FETCH_SIZE", 999 * 1024),          # not one of the kernels
    ])
    write = _pmc_csv(tmp_path / "w.csv", [
        ("void moe::gemm1_phase_kernel<FfnLarge, true>(...)", "WRITE_SIZE", 8 * 1024),
        ("void moe::gemm2_phase_kernel<FfnLarge>(...)", "WRITE_SIZE", 16 * 1024),
        ("void moe::combine_kernel<true>(...)", "WRITE_SIZE", 4 * 1024),
    ])
    md, js = str(tmp_path / "t.md"), str(tmp_path / "t.json")
    profiling.main(["steptraffic", "--fetch", fetch, "--write", write, "--copy-fetch", cf, "--copy-write", cw,
                    "--copy-kernel", "copyBuffer", "--kernels", "gemm1_phase_kernel", "gemm2_phase_kernel",
                    "combine_kernel", "--title", "t", "--command", "cmd", "--out-md", md, "--out-json", js,
                    "--workload", "mid", "--T", "4096"])
    rec = json.load(open(js))
    # reads: (200 + 50 + 10) MiB of FETCH_SIZE / 0.5 per byte; writes: 28 MiB / 1.0
    assert rec["fetch_bytes"] == 520 * MIB
    assert rec["write_bytes"] == 28 * MIB
    assert rec["traffic_bytes"] == 548 * MIB
    assert rec["fetch_factor"] == 0.5 and rec["write_factor"] == 1.0
    assert rec["kernel"] == "phase_kernels" and rec["workload"] == "mid" and rec["T"] == 4096
    assert "= 574.6 MB." in open(md).read()                          # 548 MiB in MB
    # bench.py takes the record for this workload and T while the sources match
    assert profiling.load_traffic(js, "mid", 4096)["traffic_bytes"] == 548 * MIB
    assert profiling.load_traffic(js, "mid", 2048) is None
    assert profiling.load_traffic(js, "stress", 4096) is None
    rec["source_digest"] = "0" * 64                                   # sources changed since
    stale = str(tmp_path / "stale.json")
    json.dump(rec, open(stale, "w"))
    assert profiling.load_traffic(stale, "mid", 4096) is None
    assert profiling.load_traffic(str(tmp_path / "missing.json"), "mid", 4096) is None


def test_summarize_one_kernel(tmp_path, calib):
    cf, cw = calib
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void moe::ffn_waved_kernel<FfnLarge, true, true>(WaveArgs)", "Calls": 10,
                    "TotalDurationNs": 5_000_000, "AverageNs": 500_000, "MinNs": 490_000, "MaxNs": 520_000})
    fetch = _pmc_csv(tmp_path / "f.csv", [("ffn_waved_kernel<FfnLarge, true, true>", "FETCH_SIZE", 600 * 1024)])
    write = _pmc_csv(tmp_path / "w.csv", [("ffn_waved_kernel<FfnLarge, true, true>", "WRITE_SIZE", 200 * 1024)])
    md, js = str(tmp_path / "s.md"), str(tmp_path / "s.json")
    profiling.main(["summarize", "--stats", str(stats), "--fetch", fetch, "--write", write, "--copy-fetch", cf,
                    "--copy-write", cw, "--copy-kernel", "copyBuffer", "--kernel", "ffn_waved_kernel",
                    "--workload", "mid", "--T", "4096", "--command", "cmd", "--out-md", md, "--out-json", js])
    rec = json.load(open(js))
    assert rec["fetch_bytes"] == 1200 * MIB and rec["write_bytes"] == 200 * MIB
    assert rec["avg_us"] == 500.0
    assert rec["source_digest"] == profiling.source_digest("ffn_waved_kernel")
    assert profiling.load_traffic(js, "mid", 4096)["traffic_bytes"] == 1400 * MIB


def test_step_traffic_json_needs_the_workload(tmp_path, calib):
    cf, cw = calib
    fetch = _pmc_csv(tmp_path / "f.csv", [("gemm1_phase_kernel", "FETCH_SIZE", 1024)])
    write = _pmc_csv(tmp_path / "w.csv", [("gemm1_phase_kernel", "WRITE_SIZE", 1024)])
    with pytest.raises(SystemExit):
        profiling.main(["steptraffic", "--fetch", fetch, "--write", write, "--copy-fetch", cf, "--copy-write", cw,
                        "--copy-kernel", "copyBuffer", "--kernels", "gemm1_phase_kernel", "--title", "t",
                        "--out-md", str(tmp_path / "x.md"), "--out-json", str(tmp_path / "x.json")])
