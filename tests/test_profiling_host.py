"""The rocprofv3 summaries behind the committed profiles and the bench line's traffic figure
(host logic, no GPU): per-kernel statistics, HBM traffic scaled by a device copy's reading,
matrix-core busy fraction and clock, and the source-hash guard that stops a stale traffic
figure from being reported."""
import csv
import os

import pytest

from combine_dp_gather_amd import profiling

KNAME_GEMM = ("void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<true, false>"
              "(moe::(anonymous namespace)::GemmArgs, moe::gemm::TileOrder)")
KNAME_COPY = "void at::native::elementwise_kernel_manual_unroll<128, 4, direct_copy_kernel_cuda>(int)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_short_name_drops_arguments_and_namespaces():
    assert profiling.short_name(KNAME_GEMM) == "grouped_gemm_bf16_kernel<true, false>"
    assert profiling.short_name("void moe::(anonymous namespace)::gather_kernel<HIP_vector_type<unsigned int, 4u> >"
                                "(moe::(anonymous namespace)::SliceBatch, long)") == "gather_kernel<uint4 >"


def test_kernel_stats_reads_averages_in_microseconds(tmp_path):
    p = _write(tmp_path / "s.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                    "MaxNs", "StdDev"],
               [[KNAME_GEMM, 6, 7.2e6, 1.2e6, 55.0, 1.1e6, 1.3e6, 1.0]])
    (r,) = profiling.kernel_stats(p)
    assert r["name"] == "grouped_gemm_bf16_kernel<true, false>"
    assert r["calls"] == 6 and r["avg_us"] == pytest.approx(1200.0)
    assert r["min_us"] == pytest.approx(1100.0) and r["max_us"] == pytest.approx(1300.0)


def _counter_rows(counter, gemm_vals, copy_val):
    rows = [[KNAME_COPY, counter, copy_val, 0, 1000]]
    rows += [[KNAME_GEMM, counter, v, 0, 1000] for v in gemm_vals]
    return rows


def test_traffic_scales_each_counter_by_the_copy_reading(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # a 1024 MiB copy reads 524288 KiB on FETCH_SIZE (half) and 1048576 KiB on WRITE_SIZE
    f = _write(tmp_path / "f.csv", hdr, _counter_rows("FETCH_SIZE", [1000.0, 3000.0], 524288.0))
    w = _write(tmp_path / "w.csv", hdr, _counter_rows("WRITE_SIZE", [500.0], 1048576.0))
    res = profiling.traffic(f, w, 1024, "grouped_gemm_bf16_kernel<true, false>")
    assert res["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert res["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    assert res["FETCH_SIZE"]["bytes"] == pytest.approx(2000.0 * 1024 * 2.0)   # mean of two dispatches
    assert res["bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0 + 500.0 * 1024)
    with pytest.raises(SystemExit):
        profiling.traffic(f, w, 1024, "no_such_kernel")


def test_mfma_util_from_counters_and_agent(tmp_path):
    agent = _write(tmp_path / "a.csv", ["Agent_Type", "Simd_Count", "Num_Xcc", "Max_Engine_Clk_Fcompute"],
                   [["CPU", 0, 0, 0], ["GPU", 1024, 8, 2400]])
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # one 1 ms dispatch; GRBM_GUI_ACTIVE summed over 8 XCDs at 2000 MHz; half the SIMD cycles busy
    cycles = 2.0e6
    rows = [[1, KNAME_GEMM, "GRBM_GUI_ACTIVE", 8 * cycles, 0, 1_000_000],
            [1, KNAME_GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cycles * 1024, 0, 1_000_000],
            [1, KNAME_GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1.0e9, 0, 1_000_000],
            [2, "void other_kernel(int)", "GRBM_GUI_ACTIVE", 1.0, 0, 10],
            [2, "void other_kernel(int)", "SQ_VALU_MFMA_BUSY_CYCLES", 0.0, 0, 10]]
    cnt = _write(tmp_path / "c.csv", hdr, rows)
    geo = profiling.agent_geometry(agent)
    assert geo == {"simds": 1024, "xcds": 8, "max_mhz": 2400.0}
    (r,) = profiling.mfma_util(cnt, agent)     # kernels without matrix-core work are left out
    assert r["name"] == "grouped_gemm_bf16_kernel<true, false>"
    assert r["clock_mhz"] == pytest.approx(2000.0)
    assert r["mfma_busy"] == pytest.approx(0.5)
    assert r["counted_flops"] == pytest.approx(512.0e9)


def test_traffic_summary_is_ignored_once_sources_change(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    summary = tmp_path / "t.txt"
    digest = profiling.sources_sha256([str(src)])
    summary.write_text(f"kernel: k\nsource_sha256: {digest}\ntraffic_bytes_per_launch: 12345\n")
    assert profiling.read_traffic_summary(str(summary), [str(src)]) == 12345.0
    src.write_text("kernel v2\n")
    assert profiling.read_traffic_summary(str(summary), [str(src)]) is None
    assert profiling.read_traffic_summary(str(tmp_path / "missing.txt"), [str(src)]) is None


def test_committed_traffic_summaries_match_current_sources():
    """Every committed traffic summary names its kernel's sources; the bench only reports the
    figure while they hash the same, so a summary whose sources changed is reported as null."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prof = os.path.join(root, "profiles")
    seen = 0
    for name in sorted(os.listdir(prof)):
        if not name.endswith("__traffic.txt"):
            continue
        fields = dict(line.split(":", 1) for line in open(os.path.join(prof, name))
                      if line.split(":", 1)[0] in ("sources", "traffic_bytes_per_launch"))
        sources = fields["sources"].split()
        assert all(os.path.exists(os.path.join(root, s)) for s in sources), name
        assert float(fields["traffic_bytes_per_launch"]) > 0
        seen += 1
    assert seen >= 2
