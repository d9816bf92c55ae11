"""The bench's profiling summaries (host logic, CPU only): per-kernel counter arithmetic, the HBM byte
scaling from the device copy, the gate that keeps stale traffic figures out of the bench line, and the
per-phase power and clock table.  The CSV files are small synthetic stand-ins with the columns rocprofv3
writes; the power log imitates `amd-smi metric --power --clock --json` output."""
import csv
import json
import math
import os

import pytest

import bench

KERNEL = "void moe::k_gemm_bf16_w4p<0, false, 4, true>(moe::GemmParams, int)"
COPY = "__amd_rocclr_copyBuffer"
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"]
TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
              "Correlation_Id", "Start_Timestamp", "End_Timestamp"]


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, "0") for c in cols})


def _pmc_run(d, dispatches):
    """dispatches: [(dispatch id, kernel, start ns, end ns, {counter: [values, one row per XCD or SE]})]"""
    crow, trow = [], []
    for did, name, t0, t1, counters in dispatches:
        trow.append({"Dispatch_Id": did, "Correlation_Id": did, "Kernel_Name": name, "Start_Timestamp": t0,
                     "End_Timestamp": t1})
        for cname, vals in counters.items():
            for v in vals:
                crow.append({"Dispatch_Id": did, "Correlation_Id": did, "Kernel_Name": name, "Counter_Name": cname,
                             "Counter_Value": v, "Start_Timestamp": t0, "End_Timestamp": t1})
    _write(os.path.join(d, "run_counter_collection.csv"), COUNTER_COLS, crow)
    _write(os.path.join(d, "run_kernel_trace.csv"), TRACE_COLS, trow)


def test_counter_summary_arithmetic(tmp_path):
    simds = 1024
    dur_ns = 2_000_000                     # 2 ms dispatches
    clock_ghz = 1.5
    grbm = clock_ghz * dur_ns              # cycles of the busiest XCD
    util = 60.0                            # percent
    busy = util / 100 * grbm * simds       # summed over all SIMDs (split over two rows below)
    mops = 1.0e9
    pmc = str(tmp_path / "pmc")
    _pmc_run(pmc, [
        (1, KERNEL, 0, dur_ns, {"MfmaUtil": [util], "SQ_VALU_MFMA_BUSY_CYCLES": [busy / 2, busy / 2],
                                "SQ_INSTS_VALU_MFMA_MOPS_BF16": [mops]}),
        (2, KERNEL, 10 * dur_ns, 11 * dur_ns, {"MfmaUtil": [util], "SQ_VALU_MFMA_BUSY_CYCLES": [busy],
                                               "SQ_INSTS_VALU_MFMA_MOPS_BF16": [mops]}),
        (3, COPY, 20 * dur_ns, 21 * dur_ns, {"MfmaUtil": [0.0], "SQ_VALU_MFMA_BUSY_CYCLES": [0.0]}),
    ])
    # FETCH_SIZE counts the copy's 1 GiB of reads as 512 MiB (128-byte requests counted as 64 bytes),
    # WRITE_SIZE its 1 GiB of writes as 1 GiB: scales 2 and 1
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _pmc_run(fetch, [(1, KERNEL, 0, dur_ns, {"FETCH_SIZE": [1000.0, 3000.0]}),
                     (2, COPY, 0, dur_ns, {"FETCH_SIZE": [524288.0]})])
    _pmc_run(write, [(1, KERNEL, 0, dur_ns, {"WRITE_SIZE": [500.0]}),
                     (2, COPY, 0, dur_ns, {"WRITE_SIZE": [1048576.0]})])
    text, res = bench.counter_summary(pmc, fetch, write)
    k = "k_gemm_bf16_w4p<0, false, 4, true>"
    r = res[k]
    assert r["dispatches"] == 2
    assert r["avg_ms"] == pytest.approx(2.0)
    assert r["mfma_busy_pct"] == pytest.approx(util)
    assert r["clock_ghz"] == pytest.approx(clock_ghz)
    assert r["executed_tflops"] == pytest.approx(mops * 512 / 2e-3 / 1e12)
    assert r["read_bytes"] == pytest.approx(4000.0 * 1024 * 2.0)
    assert r["write_bytes"] == pytest.approx(500.0 * 1024 * 1.0)
    assert "x 2.000" in text and "x 1.000" in text
    # short dispatches get no clock (the counter window includes the profiler's own set-up)
    assert math.isnan(res[bench._short(COPY)]["clock_ghz"])


def test_rocprof_summary_and_traffic_gate(tmp_path, monkeypatch):
    trace = tmp_path / "trace"
    trace.mkdir()
    with open(trace / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([KERNEL, 4, 28_000_000, 7_000_000, 60.0])
        w.writerow([COPY, 2, 600_000, 300_000, 1.0])
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _pmc_run(fetch, [(1, KERNEL, 0, 1, {"FETCH_SIZE": [10_000_000.0]}), (2, COPY, 0, 1, {"FETCH_SIZE": [524288.0]})])
    _pmc_run(write, [(1, KERNEL, 0, 1, {"WRITE_SIZE": [512_000.0]}), (2, COPY, 0, 1, {"WRITE_SIZE": [1048576.0]})])
    out_json = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "hash-a")
    text, res = bench.rocprof_summary(str(trace), fetch, write, out_json=out_json)
    assert res["avg_ms"] == pytest.approx(7.0)
    assert res["traffic_bytes_per_launch"] == pytest.approx(10_000_000 * 1024 * 2.0 + 512_000 * 1024)
    assert "| k_gemm_bf16_w4p<0, false, 4, true> | 4 | 7.0000 |" in text
    with open(out_json) as fh:
        assert json.load(fh)["source_sha256"] == "hash-a"
    # the bench line carries the figure only for the kernel and the sources it was taken on
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out_json)
    assert bench.measured_traffic("k_gemm_bf16_w4p<0, false, 4, true>") == pytest.approx(
        res["traffic_bytes_per_launch"])
    assert bench.measured_traffic("k_gemm_bf16_w4<0, true>") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "hash-b")
    assert bench.measured_traffic("k_gemm_bf16_w4p<0, false, 4, true>") is None


def test_committed_traffic_figure_matches_the_sources():
    """The committed traffic summary names the dominant kernel of the default bench run; when it was
    taken on the current kernel sources, the bench line reports it (else null, by the gate above)."""
    with open(os.path.join(bench.ROOT, bench.TRAFFIC_FILE)) as fh:
        t = json.load(fh)
    assert t["dominant_kernel"] == bench.dominant_kernel(True)
    assert t["traffic_bytes_per_launch"] > 0
    assert t["fetch_scale"] == pytest.approx(2.0, rel=1e-3)
    assert t["write_scale"] == pytest.approx(1.0, rel=1e-3)


def test_power_summary_per_phase(tmp_path):
    def sample(t, phase, watts, clocks):
        g = {"gpu": 0, "power": {"socket_power": {"value": watts, "unit": "W"}},
             "clock": {"gfx_%d" % i: {"clk": {"value": c, "unit": "MHz"}} for i, c in enumerate(clocks)}}
        return "t=%.3f phase=%s\n%s\n" % (t, phase, json.dumps({"gpu_data": [g]}, indent=1))
    log = tmp_path / "samples.log"
    log.write_text(sample(0.0, "setup", 250, [100] * 8) + sample(0.1, "prefill", 1398, [1600] * 8) +
                   sample(0.2, "prefill", 1402, [1580, 1620] * 4) + sample(0.3, "prefill", 1400, [1600] * 8) +
                   sample(0.4, "decode", 1270, [2380] * 8) + "t=0.5 phase=decode\nnot json\n")
    text, rows = bench.power_summary(str(log))
    assert len(rows) == 5
    assert "| prefill | 3 | 1400 / 1402 | 1600 |" in text
    assert "| decode | 1 | 1270 / 1270 | 2380 |" in text
    assert "1 samples with the GPU idle" in text and "median 250 W" in text
