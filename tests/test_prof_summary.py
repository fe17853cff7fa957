"""Host logic of the rocprofv3 summariser (profiles/ files): kernel-trace
tables and the calibrated HBM-traffic figure, on small hand-made CSVs."""
import csv
import hashlib

from decode_step_06_amd import prof_summary as ps


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_table_and_last_n_mean(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    rows = [["void ns::gemv_bf16_kernel<1, unsigned short>(int)", 0, 4000],
            ["void ns::attn_decode_kernel<unsigned short, 64, 7, 4>(int)", 5000, 17000],
            ["void ns::attn_decode_kernel<unsigned short, 64, 7, 4>(int)", 20000, 30000],
            ["void ns::attn_decode_kernel<unsigned short, 64, 7, 4>(int)", 31000, 39000],
            ["void at::native::other(int)", 40000, 90000]]
    _write(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    ps.main(["trace", str(p), "--title", "T", "--cmd", "C", "--kernel", "attn_decode_kernel", "--last", "2"])
    out = capsys.readouterr().out
    assert "| `ns::attn_decode_kernel<bf16, 64, 7, 4>` | 3 | 10.00 | 0.030 |" in out
    assert "other" not in out                       # only the library's kernels are tabled
    assert "mean 9.000 us" in out                   # (10 + 8) / 2 over the last two dispatches


def test_traffic_calibration(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    calib = 256 << 20
    # the copy's counters read half (fetch) and all (write) of its bytes, in KiB
    f_rows = [[1, "copy_kernel", "FETCH_SIZE", calib / 2 / 1024],
              [2, "ns::attn_decode_kernel<x>", "FETCH_SIZE", 100.0],
              [3, "ns::attn_decode_kernel<x>", "FETCH_SIZE", 60.0],
              [3, "ns::attn_decode_kernel<x>", "FETCH_SIZE", 40.0]]   # two rows of one dispatch add up
    w_rows = [[1, "copy_kernel", "WRITE_SIZE", calib / 1024],
              [2, "ns::attn_decode_kernel<x>", "WRITE_SIZE", 8.0],
              [3, "ns::attn_decode_kernel<x>", "WRITE_SIZE", 8.0]]
    _write(fetch, hdr, f_rows)
    _write(write, hdr, w_rows)
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    out = tmp_path / "traffic.txt"
    ps.main(["traffic", "--fetch", str(fetch), "--write", str(write), "--kernel", "attn_decode_kernel", "--last", "2",
             "--source", str(src), "--calib-bytes", str(calib), "--algorithmic-bytes", "409600", "--out", str(out),
             "--cmd", "c1"])
    vals = dict(line.split(": ", 1) for line in out.read_text().splitlines() if ": " in line and not line.startswith("#"))
    assert float(vals["fetch_scale"]) == 2.0 and float(vals["write_scale"]) == 1.0
    assert int(vals["fetch_bytes_per_launch"]) == 100 * 1024 * 2      # mean of 100 and 60 + 40, scaled
    assert int(vals["write_bytes_per_launch"]) == 8 * 1024
    assert int(vals["traffic_bytes_per_launch"]) == 100 * 1024 * 2 + 8 * 1024
    assert vals["source_sha256"] == hashlib.sha256(b"kernel source\n").hexdigest()
    assert abs(float(vals["traffic_over_algorithmic"]) - (100 * 1024 * 2 + 8 * 1024) / 409600) < 1e-3


def test_trace_splits_last_dispatches_by_grid(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    rows = [["void ns::gemm_big_kernel<0>(int)", 0, 4000, 512],
            ["void ns::gemm_big_kernel<0>(int)", 5000, 7000, 256],
            ["void ns::gemm_big_kernel<0>(int)", 8000, 10000, 256],
            ["void ns::gemm_big_kernel<0>(int)", 11000, 17000, 512]]
    _write(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"], rows)
    ps.main(["trace", str(p), "--title", "T", "--cmd", "C", "--kernel", "gemm_big_kernel<0>", "--last", "3"])
    out = capsys.readouterr().out
    assert "- grid 256: 2 dispatches, mean 2.000 us" in out
    assert "- grid 512: 1 dispatches, mean 6.000 us" in out


def test_counters_clock_mfma_rate_and_busy(tmp_path):
    p = tmp_path / "c.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # GRBM_GUI_ACTIVE summed over 8 XCDs: 8 x 2000 cycles in 2 us -> 1000 MHz;
    # SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs: half of the 2000 cycles busy
    rows = []
    for d, (t0, t1) in enumerate([(0, 2000), (5000, 7000)], 1):
        rows += [[d, "ns::gemm_big_kernel<2>", "GRBM_GUI_ACTIVE", 16000.0, t0, t1],
                 [d, "ns::gemm_big_kernel<2>", "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000.0, t0, t1],
                 [d, "ns::gemm_big_kernel<2>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.048e6, t0, t1]]
    _write(p, hdr, rows)
    out = tmp_path / "o.txt"
    ps.main(["counters", str(p), "--kernel", "gemm_big_kernel<2>", "--last", "2", "--out", str(out)])
    vals = {k.split(" (")[0]: v for k, v in
            (line.split(": ", 1) for line in out.read_text().splitlines() if ": " in line and not line.startswith("#"))}
    assert float(vals["duration_us"]) == 2.0
    assert float(vals["clock_mhz"]) == 1000.0
    # 2.048e6 x 512 FLOP in 2 us = 524.3 TFLOP/s; the peak at 1 GHz is 1024 x 1024 x 1e9 = 1048.6 TFLOP/s
    assert abs(float(vals["mfma_bf16_tflops_issued"]) - 524.3) < 0.1
    assert float(vals["issued_over_peak_at_this_clock"]) == 0.5
    assert float(vals["mfma_busy_fraction"]) == 0.5


def test_counters_wave_time_shares_and_bank_conflicts(tmp_path):
    p = tmp_path / "c.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for d in (1, 2):
        rows += [[d, "ns::gemm_big_kernel<2>", "SQ_WAVE_CYCLES", 1000.0, 0, 10],
                 [d, "ns::gemm_big_kernel<2>", "SQ_WAIT_INST_ANY", 550.0, 0, 10],
                 [d, "ns::gemm_big_kernel<2>", "SQ_WAIT_ANY", 65.0, 0, 10],
                 [d, "ns::gemm_big_kernel<2>", "SQ_LDS_IDX_ACTIVE", 300.0, 0, 10],
                 [d, "ns::gemm_big_kernel<2>", "SQ_LDS_BANK_CONFLICT", 100.0, 0, 10]]
    _write(p, hdr, rows)
    out = tmp_path / "o.txt"
    ps.main(["counters", str(p), "--kernel", "gemm_big_kernel<2>", "--last", "2", "--out", str(out)])
    text = out.read_text()
    assert "waiting to issue an instruction (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES): 0.550" in text
    assert "waiting on a counter or barrier (SQ_WAIT_ANY / SQ_WAVE_CYCLES): 0.065" in text
    assert "SQ_WAIT_INST_LDS" not in text
    # 100 conflict cycles over 200 conflict-free active cycles
    assert "SQ_LDS_BANK_CONFLICT)): 0.500" in text
