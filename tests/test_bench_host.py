"""Host logic of the benchmark that runs without a GPU: the sizing of the
co-run interference profile (how many attention launches keep the second
stream busy as long as the projections keep the first) and its caps, the
dense-batch roofline entries built from the dense leg's results, and the
runner of a leg in a child process."""
import sys

import pytest

import bench


def test_corun_launch_count_matches_the_projection_stream():
    assert bench.corun_launches(1800.0, 370.0, 4) == 19        # 4 x 1800 / 370 = 19.5 -> 19 (round half even)
    assert bench.corun_launches(1800.0, 200.0, 4) == 36
    assert bench.corun_launches(100.0, 5000.0, 4) == 1         # never fewer than one
    for bad in ((0.0, 1.0, 4), (1.0, 0.0, 4), (1.0, 1.0, 0), (-1.0, 1.0, 4)):
        with pytest.raises(ValueError):
            bench.corun_launches(*bad)


def test_corun_caps_cover_shares_of_the_chip():
    caps = bench.CORUN_CAPS
    assert caps[0] == 16 and caps[-1] == 256 and len(caps) == 16
    assert all(b - a == 16 for a, b in zip(caps, caps[1:]))


def test_dense_rooflines_from_the_dense_leg():
    d = {"attention": {"us": 340.0, "gbs": 6300.0, "hbm_frac": 0.7875, "bytes": 2164260864},
         "gemm": {"qkv_proj": {"us": 386.0}, "o_proj": {"us": 263.0}}, "gemm_tflops": 1070.0,
         "gemm_mfma_frac": 0.428, "clock_during_gate_up_gemm": {"mhz_median": 1400.0}}
    r = bench.dense_rooflines(d)
    a, g = r["dense_attention_roofline"], r["dense_gemm_roofline"]
    assert (a["bound"], a["unit"], a["frac"], a["achieved"]) == ("hbm", "GB/s", 0.7875, 6300.0)
    assert (g["bound"], g["unit"], g["frac"], g["peak"]) == ("mfma", "TFLOP/s", 0.428, 2500.0)
    assert g["per_projection_us"] == {"qkv_proj": 386.0, "o_proj": 263.0}
    assert bench.dense_rooflines({"error": "x"}) == {}


def test_child_leg_result_and_failures_are_reported():
    """The isolated leg's runner: the child's last stdout line is the result;
    a crash (a signal), a nonzero exit, silence or a time-out become an error
    entry instead of ending the benchmark (CPU-only child processes)."""
    py = sys.executable
    ok = bench.run_child_leg([py, "-c", "print('log line'); print('{\"a\": 1}')"], "t")
    assert ok == {"a": 1}
    crash = bench.run_child_leg([py, "-c", "import os, signal; os.kill(os.getpid(), signal.SIGSEGV)"], "t")
    assert "status -11" in crash["error"]
    assert "status 3" in bench.run_child_leg([py, "-c", "import sys; sys.exit(3)"], "t")["error"]
    assert "no result" in bench.run_child_leg([py, "-c", "print('not json')"], "t")["error"]
    assert "non-object" in bench.run_child_leg([py, "-c", "print('[1, 2]')"], "t")["error"]
    assert "timed out" in bench.run_child_leg([py, "-c", "import time; time.sleep(5)"], "t", timeout=0.5)["error"]
