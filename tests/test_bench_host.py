"""Host logic of the benchmark that runs without a GPU: the sizing of the
co-run interference profile (how many attention launches keep the second
stream busy as long as the projections keep the first) and its caps."""
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
