"""Host-side behaviour of bench.py that needs no GPU."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _NoLaunch:
    def run(self, i):  # the clock pass must give up before launching anything
        raise AssertionError("launched without a readable clock")


def test_visible_pairs_closed_forms():
    s = 300
    assert bench.visible_pairs(s, s, False, 0) == s * s
    assert bench.visible_pairs(s, s, True, 0) == s * (s + 1) // 2
    assert bench.visible_pairs(s, s, True, 1) == s                      # the diagonal alone
    w = 64                                                              # rows below w see i+1 keys
    assert bench.visible_pairs(s, s, True, w) == w * (w + 1) // 2 + (s - w) * w
    assert bench.visible_pairs(100, 400, True, 0) == sum(300 + i + 1 for i in range(100))


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present: amdsmi may read the clock")
def test_sampled_clock_without_driver_reports_error():
    r = bench.sampled_clock(_NoLaunch(), 0, 0.1)
    assert set(r) == {"error"} and r["error"]
