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


def test_pick_clock_rejects_implausible_readings():
    assert bench.pick_clock([1950, 2000, 2010], 1990) == (2000, "gpu_metrics.current_gfxclks")
    mhz, src = bench.pick_clock([260, 244, 245, 244, 244, 244, 242, 244], 2003)
    assert (mhz, src) == (2003, "clock_info.gfx")  # per-XCD metrics far too low: fall back
    mhz, why = bench.pick_clock([244] * 8, None)
    assert mhz is None and "no plausible clock" in why
    assert bench.pick_clock([], 100)[0] is None


def test_clock_fraction_never_above_one():
    r = bench.clock_fraction({"gfx_mhz": 244}, 852.12)  # the reading that once gave 3.33
    assert "frac_at_clock" not in r and "error" in r
    r = bench.clock_fraction({"gfx_mhz": 2000}, 1000.0)
    assert r["peak_at_clock"] == round(bench.PEAK_BF16_TFLOPS * 2000 / 2400, 1)
    assert 0 < r["frac_at_clock"] <= 1
    assert "error" in bench.clock_fraction({"error": "amdsmi unavailable"}, 1000.0)


def test_input_sets_exceed_twice_the_mall():
    from attention_forward_attn_amd.inputs import WORKLOADS

    for w in WORKLOADS.values():
        per = bench.decode_set_bytes(w) if w.kind == "decode" else bench.prefill_set_bytes(w)
        n = bench.n_sets_beyond_mall(per)
        assert 3 <= n <= 32 and (n * per > 2 * bench.MALL_BYTES or n == 32), w.name
        if w.name != "tiny_b1_h1_s256_d64":
            assert n * per > 2 * bench.MALL_BYTES, w.name
    w = WORKLOADS["mha_b1_h16_s8192_d128_causal"]
    assert bench.prefill_set_bytes(w) == 2 * 128 * (16 * 8192 * 3)


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
