"""Host-side logic of bench.py that needs no GPU: the clock summary drops the
samples read before the firmware's clock table first refreshed."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _sampler(samples):
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c._thread = None
    c.handle = None
    c.error = None
    c.samples = samples
    return c


def test_clock_summary_drops_samples_before_the_first_refresh():
    s = _sampler([(150.0, 2000.0, 0.00), (150.0, 2000.0, 0.01), (1700.0, 1900.0, 0.02),
                  (1800.0, 2000.0, 0.03), (1600.0, 2000.0, 0.04)]).stop()
    assert s["samples"] == 3
    assert s["gfx_mhz_median"] == 1700.0
    assert s["gfx_mhz_min"] == 1600.0 and s["gfx_mhz_max"] == 1800.0
    assert s["mem_mhz_median"] == 2000.0
    assert abs(s["window_s"] - 0.04) < 1e-9


def test_clock_summary_reports_a_table_that_never_refreshed():
    s = _sampler([(150.0, 2000.0, 0.0), (150.0, 2000.0, 0.01)]).stop()
    assert "gfx_mhz_median" not in s and "note" in s


def test_clock_summary_without_samples_gives_the_reason():
    c = _sampler([])
    c.error = "AmdSmiLibraryException: driver not loaded"
    s = c.stop()
    assert s["samples"] == 0 and "driver" in s["error"]
