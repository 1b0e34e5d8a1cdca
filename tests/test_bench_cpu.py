"""Host-side pieces of bench.py: the clock sampler's parsing of the driver's
DPM table (formats seen on MI355X: a sleep line while idle, the running clock
on a level line under load)."""
import importlib.util
import os
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("table,want", [
    ("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 94.0),
    ("S: 94Mhz\n0: 500Mhz\n1: 1865Mhz *\n", 1865.0),
    ("0: 500Mhz\n1: 2400Mhz\n", None),
])
def test_clock_table_parse(tmp_path, table, want):
    b = _bench()
    f = tmp_path / "pp_dpm_sclk"
    f.write_text(table)
    c = b.ClockSampler()
    c.path = str(f)
    assert c._read() == want


def test_clock_sampler_summary(tmp_path):
    b = _bench()
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 94Mhz\n0: 500Mhz\n1: 1900Mhz *\n")
    c = b.ClockSampler(period=0.001)
    c.path = str(f)
    c.start()
    time.sleep(0.05)
    c.stop()
    s = c.summary("test")
    assert s["samples"] >= 1 and s["mean"] == 1900.0 and s["min"] == s["max"] == 1900.0
    c2 = b.ClockSampler()
    c2.path = None
    c2.start()
    c2.stop()
    assert c2.summary("test") is None
