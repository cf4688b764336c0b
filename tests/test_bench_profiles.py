"""The bench reads three figures from the committed rocprofv3 summaries
under profiles/ (the headline's per-dispatch durations, its HBM bytes per
launch, the wire kernels' HBM bytes), each only while the kernel sources
still hash to the value the summary records.  These CPU tests check that
the readers find those figures and refuse a summary taken from other
sources."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

METHOD_BYTES = 26_214_400     # the headline's bytes per launch (the method's count)
MOVED_BYTES = 25_165_824      # what the kernel moves


def recorded(path, key):
    for line in open(path):
        if line.startswith(key):
            return line[len(key):].strip().lstrip(":").strip()
    return None


def test_headline_trace_figures():
    h = recorded(bench.TRACE_SUMMARY, "reduce kernel sources hash")
    assert h, "the trace summary records the sources it was taken with"
    p = bench.profiled_headline(h, METHOD_BYTES)
    assert p is not None
    assert p["dispatches"] >= 200
    assert 0 < p["median_us"] and 0 < p["mean_us"]
    assert abs(p["frac_from_mean"] - METHOD_BYTES / (p["mean_us"] * 1e3) / 8000.0) < 1e-3
    assert bench.profiled_headline("0" * 16, METHOD_BYTES) is None


def test_headline_traffic_figure():
    h = recorded(bench.PROFILE_COUNTERS, "source_hash")
    assert h
    t = bench.traffic_from_profile(h)
    assert t is not None and abs(t / MOVED_BYTES - 1) < 0.02, t
    assert bench.traffic_from_profile("0" * 16) is None


def test_wire_traffic_figures_follow_the_sources():
    h = recorded(bench.WIRE_COUNTERS, "kernel sources sha256[:16]")
    assert h
    wt = bench.wire_traffic()
    if h == bench.all_source_hash():
        # pack and decode of both formats, at 16 Mi and 16 Mi + 13
        assert len(wt) >= 8
        assert all(v > 0 for v in wt.values())
    else:
        assert wt == {}
