"""Host logic of `bench.py --timeline`: the per-layer spans, gaps and marks
and the per-workgroup statistics (dispatch groups of 256, XCDs) computed from
the profiling build's stamp record, checked on a synthetic record whose
spans, gaps, marks and dispatch-group offsets are known. No GPU: the
library, the graph, the events and the host clock are stand-ins."""
import ctypes
import types

import numpy as np
import pytest

import bench

L = 6
ROUTER_WG, GATEUP_WG, DOWN_WG = 128, 768, 512
# one layer, in ticks of a 100 MHz stamp clock (1 tick = 0.01 us)
R_SPAN, R_NORM = 185, 116
GAP_RG, GAP_GD, GAP_DN = 111, 114, 106
G_START = (7, 15, 22)            # gate/up start of dispatch group 0, 1, 2 (from the launch)
G_ROUTE = (132, 152, 196)        # routing known, from the workgroup's own start
G_ROW0 = (240, 316, 416)         # first row's dots, from the workgroup's own start
G_END = (403, 432, 500)          # last wave's end (from the launch)
D_START = (8, 13)
D_PART = (236, 336)
D_END = (268, 374)
NORM_SPAN = 50


def _write_step(rec, t, ggroups=3):
    """One decode step's stamps from tick t on (gate/up in ggroups dispatch
    groups of 256 workgroups); returns the tick after it."""
    rec[:] = 0
    for l in range(L):
        r = rec[4 * l]
        r[:ROUTER_WG, 0] = t
        r[:ROUTER_WG, 1:5] = t + R_SPAN
        r[:ROUTER_WG, 5] = t + R_NORM
        g0 = t + R_SPAN + GAP_RG - G_START[0]          # the launch; its first workgroup starts G_START[0] later
        g = rec[4 * l + 1]
        for grp in range(ggroups):
            wg = slice(256 * grp, 256 * (grp + 1))
            st = g0 + G_START[grp]
            g[wg, 0] = st
            # four waves end at different times; the workgroup's end is the last
            g[wg, 1:5] = g0 + G_END[grp] - np.array([3, 0, 2, 1], dtype=np.uint64)
            g[wg, 5] = st + G_ROUTE[grp]
            g[wg, 6] = st + G_ROW0[grp]
        gend = g0 + max(G_END[:ggroups])
        d0 = gend + GAP_GD - D_START[0]
        d = rec[4 * l + 2]
        for grp in range(2):
            wg = slice(256 * grp, 256 * (grp + 1))
            st = d0 + D_START[grp]
            d[wg, 0] = st
            d[wg, 1:5] = d0 + D_END[grp]
            d[wg, 6] = st + D_PART[grp]
        t = d0 + max(D_END) + GAP_DN
    n = rec[3]
    n[:8, 0] = t
    n[:8, 1:5] = t + NORM_SPAN
    return t + NORM_SPAN


class _Fn:
    def __init__(self, f):
        self.f = f
        self.restype = None
        self.argtypes = None

    def __call__(self, *a):
        return self.f(*a)


class _Lib:
    """moe_timeline_* stand-ins: read n returns a step starting 1e8 ticks
    (1 s at 100 MHz) after read n-1's."""

    def __init__(self, ggroups=3):
        self.ggroups = ggroups
        self.reads = 0
        self.moe_timeline_reset = _Fn(lambda: 0)
        self.moe_timeline_read = _Fn(self._read)

    def _read(self, ptr):
        rec = np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_uint64)), shape=(256, 1024, 8))
        _write_step(rec, 1_000_000 + 100_000_000 * self.reads, self.ggroups)
        self.reads += 1
        return 0


class _Event:
    def __init__(self, **kw):
        pass

    def record(self, stream):
        pass

    def elapsed_time(self, other):
        return 0.672 * 48


def _run(ggroups=3):
    lib = _Lib(ggroups)
    q = types.SimpleNamespace(load=lambda: lib)
    graph = types.SimpleNamespace(launch=lambda stream: None)
    torch = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=_Event, synchronize=lambda: None))
    clock = iter([0.0, 1.0])                     # the two calibration replays, 1 s apart
    fake_time = types.SimpleNamespace(perf_counter=lambda: next(clock), sleep=lambda s: None)
    saved = bench.time
    bench.time = fake_time
    try:
        return bench.decode_timeline(None, None, graph, None, L, 0.672, q, np, torch, reps=3, batch=48)["timeline"]
    finally:
        bench.time = saved


@pytest.fixture(scope="module")
def tl():
    return _run()


def test_clock_from_the_two_calibration_replays(tl):
    assert tl["clock_mhz_measured"] == pytest.approx(100.0)


def test_per_layer_spans_gaps_and_marks(tl):
    med = tl["per_layer_median_us"]
    us = lambda ticks: ticks / 100.0
    g_span = max(G_END) - G_START[0]
    d_span = max(D_END) - D_START[0]
    assert med["router"] == pytest.approx(us(R_SPAN))
    assert med["gap_router_gateup"] == pytest.approx(us(GAP_RG))
    assert med["gateup"] == pytest.approx(us(g_span))
    assert med["gap_gateup_down"] == pytest.approx(us(GAP_GD))
    assert med["down"] == pytest.approx(us(d_span))
    assert med["gap_down_next"] == pytest.approx(us(GAP_DN))
    period = R_SPAN + GAP_RG + g_span + GAP_GD + d_span + GAP_DN
    assert med["layer_period"] == pytest.approx(us(period))
    assert tl["sum_of_parts_us"] == pytest.approx(us(period))
    assert med["router_norm_mark"] == pytest.approx(us(R_NORM))
    # marks: median over the workgroups, from the kernel's first start
    topk = [G_START[i] + G_ROUTE[i] - G_START[0] for i in range(3)]
    row0 = [G_START[i] + G_ROW0[i] - G_START[0] for i in range(3)]
    assert med["gateup_topk_mark"] == pytest.approx(us(sorted(topk)[1]))
    assert med["gateup_row0_mark"] == pytest.approx(us(sorted(row0)[1]))
    part = [D_START[i] + D_PART[i] - D_START[0] for i in range(2)]
    assert med["down_partials_mark"] == pytest.approx(us((part[0] + part[1]) / 2))
    assert tl["step_us_stamps_median"] == pytest.approx(us(L * period + NORM_SPAN), abs=0.05)


def test_dispatch_groups_and_xcds(tl):
    groups = tl["workgroups_by_dispatch_group_p10_p50_p90_us"]
    assert sorted(groups) == sorted(["gateup_wg0-255", "gateup_wg256-511", "gateup_wg512-767",
                                     "down_wg0-255", "down_wg256-511"])
    for grp in range(3):
        s = groups[f"gateup_wg{256 * grp}-{256 * grp + 255}"]
        assert s["start"] == [pytest.approx((G_START[grp] - G_START[0]) / 100.0)] * 3
        assert s["end"] == [pytest.approx((G_END[grp] - G_START[0]) / 100.0)] * 3
        assert s["routing_known"] == [pytest.approx(G_ROUTE[grp] / 100.0)] * 3
        assert s["row0_dots"] == [pytest.approx(G_ROW0[grp] / 100.0)] * 3
    for grp in range(2):
        s = groups[f"down_wg{256 * grp}-{256 * grp + 255}"]
        assert s["start"] == [pytest.approx((D_START[grp] - D_START[0]) / 100.0)] * 3
        assert s["end"] == [pytest.approx((D_END[grp] - D_START[0]) / 100.0)] * 3
        assert s["row_partials"] == [pytest.approx(D_PART[grp] / 100.0)] * 3
    # every XCD (workgroup id mod 8) holds the same mix of groups
    assert all(v == pytest.approx(0.0) for v in tl["xcd_median_spread_us"].values())


def test_one_gateup_group_of_256_workgroups():
    """One-token gate/up launches of 256 workgroups (one per CU) give one
    dispatch group and the span of that group alone."""
    tl1 = _run(ggroups=1)
    groups = tl1["workgroups_by_dispatch_group_p10_p50_p90_us"]
    assert sorted(k for k in groups if k.startswith("gateup")) == ["gateup_wg0-255"]
    s = groups["gateup_wg0-255"]
    assert s["end"] == [pytest.approx((G_END[0] - G_START[0]) / 100.0)] * 3
    assert s["routing_known"] == [pytest.approx(G_ROUTE[0] / 100.0)] * 3
    assert tl1["per_layer_median_us"]["gateup"] == pytest.approx((G_END[0] - G_START[0]) / 100.0)
