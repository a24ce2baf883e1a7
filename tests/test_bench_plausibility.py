"""bench.py's two-sided plausibility check on a result dict (no GPU): a
bandwidth above the HBM peak or a utilisation above 1 is withheld and named."""
import bench


def _result(gateup_gbps, decode_gbps, util):
    return {
        "value": 1500.0,
        "hbm": {"achieved_gbps": decode_gbps, "frac_of_peak": decode_gbps / bench.HBM_PEAK_GBPS},
        "roofline": {"achieved": gateup_gbps, "peak": bench.HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gateup_gbps / bench.HBM_PEAK_GBPS, "avg_launch_us": 7.8},
        "batched": {"T32": {"grouped": {"us": 100.0, "unique_expert_gbps": 3000.0, "tflops": 24.0}},
                    "T4096_zipf": {"us": 967.0, "mfma_util": util}},
        "cpu_baseline": {"value": 0.37, "cores": 1},
    }


def test_plausible_figures_pass_untouched():
    r = _result(1817.0, 1525.0, 0.128)
    assert bench.plausibility(r) == []
    assert r["implausible"] == []
    assert r["roofline"]["achieved"] == 1817.0 and r["batched"]["T4096_zipf"]["mfma_util"] == 0.128


def test_figures_above_peak_are_withheld():
    r = _result(9100.0, 1525.0, 1.2)
    bad = bench.plausibility(r)
    assert sorted(bad) == sorted(["roofline.achieved", "roofline.frac", "batched.T4096_zipf.mfma_util"])
    assert r["roofline"]["achieved"] is None and r["roofline"]["frac"] is None
    assert r["batched"]["T4096_zipf"]["mfma_util"] is None
    # the other figures, and the peak itself, stay
    assert r["roofline"]["peak"] == bench.HBM_PEAK_GBPS and r["hbm"]["achieved_gbps"] == 1525.0
    assert r["batched"]["T32"]["grouped"]["unique_expert_gbps"] == 3000.0
    assert r["value"] == 1500.0


def test_nan_is_withheld():
    r = _result(1817.0, float("nan"), 0.1)
    assert bench.plausibility(r) == ["hbm.achieved_gbps", "hbm.frac_of_peak"]


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits at once with a message
    (before any GPU or library work)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
