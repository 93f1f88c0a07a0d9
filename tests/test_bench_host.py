"""Host-side checks of bench.py (no GPU needed): it refuses more than one GPU before
touching a device, and its sweep size fit recovers a known fixed cost and streaming
rate from durations that follow duration = fixed + bytes / rate exactly, and skips the fit
when a quarter round would not fill the GPU twice over."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import bench  # noqa: E402
import drafter_routing_verification_amd as wf  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _Work:
    rows, V = 4352, 151936
    wf = wf


def test_sweep_size_fit_recovers_a_line():
    fixed_us, rate_gbps = 7.0, 7400.0
    calls = []

    def timed_loop(fn, n):
        fn(0)                              # records the launch size
        nbytes = calls[-1] * _Work.V * 2
        return (fixed_us + nbytes / rate_gbps / 1e3) * 1e-6

    work = _Work()
    work.sweep = lambda i, rows=None: calls.append(rows)
    fit = bench._sweep_size_fit(work, timed_loop, 10)
    assert fit["rows"] == [1088, 2176, 3264, 4352] and calls == fit["rows"]
    assert abs(fit["fixed_us"] - fixed_us) < 0.01
    assert abs(fit["steady_GBps"] - rate_gbps) < 0.5
    assert abs(fit["steady_frac"] - rate_gbps / bench.HBM_PEAK_GBS) < 1e-4


def test_sweep_size_fit_skipped_for_latency_bound_sizes():
    work = _Work()
    work.rows = 544                        # 32 chains: a quarter round is 136 rows
    work.sweep = lambda i, rows=None: None
    blocks = 136 * wf.argmax_sweep_plan(136, work.V)[0]
    assert blocks < 2 * bench.RESIDENT_WORKGROUPS
    fit = bench._sweep_size_fit(work, lambda fn, n: 1e-5, 10)
    assert f"{blocks} workgroups" in fit["skipped"] and "rows" not in fit


# ------------------------------------------------------------------ the bench's parity check


def _ref():
    return {"dal": np.array([0.5, 1.0005, 1.7, 2.0]), "choice": np.array([0, 1, 1, 1]),
            "al": np.array([3, 1, 5, 2]), "bonus": np.array([7, 8, 9, 10]),
            "best": np.array([2, 0, 4, 1]), "rows": np.arange(12)}


def _gpu():
    g = {k: np.array(v, copy=True) for k, v in _ref().items()}
    g["dal"] = g["dal"] * (1 + 1e-6)
    return g


def test_parity_accepts_matching_results():
    d = bench._parity(_gpu(), _ref(), 1.0, 2e-2)
    assert d["status"] == "ok" and d["rows_compared"] == 12
    assert d["sequences_within_1e-3_of_threshold"] == 1 and d["dal_max_rel_err"] < 2e-6


def test_parity_fails_on_any_planted_mismatch():
    for key, idx, val in [("al", 2, 4), ("bonus", 0, 1), ("best", 3, 0), ("rows", 11, 3),
                          ("choice", 0, 1), ("dal", 2, 1.0)]:
        g = _gpu()
        g[key][idx] = val
        d = bench._parity(g, _ref(), 1.0, 2e-2)
        assert d["status"].startswith("FAILED"), (key, d)


def test_parity_excludes_the_threshold_band_and_skipped_rows():
    g = _gpu()
    g["choice"][1] = 0                       # 1.0005 lies within 1e-3 of the threshold
    g["routed"] = True                       # a routed round verifies with the GPU's choice,
    g["al"][1] = 0                           # so that sequence's results may differ too
    g["rows"][5:8] = -1                      # rows an early-exit schedule did not read
    d = bench._parity(g, _ref(), 1.0, 2e-2)
    assert d["status"] == "ok" and d["rows_compared"] == 9
    g["al"][0] = 9                           # outside the band it still counts
    assert bench._parity(g, _ref(), 1.0, 2e-2)["status"].startswith("FAILED")


def test_parity_without_router_compares_acceptance_only():
    ref = _ref()
    g = _gpu()
    del g["dal"], g["choice"]
    assert bench._parity(g, ref, None, 2e-2)["status"] == "ok"
