"""Host-side checks of bench.py (no GPU needed): it refuses more than one GPU before
touching a device, and its sweep size fit recovers a known fixed cost and streaming
rate from durations that follow duration = fixed + bytes / rate exactly, and skips the fit
when a quarter round would not fill the GPU twice over."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

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
