"""Pins of the oracle's WhiFlash-Entropy policy: closed forms (uniform rows, two-level
rows), scipy's softmax + entropy (independent library routines), the strict threshold and
its polarity, invalid row indices."""

import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy as scipy_entropy

from oracle import entropy, route_entropy
from synth import f32_to_bf16_bits


def test_uniform_row_is_log_v():
    for V in (1, 2, 7, 151936):
        assert abs(entropy(np.full(V, 0.25, np.float32), "f32") - math.log(V)) < 1e-9


def test_two_level_closed_form():
    # one entry at c, V-1 entries at 0:  p1 = e^c / (e^c + V - 1)
    for V, c in ((2, 0.0), (10, 3.0), (1000, -2.5), (151936, 8.0)):
        x = np.zeros(V, np.float32)
        x[V // 2] = c
        z = math.exp(c) + (V - 1)
        p1, p0 = math.exp(c) / z, 1.0 / z
        expect = -(p1 * math.log(p1) + (V - 1) * p0 * math.log(p0))
        assert abs(entropy(x, "f32") - expect) < 1e-9 * max(1.0, expect)


def test_matches_scipy_on_random_rows():
    rng = np.random.default_rng(0)
    for scale in (0.1, 1.0, 5.0, 30.0):
        x = (rng.standard_normal(5000) * scale).astype(np.float32)
        ref = scipy_entropy(softmax(x.astype(np.float64)))
        assert abs(entropy(x, "f32") - ref) < 1e-9 * max(1.0, ref)
        xb = f32_to_bf16_bits(x)
        dec = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert abs(entropy(xb, "bf16") - scipy_entropy(softmax(dec))) < 1e-9 * max(1.0, ref)


def test_peaked_row_is_near_zero_and_shift_invariant():
    x = np.zeros(100, np.float32)
    x[3] = 200.0
    assert entropy(x, "f32") < 1e-80
    y = np.random.default_rng(1).standard_normal(300).astype(np.float32)
    assert abs(entropy(y, "f32") - entropy(y + np.float32(64.0), "f32")) < 1e-5


def test_route_entropy_threshold_and_rows():
    V = 50
    raw = np.zeros((4, V), np.float32)
    raw[1, 0] = 100.0                        # ~0 entropy
    H_uniform = math.log(V)
    rows = np.array([0, 1, 7, -1, 0])
    tau = np.float32(H_uniform)              # equal to the uniform row's entropy (in float32)
    H, ch = route_entropy(raw, "f32", rows, float(tau))
    assert abs(H[0] - H_uniform) < 1e-12 and H[1] < 1e-30
    assert np.isnan(H[2]) and np.isnan(H[3]) and ch[2] == 0 and ch[3] == 0
    # strict ">": H == tau (up to float32 rounding of tau) picks DFlash unless H exceeds tau
    assert ch[0] == (1 if H_uniform > float(tau) else 0)
    H, ch = route_entropy(raw, "f32", rows, 1.0)
    assert list(ch) == [1, 0, 0, 0, 1]       # high entropy -> EAGLE-3 (autoregressive)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        entropy(np.array([0.0, np.inf], np.float32), "f32")
