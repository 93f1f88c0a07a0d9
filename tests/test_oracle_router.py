"""Pins of the oracle's router (two linear layers around an exact-erf GELU) and threshold.

Pinned against: scipy's normal CDF (GELU(z) = z * Phi(z), an independent library
routine); closed forms with one-hot inputs; the odd-part identity of GELU; the
strict threshold and its polarity; and the router parameter counts printed in
the paper's router table (golden fixture).
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import gelu, route
from synth import f32_to_bf16_bits, make_router_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_gelu_matches_normal_cdf():
    z = np.linspace(-12, 12, 2001)
    # the erf form cancels in the far negative tail (1 + erf(-x) underflows), so the
    # agreement is absolute there: |error| stays at float64 rounding of |z|
    np.testing.assert_allclose(gelu(z), z * norm.cdf(z), rtol=1e-13, atol=1e-15)
    assert gelu(np.array([0.0]))[0] == 0.0
    assert abs(gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15   # Phi(1)


def test_gelu_odd_part_identity():
    z = np.random.default_rng(0).normal(size=1000) * 4
    np.testing.assert_allclose(gelu(z) - gelu(-z), z, rtol=0, atol=1e-12)


def test_route_one_hot_closed_form():
    rng = np.random.default_rng(1)
    d, m, B = 7, 5, 3
    W1 = rng.normal(size=(m, d)).astype(np.float32)
    b1 = rng.normal(size=m).astype(np.float32)
    W2 = rng.normal(size=m).astype(np.float32)
    b2 = np.float32(0.375)
    for i in range(d):
        for j in range(m):
            h = np.zeros((B, d), np.float32)
            h[:, i] = np.float32(2.0)
            w2 = np.zeros(m, np.float32)
            w2[j] = W2[j]
            dal, _ = route(h, W1, b1, w2, b2, 1.0, "f32")
            z = 2.0 * float(W1[j, i]) + float(b1[j])
            expect = float(W2[j]) * z * norm.cdf(z) + 0.375
            np.testing.assert_allclose(dal, expect, rtol=1e-13)


def test_route_is_sum_over_hidden_units():
    # Delta-AL minus b2 is additive over the columns of W2 (second layer is linear)
    rng = np.random.default_rng(2)
    d, m = 9, 6
    h = rng.normal(size=(4, d)).astype(np.float32)
    W1 = rng.normal(size=(m, d)).astype(np.float32)
    W2 = rng.normal(size=m).astype(np.float32)
    full, _ = route(h, W1, None, W2, None, 0.0, "f32")
    parts = 0.0
    for j in range(m):
        w = np.zeros(m, np.float32)
        w[j] = W2[j]
        parts = parts + route(h, W1, None, w, None, 0.0, "f32")[0]
    np.testing.assert_allclose(full, parts, rtol=1e-12, atol=1e-12)


def test_threshold_strict_and_polarity():
    d, m = 4, 2
    h = np.ones((1, d), np.float32)
    W1 = np.zeros((m, d), np.float32)
    W2 = np.ones(m, np.float32)
    tau = 1.0
    # W1 = 0, b1 = 0: GELU(0) = 0, so Delta-AL = b2 exactly
    assert route(h, W1, None, W2, np.float32(tau), tau, "f32")[1][0] == 0          # equal: DFlash
    up = np.nextafter(np.float32(tau), np.float32(2))
    assert route(h, W1, None, W2, up, tau, "f32")[1][0] == 1                         # above: EAGLE-3
    assert route(h, W1, None, W2, np.float32(-5.0), tau, "f32")[1][0] == 0


def test_route_bf16_equals_decoded_f32():
    r = make_router_inputs(9, B=3, d=64, m=16, dtype="bf16")
    dal, ch = route(r.hidden, r.W1, r.b1, r.W2, r.b2, 0.0, "bf16")
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    dal32, ch32 = route(dec(r.hidden), dec(r.W1), r.b1, dec(r.W2), r.b2, 0.0, "f32")
    assert np.array_equal(dal, dal32) and np.array_equal(ch, ch32)


def test_router_parameter_counts_from_paper():
    """Router width m = d/8 with both biases reproduces the printed parameter counts."""
    with open(os.path.join(GOLDEN, "router_params.json")) as f:
        fx = json.load(f)
    for row in fx["rows"]:
        d = row["hidden_size"]
        m = d // 8
        h = np.zeros((1, d), np.float32)
        W1 = np.zeros((m, d), np.float32)
        b1 = np.zeros(m, np.float32)
        W2 = np.zeros(m, np.float32)
        route(h, W1, b1, W2, np.float32(0), 0.0, "f32")  # the oracle accepts these shapes
        count = W1.size + b1.size + W2.size + 1
        assert round(count / 1e6, 2) == row["params_millions"], (d, count)


def test_bf16_rounding_is_nearest_even():
    import torch
    x = np.random.default_rng(4).normal(size=100000).astype(np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e38]   # exact halfway cases + large
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_route_gather_selects_rows_and_flags_invalid():
    from oracle import route_gather
    r = make_router_inputs(11, B=9, d=40, m=12, dtype="f32")
    rows = np.array([3, 0, 8, -1, 9, 3], np.int64)
    dal, ch = route_gather(r.hidden, rows, r.W1, r.b1, r.W2, np.float32(0.1), 0.0, "f32")
    full, fch = route(r.hidden, r.W1, r.b1, r.W2, np.float32(0.1), 0.0, "f32")
    assert dal[0] == full[3] and dal[1] == full[0] and dal[2] == full[8] and dal[5] == full[3]
    assert np.isnan(dal[3]) and np.isnan(dal[4]) and ch[3] == 0 and ch[4] == 0
    assert ch[0] == fch[3]


def test_negated_second_layer_flips_every_choice_off_the_band():
    """Negating W2, b2 and tau negates the gain exactly (IEEE rounding is sign-symmetric)
    and flips the choice of every sequence whose gain differs from tau: the routed
    workload's literal-polarity form rests on this."""
    from synth import negate_second_layer
    for dtype in ("bf16", "f32"):
        r = make_router_inputs(13, B=64, d=96, m=24, dtype=dtype, b2=1.0)
        dal, ch = route(r.hidden, r.W1, r.b1, r.W2, r.b2, r.tau, dtype)
        n = negate_second_layer(r)
        ndal, nch = route(n.hidden, n.W1, n.b1, n.W2, n.b2, n.tau, dtype)
        assert np.array_equal(ndal, -dal)
        off = dal != np.float32(r.tau)
        assert off.all() and np.array_equal(nch[off], 1 - ch[off])
        assert 0 < ch.sum() < 64                   # both choices occur


def test_routed_literal_layout_is_the_flipped_split():
    from synth import make_config
    paper, _ = make_config("routed_bf16", logits=False)
    lit, r = make_config("routed_bf16", logits=False, polarity="literal")
    assert np.array_equal(lit.layout_choice, 1 - paper.layout_choice)
    dal, ch = route(r.hidden, r.W1, r.b1, r.W2, r.b2, r.tau, r.dtype)
    assert np.array_equal(ch, lit.layout_choice)   # the negated router picks the flipped layout
    assert np.min(np.abs(dal - r.tau)) >= 1e-3
    sizes = np.diff(lit.offsets)
    assert np.array_equal(sizes, np.where(lit.layout_choice == 1, 61, 17))
