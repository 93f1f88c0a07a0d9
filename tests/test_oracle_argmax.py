"""Pins of the oracle's logits decode and greedy row argmax.

Pinned against: the defining property of "first index of the maximum" checked
exhaustively on tiny rows (including -0/+0 ties and infinities), known IEEE bit
patterns, and torch's own bfloat16 conversion (an independent library routine).
"""

import itertools
import struct

import numpy as np
import pytest
import torch

from oracle import decode_logits, row_argmax

VALUES = [-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, float("-inf"), float("inf")]


def _f32(vals):
    return np.array(vals, dtype=np.float32)


def _bf16_bits(vals):
    # every value above is exactly representable in bfloat16: take the high half of its binary32 word
    return np.array([struct.unpack("<I", struct.pack("<f", v))[0] >> 16 for v in vals], np.uint16)


def _is_first_max(x, i):
    # x[i] is not below any element, and every earlier element is strictly below it
    return all(not (x[j] > x[i]) for j in range(len(x))) and all(x[j] < x[i] for j in range(i))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_exhaustive_tiny_rows(dtype):
    for n in range(1, 5):
        rows = list(itertools.product(VALUES, repeat=n))
        enc = _f32 if dtype == "f32" else _bf16_bits
        raw = np.stack([enc(r) for r in rows])
        got = row_argmax(raw, dtype)
        for r, i in zip(rows, got):
            assert _is_first_max(r, int(i)), (r, int(i))


def test_signed_zero_ties_go_to_lowest_index():
    assert row_argmax(_f32([[-0.0, 0.0, -1.0]]), "f32")[0] == 0
    assert row_argmax(_f32([[-1.0, 0.0, -0.0]]), "f32")[0] == 1
    assert row_argmax(_bf16_bits([-3.0, -0.0, 0.0]).reshape(1, -1), "bf16")[0] == 1


def test_all_minus_inf_row_gives_index_zero():
    assert row_argmax(_f32([[float("-inf")] * 7]), "f32")[0] == 0


def test_nan_is_rejected():
    with pytest.raises(ValueError):
        row_argmax(_f32([[0.0, float("nan")]]), "f32")


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], np.uint16)
    got = decode_logits(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 2.0
    assert got[3] == np.inf and got[4] == -np.inf
    assert got[5] == 2.0 ** -133
    assert got[6] == 0.0 and np.signbit(got[6])
    assert got[7] == 3.140625


def test_bf16_decode_matches_torch_on_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_logits(bits, "bf16")
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_argmax_random_rows_match_independent_scan():
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, size=(50, 37)).astype(np.float32)  # many ties
    got = row_argmax(x, "f32")
    for r in range(x.shape[0]):
        best = 0
        for i in range(1, x.shape[1]):
            if x[r, i] > x[r, best]:
                best = i
        assert got[r] == best
