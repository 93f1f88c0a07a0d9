"""Rows holding NaN (a documented precondition violation): the verify calls must not
fault, every row argmax must still be an index in [0, V), accept lengths stay in
[1, K + 1] (tree: [1, depth + 1]), and rows without NaN in the same batch keep their exact
oracle results.  Covers whole-NaN rows and rows with a few NaNs, in both element types, on
the full and early-exit chain paths, the tree path and the sweep alone."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import dev, host, padded_logits
from synth import f32_to_bf16_bits, make_chain_batch, make_tree_batch

pytestmark = pytest.mark.gpu

V = 20011


def _stride(V):
    return (V + 7) // 8 * 8 + 8


def _poison(raw, dtype, rows, seed):
    """NaN in whole rows (the first half of `rows`) or at a few positions (the rest)."""
    raw = raw.copy()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    g = np.random.default_rng(seed)
    for k, r in enumerate(rows):
        if k < len(rows) // 2:
            raw[r, :] = nan
        else:
            raw[r, g.integers(0, raw.shape[1], 5)] = nan
    return raw


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_rows_with_nan(dtype):
    print(f"nan rows chain {dtype}", flush=True)
    B, K = 12, 6
    cb = make_chain_batch(301, B, K, V, dtype)
    bad = [3, 9, 20, 40, 55, 77]                  # rows of sequences 0, 1, 2, 5, 7, 11
    raw = _poison(cb.logits, dtype, bad, 302)
    logits = padded_logits(raw, _stride(V))
    al, bo, rows = (host(x) for x in wf.verify_chain(logits, dev(cb.draft)))
    e_al, e_bo, e_rows = (host(x) for x in wf.verify_chain_early_exit(logits, dev(cb.draft)))
    assert rows.min() >= 0 and rows.max() < V
    assert al.min() >= 1 and al.max() <= K + 1 and bo.min() >= 0 and bo.max() < V
    assert np.all((e_rows == -1) | ((e_rows >= 0) & (e_rows < V)))
    R = K + 1
    clean = [b for b in range(B) if not any(b * R <= r < (b + 1) * R for r in bad)]
    assert clean
    t = oracle.row_argmax(cb.logits, dtype).reshape(B, R)
    x_al, x_bo = oracle.verify_chain(t, cb.draft)
    for b in clean:
        assert np.array_equal(rows.reshape(B, R)[b], t[b])
        assert al[b] == x_al[b] and bo[b] == x_bo[b]
        assert e_al[b] == x_al[b] and e_bo[b] == x_bo[b]
    # the sweep alone over the same rows: every chunk record holds an index of its row
    _, idx = wf.argmax_sweep(logits)
    idx = host(idx)
    assert idx.min() >= 0 and idx.max() < V


def test_tree_rows_with_nan():
    print("nan rows tree", flush=True)
    B, N = 6, 61
    tb = make_tree_batch(303, B, N, V, 900, "bf16")
    bad = [0, 61 + 5, 4 * 61 + 30]               # the root row of sequence 0, rows of 1 and 4
    raw = _poison(tb.logits, "bf16", bad, 304)
    logits = padded_logits(raw, _stride(V))
    for early in (False, True):
        fn = wf.verify_tree_early_exit if early else wf.verify_tree
        al, bo, be, rows = (host(x) for x in fn(logits, dev(tb.parent), dev(tb.draft_ids),
                                                dev(tb.d2t)))
        assert al.min() >= 1 and al.max() <= 9 and bo.min() >= 0 and bo.max() < V
        assert np.all((rows == -1) | ((rows >= 0) & (rows < V)))
        t = oracle.row_argmax(tb.logits, "bf16").reshape(B, N)
        x_al, x_bo, x_be = oracle.verify_tree(t, tb.parent, tb.draft_ids, tb.d2t, V)
        for b in (2, 3, 5):                      # sequences without NaN rows
            assert al[b] == x_al[b] and bo[b] == x_bo[b] and be[b] == x_be[b]
