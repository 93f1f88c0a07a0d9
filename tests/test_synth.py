"""Checks of the seeded generators: determinism, shapes, tree constraints, d2t
injectivity, and the closed-form expected acceptance length of the chain recipe."""

import numpy as np

from oracle import row_argmax, verify_chain, verify_tree
from synth import (CONFIGS, make_chain_batch, make_config, make_d2t, make_router_inputs,
                   make_routed_batch, make_tree_batch, routed_calibration)


def test_chain_batch_deterministic_and_shaped():
    a = make_chain_batch(1, B=3, K=5, V=300, dtype="bf16")
    b = make_chain_batch(1, B=3, K=5, V=300, dtype="bf16")
    assert a.logits.shape == (18, 300) and a.logits.dtype == np.uint16
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.draft, b.draft)
    c = make_chain_batch(2, B=3, K=5, V=300, dtype="bf16")
    assert not np.array_equal(a.logits, c.logits)
    assert a.draft.dtype == np.int32 and np.all((a.draft >= 0) & (a.draft < 300))


def test_d2t_injective_in_range():
    d2t = make_d2t(2)
    assert d2t.shape == (32000,) and len(np.unique(d2t)) == 32000
    assert d2t.min() >= 0 and d2t.max() < 151936


def test_tree_constraints():
    tb = make_tree_batch(2, B=8, N=61, V=5000, Vd=1000, logits=False)
    for b in range(8):
        par = tb.parent[b]
        assert par[0] == -1 and np.all(par[1:] < np.arange(1, 61)) and np.all(par[1:] >= 0)
        assert tb.depth[b].max() <= 8
        counts = np.bincount(par[1:], minlength=61)
        assert counts.max() <= 10
        for u in range(61):
            kids = np.flatnonzero(par == u)
            assert len(set(tb.draft_ids[b, kids])) == len(kids)      # distinct sibling ids


def test_chain_expected_acceptance_length():
    """E[AL] = sum_{i=0..K} p^i when the planted id is the argmax of every row."""
    K, p, B = 16, 0.8, 3000
    cb = make_chain_batch(123, B=B, K=K, V=256, dtype="f32", p_match=p)
    t = row_argmax(cb.logits, "f32").reshape(B, K + 1)
    assert np.mean(t == cb.planted) > 0.99
    al, _ = verify_chain(t, cb.draft)
    expect = sum(p ** i for i in range(K + 1))
    var = sum((2 * i + 1) * p ** i for i in range(K + 1)) - expect ** 2   # E[AL^2] - E[AL]^2
    assert abs(al.mean() - expect) < 4 * np.sqrt(var / B)


def test_tree_expected_acceptance_length():
    """E[AL] = 1 + sum over nodes of prod over edges on the root path of p / |children(parent)|."""
    B, N, p = 400, 61, 0.7
    tb = make_tree_batch(77, B=B, N=N, V=4096, Vd=2048, dtype="f32", p_match=p)
    t = row_argmax(tb.logits, "f32").reshape(B, N)
    al, _, _ = verify_tree(t, tb.parent, tb.draft_ids, tb.d2t, 4096)
    exp = []
    for b in range(B):
        par = tb.parent[b]
        nk = np.bincount(par[1:], minlength=N)
        reach = np.zeros(N)
        reach[0] = 1.0
        for u in range(1, N):
            reach[u] = reach[par[u]] * p / nk[par[u]]
        exp.append(reach.sum())
    exp = np.array(exp)
    assert abs(al.mean() - exp.mean()) < 4 * al.std() / np.sqrt(B)


def test_router_inputs_scale():
    r = make_router_inputs(0, B=4, d=2560, m=1024, dtype="f32")
    assert r.W1.shape == (1024, 2560) and r.W2.shape == (1024,) and r.hidden.shape == (4, 2560)
    assert abs(r.W1.std() * np.sqrt(2560) - 1) < 0.01


def test_routed_layout_from_calibration():
    cal = routed_calibration()
    assert len(cal["choice"]) == CONFIGS["routed_bf16"]["B"] and sum(cal["choice"]) == 64
    rb = make_routed_batch(3, np.array(cal["choice"][:6]), V=1000, logits=True)
    rows = [61 if c else 17 for c in cal["choice"][:6]]
    assert np.array_equal(np.diff(rb.offsets), rows)
    assert rb.logits.shape == (sum(rows), 1000)


def test_make_config_structure_only():
    batch, router = make_config("routed_bf16", logits=False)
    assert batch.rows == 64 * 17 + 64 * 61 and router.B == 128


def test_tree_generator_rejects_more_children_than_draft_ids():
    import pytest
    from synth import make_tree_batch
    with pytest.raises(ValueError):
        make_tree_batch(1, 1, 20, V=7, Vd=7, children_max=10, logits=False)
    with pytest.raises(ValueError):
        make_tree_batch(1, 1, 20, V=7, Vd=7, children_max=7, logits=False)
