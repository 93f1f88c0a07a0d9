"""GPU parity at vocabularies beyond the Qwen3 and Llama-3.1 ones: 262,144 (2^18) and
1,000,003 (odd, so bf16 and float32 rows both end in a partial 16-byte vector).  The
sweep then splits a row into 21 or 79 chunks and the early-exit schedule into more
chunks than at the workload sizes, and winning indices pass 2^18 and 2^19.

Covers the full and early-exit chain verification, tree verification (full and
early-exit), and planted rows: a tie between indices half a million apart, the
maximum in the ragged tail (index V - 1), a tie at 2^18 and 2^18 + 1, and a row of equal
values.  Integer results are compared with the oracle bit for bit."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import dev, host, padded_logits
from synth import f32_to_bf16_bits, make_chain_batch, make_tree_batch

pytestmark = pytest.mark.gpu

BIG = [262144, 1000003]


def _stride(V):
    return (V + 7) // 8 * 8 + 8


def _chain_expect(raw, dtype, draft):
    B, K = draft.shape
    t = oracle.row_argmax(raw, dtype)
    al, bo = oracle.verify_chain(t.reshape(B, K + 1), draft)
    early_rows = np.where(np.arange(K + 1)[None, :] <= (al - 1)[:, None], t.reshape(B, K + 1), -1)
    return t, al, bo, early_rows.reshape(-1)


def _chain_both(raw, dtype, draft, V):
    """Full and early-exit chain verification of the same logits against the oracle."""
    logits = padded_logits(raw, _stride(V))
    al, bo, rows = wf.verify_chain(logits, dev(draft))
    e_al, e_bo, e_rows = wf.verify_chain_early_exit(logits, dev(draft))
    torch.cuda.synchronize()
    t, x_al, x_bo, x_early = _chain_expect(raw, dtype, draft)
    assert np.array_equal(host(rows), t), "row_argmax"
    assert np.array_equal(host(al), x_al) and np.array_equal(host(bo), x_bo)
    assert np.array_equal(host(e_al), x_al) and np.array_equal(host(e_bo), x_bo), "early exit"
    assert np.array_equal(host(e_rows), x_early), "early-exit row_argmax"
    return t, host(al)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", BIG)
def test_chain_large_vocab(dtype, V):
    print(f"large-vocab chain dtype={dtype} V={V}", flush=True)
    cb = make_chain_batch(V % 97, 3, 4, V, dtype, p_match=0.8)
    chunks, _ = wf.argmax_sweep_plan(cb.rows, V)
    assert chunks >= 21
    _chain_both(cb.logits, dtype, cb.draft, V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_one_row_per_sequence_widest_merge(dtype):
    """K = 0 over 1,000,003 tokens: one row per sequence, so the verify call's sweep cuts
    each row into 256 chunks and the acceptance merges them with 64-lane groups (DPP moves
    within rows of 16 lanes, then shuffles at offsets 16 and 32)."""
    V = 1000003
    print(f"one-row chains, widest merge, dtype={dtype}", flush=True)
    cb = make_chain_batch(17, 3, 0, V, dtype)
    t, al = _chain_both(cb.logits, dtype, cb.draft, V)
    assert np.all(al == 1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_planted_far_ties_and_tail(dtype):
    V = 1000003
    print(f"large-vocab planted rows dtype={dtype}", flush=True)
    g = np.random.default_rng(5)
    base = -np.abs(g.standard_normal((4, V))) - 1.0
    base[0, [500000, 999999]] = 3.0           # tie half a million apart: the lower index wins
    base[1, V - 1] = 2.5                      # the maximum in the ragged tail
    base[2, [262144, 262145]] = 4.0           # tie straddling 2^18
    base[3, :] = -1.5                         # every entry equal: index 0
    raw = base.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(base.astype(np.float32))
    # One chain of K = 3 whose drafts match rows 0 and 1 and miss at row 2.
    draft = np.array([[500000, V - 1, 262145]], np.int32)
    t, al = _chain_both(raw, dtype, draft, V)
    assert t.tolist() == [500000, V - 1, 262144, 0]
    assert al.tolist() == [3]


@pytest.mark.parametrize("early", [False, True])
def test_tree_large_vocab(early):
    V, Vd, B, N = 1000003, 5000, 2, 21
    print(f"large-vocab tree early={early}", flush=True)
    tb = make_tree_batch(17, B, N, V, Vd, "bf16")
    fn = wf.verify_tree_early_exit if early else wf.verify_tree
    al, bo, be, rows = fn(padded_logits(tb.logits, _stride(V)), dev(tb.parent),
                          dev(tb.draft_ids), dev(tb.d2t))
    torch.cuda.synchronize()
    t = oracle.row_argmax(tb.logits, "bf16")
    e_al, e_bo, e_be = oracle.verify_tree(t.reshape(B, N), tb.parent, tb.draft_ids, tb.d2t, V)
    assert np.array_equal(host(al), e_al) and np.array_equal(host(bo), e_bo)
    assert np.array_equal(host(be), e_be)
    if early:
        want = np.full(B * N, -1, np.int64)
        for b in range(B):
            acc, _ = oracle.tree_accepted(t.reshape(B, N)[b], tb.parent[b], tb.draft_ids[b],
                                          tb.d2t, V)
            want[b * N:(b + 1) * N] = np.where(acc, t.reshape(B, N)[b], -1)
        assert np.array_equal(host(rows), want)
    else:
        assert np.array_equal(host(rows), t)
