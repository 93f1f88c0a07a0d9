"""GPU parity of the early-exit DFlash chain verification (whiflash_verify_chain_early_exit)
against the oracle: accept_len and bonus bit for bit equal to the oracle's chain
acceptance over the full row argmax; row_argmax equal to the oracle's argmax on rows
0..n of each sequence (n = AL - 1) and -1 after.  Covers ragged vocabularies, planted
ties across chunks, out-of-vocabulary drafts, K = 0, long chains, reuse of one
workspace across calls (the per-sequence flags must be cleared by each call), and the
chain workloads at full size."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import dev, host, padded_logits
from synth import f32_to_bf16_bits, make_chain_batch, make_config

pytestmark = pytest.mark.gpu


def _stride(V):
    return (V + 7) // 8 * 8 + 8


def _expect(raw, dtype, draft):
    B, K = draft.shape
    t = oracle.row_argmax(raw, dtype).reshape(B, K + 1)
    al, bo = oracle.verify_chain(t, draft)
    rows = np.where(np.arange(K + 1)[None, :] <= (al - 1)[:, None], t, -1)
    return al, bo, rows.reshape(-1)


def _run(logits, draft, ws=None):
    al, bo, rows = wf.verify_chain_early_exit(logits, dev(draft), workspace=ws)
    torch.cuda.synchronize()
    return host(al), host(bo), host(rows)


def _check(raw, dtype, draft, got):
    e_al, e_bo, e_rows = _expect(raw, dtype, draft)
    al, bo, rows = got
    assert np.array_equal(al, e_al), "accept_len"
    assert np.array_equal(bo, e_bo), "bonus"
    assert np.array_equal(rows, e_rows), "row_argmax"


def _case(B, K, V, dtype, seed, p=0.8):
    cb = make_chain_batch(seed, B, K, V, dtype, p_match=p)
    got = _run(padded_logits(cb.logits, _stride(V)), cb.draft)
    _check(cb.logits, dtype, cb.draft, got)
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 9, 2049, 12801, 20011, 151936])
def test_early_exit_ragged_vocab(dtype, V):
    print(f"early-exit dtype={dtype} V={V}", flush=True)
    _case(B=5, K=6, V=V, dtype=dtype, seed=V + 3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_exit_k0_long_chain_and_full_accept(dtype):
    print(f"early-exit shapes dtype={dtype}", flush=True)
    _case(B=9, K=0, V=5000, dtype=dtype, seed=21)
    _case(B=2, K=1023, V=300, dtype=dtype, seed=22, p=0.995)
    al, _, _ = _case(B=16, K=16, V=40000, dtype=dtype, seed=23, p=1.0)
    assert (al == 17).all()
    al, _, _ = _case(B=16, K=16, V=40000, dtype=dtype, seed=24, p=0.0)
    assert (al == 1).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_exit_ties_and_out_of_vocab(dtype):
    """Ties between the draft token and other indices in other chunks decide by index."""
    print(f"early-exit ties dtype={dtype}", flush=True)
    V, K = 60000, 4
    rng = np.random.default_rng(5)
    base = -np.abs(rng.standard_normal((6 * (K + 1), V))).astype(np.float32) - 1.0
    draft = np.full((6, K), 7, np.int32)
    x = base.reshape(6, K + 1, V)
    for b in range(6):
        for i in range(K + 1):
            x[b, i, 7 + 1000 * i] = 2.0           # planted greedy token
        draft[b] = 7 + 1000 * np.arange(K)
    x[0, 1, 50000] = 2.0      # tie after the draft token (later chunk): still accepted
    x[1, 1, 3] = 2.0          # tie before the draft token: rejected at position 1
    x[2, 2, 59999] = 2.5      # larger in the last chunk: rejected at 2
    draft[3, 0] = V           # out of vocabulary: rejected at 0
    draft[4, 2] = -1          # negative id: rejected at 2
    x[5, 0, 7] = 0.0          # +0 at the draft token and -0 right after: the row maxima tie,
    x[5, 0, 8] = -0.0         # the lower index (the draft) wins
    raw = x.reshape(-1, V) if dtype == "f32" else f32_to_bf16_bits(x.reshape(-1, V))
    got = _run(padded_logits(raw, _stride(V)), draft)
    _check(raw, dtype, draft, got)
    assert list(got[0]) == [5, 2, 3, 1, 3, 5]
    assert list(got[1]) == [4007, 3, 59999, 7, 2007, 4007]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_exit_workspace_reuse(dtype):
    """One workspace, three calls: all rejected at 0, all accepted, then mixed."""
    print(f"early-exit reuse dtype={dtype}", flush=True)
    B, K, V = 64, 16, 25000
    ws = torch.empty(wf.early_exit_workspace_bytes(B, K, V), dtype=torch.uint8, device="cuda:0")
    for seed, p in ((31, 0.0), (32, 1.0), (33, 0.8)):
        cb = make_chain_batch(seed, B, K, V, dtype, p_match=p)
        got = _run(padded_logits(cb.logits, _stride(V)), cb.draft, ws)
        _check(cb.logits, dtype, cb.draft, got)


def test_early_exit_matches_full_verify_without_row_argmax():
    cb = make_chain_batch(41, 32, 16, 151936, "bf16")
    logits = dev(cb.logits)
    al, bo, none = wf.verify_chain_early_exit(logits, dev(cb.draft), row_argmax=False)
    f_al, f_bo, _ = wf.verify_chain(logits, dev(cb.draft))
    assert none is None
    assert torch.equal(al, f_al) and torch.equal(bo, f_bo)


@pytest.mark.parametrize("name,rnd", [("batched_chain_bf16", 0), ("sweep_bf16", 0), ("sweep_bf16", 57)])
def test_early_exit_workloads(name, rnd):
    """The batched chain workloads at full size, twice (results must not vary)."""
    print(f"early-exit workload {name} round {rnd}", flush=True)
    batch, _ = make_config(name, rnd=rnd)
    logits = dev(batch.logits)
    runs = [_run(logits, batch.draft) for _ in range(2)]
    assert all(np.array_equal(a, b) for a, b in zip(*runs))
    _check(batch.logits, batch.dtype, batch.draft, runs[0])


@pytest.mark.parametrize("name", ["single_chain_f32", "batched_chain_bf16", "sweep_bf16"])
def test_round_chain_early_exit(name):
    """whiflash_round_chain_early_exit against route + verify_chain_early_exit and the oracle;
    twice on one workspace (the flags are cleared by router stage 1 on every call)."""
    from gpu_helpers import check_router
    print(f"round_chain_early_exit {name}", flush=True)
    batch, r = make_config(name)
    logits = dev(batch.logits)
    h, W1, W2, b1 = dev(r.hidden), dev(r.W1), dev(r.W2), dev(r.b1)
    ws = torch.empty(wf.round_chain_early_exit_workspace_bytes(batch.B, r.m, batch.K, batch.V),
                     dtype=torch.uint8, device="cuda:0")
    outs = [[host(x) for x in wf.round_chain_early_exit(h, W1, b1, W2, 0.0, r.tau, logits,
                                                        dev(batch.draft), workspace=ws)]
            for _ in range(2)]
    assert all(np.array_equal(a, b) for a, b in zip(*outs))
    dal, ch, al, bo, rows = outs[0]
    e_dal, e_ch = oracle.route(r.hidden, r.W1, r.b1, r.W2, r.b2, r.tau, r.dtype)
    check_router(dal, ch, e_dal, e_ch, r.dtype, r.tau)
    _check(batch.logits, batch.dtype, batch.draft, (al, bo, rows))
    s_al, s_bo, s_rows = _run(logits, batch.draft)
    assert np.array_equal(al, s_al) and np.array_equal(bo, s_bo) and np.array_equal(rows, s_rows)
