"""The entry points can be captured in a HIP graph: no call allocates, copies, sets memory
or synchronises, and every argument, workspace included, is a pointer the caller owns.

Each case captures two calls of one entry point, each with its own inputs, outputs and
workspace, then replays the graph three times.  Before each replay the graph's outputs are
overwritten and the same calls run eagerly into other outputs, with a synchronisation; after
it, every output of both calls must equal the eager results bit for bit."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
from gpu_helpers import dev, padded_logits
from synth import make_chain_batch, make_routed_batch, make_router_inputs, make_tree_batch

pytestmark = pytest.mark.gpu
DEVICE = "cuda:0"


def _ws(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEVICE)


def _i32(n):
    return torch.empty(max(n, 1), dtype=torch.int32, device=DEVICE)


def _f32(n):
    return torch.empty(max(n, 1), dtype=torch.float32, device=DEVICE)


def _graph_check(calls):
    """calls: (fn, outs) pairs; fn(outs) launches one call writing into the tensors outs."""
    eager_outs = [tuple(torch.empty_like(t) for t in outs) for _, outs in calls]
    for (fn, _), eo in zip(calls, eager_outs):
        fn(eo)
    torch.cuda.synchronize()
    want = [tuple(t.clone() for t in eo) for eo in eager_outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn, outs in calls:
            fn(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn, outs in calls:
            fn(outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for _, outs in calls:
            for t in outs:
                t.fill_(-7)
        for (fn, _), eo in zip(calls, eager_outs):
            fn(eo)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((_, outs), w, eo) in enumerate(zip(calls, want, eager_outs)):
            for k, (a, b, e) in enumerate(zip(outs, w, eo)):
                assert torch.equal(a, b), f"replay {rep}, call {i}, output {k}"
                assert torch.equal(e, b), f"eager call {i}, output {k}, before replay {rep}"


def _router(seed, B, d, m, dtype):
    r = make_router_inputs(seed, B, d, m, dtype)
    b1 = dev((np.random.default_rng(seed).standard_normal(m) * 0.5).astype(np.float32))
    b2 = torch.tensor([0.125], dtype=torch.float32, device=DEVICE)
    return r, (dev(r.hidden), dev(r.W1), b1, dev(r.W2), b2)


# (B, hidden/logits dtype, m): one float32 sequence (router tiles after the sweep's chunks
# in one launch), 20 bf16 sequences (MFMA tiles inside the sweep's launch), 70 bf16
# sequences (MFMA router in a launch of its own).
@pytest.mark.parametrize("B,dt,m", [(1, "f32", 1024), (20, "bf16", 1024), (70, "bf16", 1024)])
def test_graph_round_chain(B, dt, m):
    print(f"graph round_chain B={B} {dt}", flush=True)
    K, V, d = 16, 30011, 2560
    calls = []
    for i in range(2):
        r, (h, W1, b1, W2, b2) = _router(900 + 10 * B + i, B, d, m, dt)
        cb = make_chain_batch(901 + 10 * B + i, B, K, V, dt)
        logits = padded_logits(cb.logits, (V + 7) // 8 * 8 + 8)
        draft = dev(cb.draft)
        ws = _ws(wf.round_chain_workspace_bytes(B, m, K, V))

        def fn(o, h=h, W1=W1, b1=b1, W2=W2, b2=b2, tau=r.tau, logits=logits, draft=draft, ws=ws):
            wf.round_chain(h, W1, b1, W2, b2, tau, logits, draft, delta_al=o[0], choice=o[1],
                           accept_len=o[2], bonus=o[3], row_argmax=o[4], workspace=ws)
        calls.append((fn, (_f32(B), _i32(B), _i32(B), _i32(B), _i32(B * (K + 1)))))
    _graph_check(calls)


@pytest.mark.parametrize("B", [6, 40])
def test_graph_round_routed(B):
    print(f"graph round_routed B={B}", flush=True)
    K, N, V, Vd, d, m = 16, 61, 20011, 500, 2560, 1024
    calls = []
    for i in range(2):
        r, (h, W1, b1, W2, b2) = _router(950 + B + i, B, d, m, "bf16")
        layout = np.random.default_rng(B + i).integers(0, 2, B).astype(np.int32)
        rb = make_routed_batch(960 + B + i, layout, K=K, N=N, V=V, Vd=Vd, dtype="bf16")
        logits = padded_logits(rb.logits, (V + 7) // 8 * 8 + 8)
        args = (dev(rb.offsets), rb.rows, dev(rb.chain_draft), dev(rb.parent),
                dev(rb.draft_ids), dev(rb.d2t))
        ws = _ws(wf.round_workspace_bytes(B, m, rb.rows, V))

        def fn(o, h=h, W1=W1, b1=b1, W2=W2, b2=b2, tau=r.tau, logits=logits, args=args, ws=ws):
            wf.round_routed(h, W1, b1, W2, b2, tau, logits, *args, delta_al=o[0], choice=o[1],
                            accept_len=o[2], bonus=o[3], best_node=o[4], row_argmax=o[5],
                            workspace=ws)
        calls.append((fn, (_f32(B), _i32(B), _i32(B), _i32(B), _i32(B), _i32(rb.rows))))
    _graph_check(calls)


def test_graph_verify_tree():
    print("graph verify_tree", flush=True)
    B, N, V, Vd = 4, 61, 20011, 500
    calls = []
    for i in range(2):
        tb = make_tree_batch(980 + i, B, N, V, Vd, "bf16")
        logits = padded_logits(tb.logits, (V + 7) // 8 * 8 + 8)
        args = (dev(tb.parent), dev(tb.draft_ids), dev(tb.d2t))
        ws = _ws(wf.verify_workspace_bytes(B * N, V))

        def fn(o, logits=logits, args=args, ws=ws):
            wf.verify_tree(logits, *args, accept_len=o[0], bonus=o[1], best_node=o[2],
                           row_argmax=o[3], workspace=ws)
        calls.append((fn, (_i32(B), _i32(B), _i32(B), _i32(B * N))))
    _graph_check(calls)


def test_graph_round_chain_early_exit():
    print("graph round_chain_early_exit", flush=True)
    B, K, V, d, m = 16, 16, 30011, 2560, 1024
    calls = []
    for i in range(2):
        r, (h, W1, b1, W2, b2) = _router(990 + i, B, d, m, "bf16")
        cb = make_chain_batch(991 + i, B, K, V, "bf16")
        logits = padded_logits(cb.logits, (V + 7) // 8 * 8 + 8)
        draft = dev(cb.draft)
        ws = _ws(wf.round_chain_early_exit_workspace_bytes(B, m, K, V))

        def fn(o, h=h, W1=W1, b1=b1, W2=W2, b2=b2, tau=r.tau, logits=logits, draft=draft, ws=ws):
            wf.round_chain_early_exit(h, W1, b1, W2, b2, tau, logits, draft, delta_al=o[0],
                                      choice=o[1], accept_len=o[2], bonus=o[3],
                                      row_argmax=o[4], workspace=ws)
        calls.append((fn, (_f32(B), _i32(B), _i32(B), _i32(B), _i32(B * (K + 1)))))
    _graph_check(calls)


def test_graph_round_routed_early_exit():
    print("graph round_routed_early_exit", flush=True)
    B, K, N, V, Vd, d, m = 12, 16, 61, 20011, 500, 2560, 1024
    calls = []
    for i in range(2):
        r, (h, W1, b1, W2, b2) = _router(1000 + i, B, d, m, "bf16")
        layout = np.random.default_rng(1001 + i).integers(0, 2, B).astype(np.int32)
        rb = make_routed_batch(1002 + i, layout, K=K, N=N, V=V, Vd=Vd, dtype="bf16")
        logits = padded_logits(rb.logits, (V + 7) // 8 * 8 + 8)
        args = (dev(rb.offsets), rb.rows, dev(rb.chain_draft), dev(rb.parent),
                dev(rb.draft_ids), dev(rb.d2t))
        ws = _ws(wf.round_early_exit_workspace_bytes(B, m, K, N, rb.rows, V))

        def fn(o, h=h, W1=W1, b1=b1, W2=W2, b2=b2, tau=r.tau, logits=logits, args=args, ws=ws):
            wf.round_routed_early_exit(h, W1, b1, W2, b2, tau, logits, *args, delta_al=o[0],
                                       choice=o[1], accept_len=o[2], bonus=o[3],
                                       best_node=o[4], row_argmax=o[5], workspace=ws)
        calls.append((fn, (_f32(B), _i32(B), _i32(B), _i32(B), _i32(B), _i32(rb.rows))))
    _graph_check(calls)


def test_graph_verify_routed_entropy():
    print("graph verify_routed_entropy", flush=True)
    B, K, N, V, Vd = 8, 16, 61, 20011, 500
    calls = []
    for i in range(2):
        layout = np.random.default_rng(1010 + i).integers(0, 2, B).astype(np.int32)
        rb = make_routed_batch(1012 + i, layout, K=K, N=N, V=V, Vd=Vd, dtype="bf16")
        logits = padded_logits(rb.logits, (V + 7) // 8 * 8 + 8)
        args = (dev(rb.offsets), rb.rows, dev(layout), dev(rb.chain_draft), dev(rb.parent),
                dev(rb.draft_ids), dev(rb.d2t))
        ws = _ws(wf.verify_routed_entropy_workspace_bytes(B, rb.rows, V))

        def fn(o, logits=logits, args=args, ws=ws):
            wf.verify_routed_entropy(logits, *args, 2.0, accept_len=o[0], bonus=o[1],
                                     best_node=o[2], row_argmax=o[3], entropy=o[4],
                                     next_choice=o[5], workspace=ws)
        calls.append((fn, (_i32(B), _i32(B), _i32(B), _i32(rb.rows), _f32(B), _i32(B))))
    _graph_check(calls)
