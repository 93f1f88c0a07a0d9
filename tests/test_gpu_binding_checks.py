"""The Python binding rejects malformed output and workspace tensors before any launch.

The kernels write accept_len, bonus, best_node, row_argmax, delta_al, choice, entropy and
the workspace through raw device pointers, so a host tensor, a wrong element type, a
strided view or a short buffer must raise in Python instead of reaching the GPU.  Each case
below raises before the library is called; a well-formed call afterwards still matches the
oracle."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import DEV, dev, host, padded_logits
from synth import make_chain_batch, make_router_inputs, make_tree_batch

pytestmark = pytest.mark.gpu

B, K, V = 4, 5, 3001


@pytest.fixture(scope="module")
def chain():
    cb = make_chain_batch(71, B, K, V, "bf16")
    return cb, padded_logits(cb.logits, 3008), dev(cb.draft)  # 16-byte aligned row stride


def _i32(n, **kw):
    return torch.empty(n, dtype=torch.int32, device=kw.get("device", DEV))


# Each case builds its bad keyword argument when run (no device tensors at collection).
BAD_CHAIN_OUTPUTS = {
    "host_accept_len": (lambda: dict(accept_len=torch.empty(B, dtype=torch.int32)), TypeError),
    "int64_accept_len": (lambda: dict(accept_len=torch.empty(B, dtype=torch.int64, device=DEV)),
                         TypeError),
    "short_bonus": (lambda: dict(bonus=torch.empty(B - 1, dtype=torch.int32, device=DEV)),
                    ValueError),
    "strided_row_argmax": (lambda: dict(row_argmax=torch.empty(2 * B * (K + 1), dtype=torch.int32,
                                                               device=DEV)[::2]), TypeError),
    "short_row_argmax": (lambda: dict(row_argmax=torch.empty(B * (K + 1) - 1, dtype=torch.int32,
                                                             device=DEV)), ValueError),
    "host_workspace": (lambda: dict(workspace=torch.empty(1 << 20, dtype=torch.uint8)), TypeError),
    "short_workspace": (lambda: dict(workspace=torch.empty(2, dtype=torch.uint8, device=DEV)),
                        ValueError),
}


@pytest.mark.parametrize("case", sorted(BAD_CHAIN_OUTPUTS))
def test_verify_chain_rejects_bad_outputs(chain, case):
    cb, logits, draft = chain
    make, exc = BAD_CHAIN_OUTPUTS[case]
    print(f"verify_chain bad output: {case}", flush=True)
    with pytest.raises(exc):
        wf.verify_chain(logits, draft, **make())


def test_verify_tree_rejects_host_best_node_and_d2t():
    tb = make_tree_batch(72, 2, 13, V, 500, "bf16")
    logits = padded_logits(tb.logits, 3008)
    args = (dev(tb.parent), dev(tb.draft_ids))
    print("verify_tree bad best_node / d2t", flush=True)
    with pytest.raises(TypeError):
        wf.verify_tree(logits, *args, dev(tb.d2t), best_node=torch.empty(2, dtype=torch.int32))
    with pytest.raises(TypeError):
        wf.verify_tree(logits, *args, torch.from_numpy(tb.d2t))


def test_route_rejects_bad_biases_and_outputs():
    r = make_router_inputs(73, B, 96, 40, "f32")
    h, W1, W2 = dev(r.hidden), dev(r.W1), dev(r.W2)
    print("route bad b1 / b2 / delta_al / choice", flush=True)
    with pytest.raises(TypeError):    # b1 on the host
        wf.route(h, W1, torch.from_numpy(r.b1), W2, 0.0, r.tau)
    with pytest.raises(TypeError):    # b2 of the wrong element type
        wf.route(h, W1, dev(r.b1), W2, torch.zeros(1, dtype=torch.float64, device=DEV), r.tau)
    with pytest.raises(TypeError):    # b2 of two elements
        wf.route(h, W1, dev(r.b1), W2, torch.zeros(2, dtype=torch.float32, device=DEV), r.tau)
    with pytest.raises(TypeError):
        wf.route(h, W1, dev(r.b1), W2, 0.0, r.tau,
                 delta_al=torch.empty(B, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        wf.route(h, W1, dev(r.b1), W2, 0.0, r.tau, choice=_i32(B - 1))


def test_round_chain_and_catchup_reject_bad_outputs(chain):
    cb, logits, draft = chain
    r = make_router_inputs(74, B, 96, 40, "bf16")
    h, W1, W2 = dev(r.hidden), dev(r.W1), dev(r.W2)
    print("round_chain / catchup bad outputs", flush=True)
    with pytest.raises(TypeError):
        wf.round_chain(h, W1, None, W2, 0.0, r.tau, logits, draft,
                       delta_al=torch.empty(B, dtype=torch.float32))
    with pytest.raises(ValueError):
        wf.round_chain(h, W1, None, W2, 0.0, r.tau, logits, draft, accept_len=_i32(1))
    z = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        wf.catchup_update(z, z, z, torch.zeros(2 * B, dtype=torch.int32, device=DEV),
                          switch_flag=_i32(B - 1))


def test_good_call_after_rejections_matches_oracle(chain):
    """Supplied outputs of the right form are used as given, and the results are exact."""
    cb, logits, draft = chain
    al, bo, rows = _i32(B), _i32(B), _i32(B * (K + 1))
    ws = torch.empty(wf.verify_workspace_bytes(B * (K + 1), V), dtype=torch.uint8, device=DEV)
    print("verify_chain with supplied outputs", flush=True)
    out = wf.verify_chain(logits, draft, accept_len=al, bonus=bo, row_argmax=rows, workspace=ws)
    assert out[0] is al and out[1] is bo and out[2] is rows
    t = oracle.row_argmax(cb.logits, cb.dtype)
    e_al, e_bo = oracle.verify_chain(t.reshape(B, K + 1), cb.draft)
    assert np.array_equal(host(rows), t)
    assert np.array_equal(host(al), e_al) and np.array_equal(host(bo), e_bo)
