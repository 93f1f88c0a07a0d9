"""GPU parity of whiflash_route_gather (router on the hidden state at each sequence's final
accepted position) against the oracle: GEMV and MFMA paths, explicit and implicit row0,
invalid positions, and the routed workload's accepted rows."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import check_router, dev, host
from synth import make_config, make_hidden_rows, make_router_inputs

pytestmark = pytest.mark.gpu


def _check(dal, ch, e_dal, e_ch, dtype, tau):
    dal, ch = host(dal), host(ch)
    nan = np.isnan(e_dal)
    assert np.array_equal(np.isnan(dal), nan) and np.all(ch[nan] == 0)
    check_router(dal[~nan], ch[~nan], e_dal[~nan], e_ch[~nan], dtype, tau)


@pytest.mark.parametrize("dtype,B,d,m", [("f32", 5, 2560, 1024), ("bf16", 3, 96, 50),
                                         ("bf16", 40, 2560, 1024), ("bf16", 128, 256, 64)])
def test_route_gather_small(dtype, B, d, m):
    print(f"route_gather dtype={dtype} B={B} d={d} m={m}", flush=True)
    rps = 7
    total = B * rps
    rows = make_hidden_rows(B + d, total, d, dtype)
    r = make_router_inputs(B * 7 + d, 1, d, m, dtype)
    rng = np.random.default_rng(B)
    pos = rng.integers(0, rps, size=B).astype(np.int32)
    pos[0] = -1
    b1 = (rng.standard_normal(m) * 0.3).astype(np.float32)
    tau = 0.05
    dal, ch = wf.route_gather(dev(rows), dev(pos), dev(r.W1), dev(b1), dev(r.W2), 0.125, tau,
                              rows_per_seq=rps)
    sel = np.where(pos >= 0, np.arange(B) * rps + pos, -1)
    e_dal, e_ch = oracle.route_gather(rows, sel, r.W1, b1, r.W2, np.float32(0.125), tau, dtype)
    _check(dal, ch, e_dal, e_ch, dtype, tau)
    row0 = (np.arange(B) * rps).astype(np.int32)
    row0[-1] = total          # out of range
    dal2, ch2 = wf.route_gather(dev(rows), dev(pos), dev(r.W1), dev(b1), dev(r.W2), 0.125, tau,
                                row0=dev(row0))
    sel2 = np.where((pos >= 0) & (row0 + pos < total), row0 + pos, -1)
    e2 = oracle.route_gather(rows, sel2, r.W1, b1, r.W2, np.float32(0.125), tau, dtype)
    _check(dal2, ch2, e2[0], e2[1], dtype, tau)


def test_route_gather_routed_workload():
    """Verify the routed batch, then route its next round from the accepted rows."""
    print("route_gather on routed_bf16", flush=True)
    batch, r = make_config("routed_bf16")
    logits = dev(batch.logits)
    offs = dev(batch.offsets)
    _, _, be, _ = wf.verify_routed(logits, offs, batch.rows, dev(batch.layout_choice),
                                   dev(batch.chain_draft), dev(batch.parent), dev(batch.draft_ids),
                                   dev(batch.d2t))
    hidden_rows = make_hidden_rows(3, batch.rows)
    dal, ch = wf.route_gather(dev(hidden_rows), be, dev(r.W1), dev(r.b1), dev(r.W2), r.b2, r.tau,
                              row0=offs)
    # the oracle's own accepted rows (the GPU path feeds its own verify output)
    t = oracle.row_argmax(batch.logits, "bf16")
    _, _, e_best = oracle.verify_routed(t, batch.offsets, batch.layout_choice, batch.K,
                                        batch.chain_draft, batch.N, batch.parent, batch.draft_ids,
                                        batch.d2t, batch.V)
    assert np.array_equal(host(be), e_best)
    sel = batch.offsets[:-1] + e_best
    e_dal, e_ch = oracle.route_gather(hidden_rows, sel, r.W1, r.b1, r.W2, r.b2, r.tau, "bf16")
    _check(dal, ch, e_dal, e_ch, "bf16", r.tau)
