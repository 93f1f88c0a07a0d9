"""GPU parity of the router and the fused chain round at batch sizes far beyond the
workloads': the largest batch the router accepts (65,535 sequences) on its MFMA path
(bfloat16) and its GEMV path (float32), and whiflash_round_chain over 8,192 sequences.
A narrow router (64 -> 32) and vocabulary (600) keep the oracle quick; the grids
(1,024 MFMA sequence tiles, 8,192 GEMV sequence groups, 65,535 finish workgroups)
are the large ones."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import check_router, dev, host, padded_logits
from synth import make_chain_batch, make_router_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_largest_batch(dtype):
    B, d, m = 65535, 64, 32
    print(f"route B={B} {dtype}", flush=True)
    r = make_router_inputs(91, B, d, m, dtype)
    b1 = (np.random.default_rng(92).standard_normal(m) * 0.5).astype(np.float32)
    dal, ch = wf.route(dev(r.hidden), dev(r.W1), dev(b1), dev(r.W2), 0.25, r.tau)
    torch.cuda.synchronize()
    e_dal, e_ch = oracle.route(r.hidden, r.W1, b1, r.W2, np.float32(0.25), r.tau, dtype)
    check_router(host(dal), host(ch), e_dal, e_ch, dtype, r.tau)


def test_round_chain_many_sequences():
    B, K, V, d, m = 8192, 4, 600, 64, 32
    print(f"round_chain B={B}", flush=True)
    r = make_router_inputs(93, B, d, m, "bf16")
    cb = make_chain_batch(94, B, K, V, "bf16")
    logits = padded_logits(cb.logits, (V + 7) // 8 * 8 + 8)
    out = [host(x) for x in wf.round_chain(dev(r.hidden), dev(r.W1), dev(r.b1), dev(r.W2), 0.0,
                                           r.tau, logits, dev(cb.draft))]
    torch.cuda.synchronize()
    e_dal, e_ch = oracle.route(r.hidden, r.W1, r.b1, r.W2, np.float32(0.0), r.tau, "bf16")
    check_router(out[0], out[1], e_dal, e_ch, "bf16", r.tau)
    t = oracle.row_argmax(cb.logits, "bf16")
    e_al, e_bo = oracle.verify_chain(t.reshape(B, K + 1), cb.draft)
    assert np.array_equal(out[4], t)
    assert np.array_equal(out[2], e_al) and np.array_equal(out[3], e_bo)
