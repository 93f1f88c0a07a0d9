"""whiflash_round_chain_noalloc (the round with the library's fixed device scratch) against
whiflash_round_chain (the same round with a caller workspace) and the oracle: two calls in
a row on one GPU, the second smaller and of other element types and on another stream, so
the second reuses the scratch the first left behind."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import check_router, dev, host, padded_logits
from synth import make_chain_batch, make_router_inputs

pytestmark = pytest.mark.gpu


def _case(seed, B, K, V, d, m, hdt, ldt, stream):
    r = make_router_inputs(seed, B, d, m, hdt)
    b1 = (np.random.default_rng(seed).standard_normal(m) * 0.5).astype(np.float32)
    cb = make_chain_batch(seed + 1, B, K, V, ldt)
    logits = padded_logits(cb.logits, (V + 7) // 8 * 8 + 8)
    args = (dev(r.hidden), dev(r.W1), dev(b1), dev(r.W2), 0.125, r.tau, logits, dev(cb.draft))
    need = wf.round_chain_workspace_bytes(B, m, K, V)
    print(f"noalloc B={B} K={K} V={V} d={d} m={m} hidden={hdt} logits={ldt} "
          f"scratch needed {need} bytes", flush=True)
    with torch.cuda.stream(stream):
        got = [host(x) for x in wf.round_chain_noalloc(*args)]
        ref = [host(x) for x in wf.round_chain(*args)]
    torch.cuda.synchronize()
    # Same kernels, same launch plan: every output identical, delta-AL bit for bit too.
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    e_dal, e_ch = oracle.route(r.hidden, r.W1, b1, r.W2, np.float32(0.125), r.tau, hdt)
    check_router(got[0], got[1], e_dal, e_ch, hdt, r.tau)
    t = oracle.row_argmax(cb.logits, ldt)
    e_al, e_bo = oracle.verify_chain(t.reshape(B, K + 1), cb.draft)
    assert np.array_equal(got[4], t)
    assert np.array_equal(got[2], e_al) and np.array_equal(got[3], e_bo)
    return need


def test_noalloc_two_calls_second_smaller():
    # First: 96 bf16 chains, MFMA router, three launches, on the current stream.
    big = _case(31, 96, 16, 50021, 2560, 1024, "bf16", "bf16", torch.cuda.current_stream())
    # Second: 5 chains with float32 logits and router on another stream: the GEMV router
    # sharing the sweep's launch (two launches), over a smaller part of the same scratch.
    small = _case(32, 5, 7, 3001, 256, 64, "f32", "f32", torch.cuda.Stream())
    assert small < big


def test_noalloc_shared_launch_then_larger():
    # 24 bf16 chains: router tiles inside the sweep's launch; then 70 chains with a
    # separate router launch, over more of the scratch than the first call used.
    first = _case(33, 24, 16, 40009, 2560, 1024, "bf16", "bf16", torch.cuda.current_stream())
    second = _case(34, 70, 16, 20011, 2560, 1024, "bf16", "bf16", torch.cuda.current_stream())
    assert first < second

