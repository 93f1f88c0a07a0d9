"""GPU parity of the lazy catch-up bookkeeping over a multi-round trajectory, against the
oracle round by round (bit exact), including invalid drafter ids and malformed rounds."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [1, 255, 256, 257, 1000])
def test_catchup_trajectory(B):
    rng = np.random.default_rng(B)
    backlog_ref = np.zeros((B, 2), np.int32)
    backlog = dev(backlog_ref.copy())
    cur = rng.integers(0, 2, B).astype(np.int32)
    for r in range(20):
        al = rng.integers(0, 18, B).astype(np.int32)
        nxt = np.where(rng.random(B) < 0.35, 1 - cur, cur).astype(np.int32)
        if r == 5:
            nxt[: min(3, B)] = 9            # not a drafter: sequence untouched
        sw, cu = wf.catchup_update(dev(cur), dev(al), dev(nxt), backlog)
        backlog_ref, e_sw, e_cu = oracle.catchup_update(cur, al, nxt, backlog_ref)
        assert np.array_equal(host(backlog), backlog_ref), r
        assert np.array_equal(host(sw), e_sw) and np.array_equal(host(cu), e_cu)
        cur = np.where((nxt == 0) | (nxt == 1), nxt, cur).astype(np.int32)
