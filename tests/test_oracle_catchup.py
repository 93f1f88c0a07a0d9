"""Pins of the lazy catch-up bookkeeping: a conservation law over simulated trajectories
(every accepted token is seen by each drafter exactly once, either while it is active,
through a catch-up prefill, or still pending in its backlog), the catch-up length equals
the tokens accepted since that drafter was last active (recomputed from the history),
and invalid drafter ids leave a sequence untouched."""

import numpy as np

from oracle import catchup_update


def test_conservation_and_history():
    rng = np.random.default_rng(0)
    B, R = 16, 60
    backlog = np.zeros((B, 2), np.int64)
    cur = rng.integers(0, 2, B)
    seen_active = np.zeros((B, 2), np.int64)
    caught = np.zeros((B, 2), np.int64)
    total = np.zeros(B, np.int64)
    history = [[] for _ in range(B)]          # (drafter, accepted) per round
    for _ in range(R):
        al = rng.integers(1, 18, B)
        nxt = np.where(rng.random(B) < 0.3, 1 - cur, cur)
        new, sw, cu = catchup_update(cur, al, nxt, backlog)
        for b in range(B):
            seen_active[b, cur[b]] += al[b]
            total[b] += al[b]
            history[b].append((int(cur[b]), int(al[b])))
            caught[b, nxt[b]] += cu[b]
            if sw[b]:
                # tokens accepted since drafter nxt was last active
                since = 0
                for d, a in reversed(history[b]):
                    if d == nxt[b]:
                        break
                    since += a
                assert cu[b] == since
            else:
                assert cu[b] == 0 and nxt[b] == cur[b]
        backlog, cur = new, nxt
        for x in (0, 1):
            assert np.array_equal(seen_active[:, x] + caught[:, x] + backlog[:, x], total)
        assert np.all(backlog[np.arange(B), cur] == 0)   # the active drafter is never behind


def test_invalid_ids_unchanged():
    backlog = np.array([[3, 4], [5, 6], [1, 2]])
    new, sw, cu = catchup_update([0, 7, 1], [5, 5, 0], [2, 1, 0], backlog)
    assert np.array_equal(new[0], [3, 4]) and np.array_equal(new[1], [5, 6])
    assert list(sw) == [0, 0, 1] and list(cu) == [0, 0, 1]
    assert np.array_equal(new[2], [0, 2])     # AL 0 adds nothing, switch still catches up
