"""GPU parity of the WhiFlash-Entropy policy (whiflash_route_entropy) against the oracle.

Tolerance on H: |gpu - ref| <= 1e-4 * max(1, ref).  The kernel accumulates in float32
(a few dozen terms per thread, then a fixed merge tree over <= 2^18 terms, so the sums
carry ~1e-6 relative error) and evaluates exp2 with the hardware instruction (<= 2 ulp);
the result is ~1e-5 absolute at the entropies here (<= 12 nats), a 10x margin.
Choices must match exactly except within 1e-3 of the threshold."""

import math

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import DEV, dev, host, padded_logits
from synth import f32_to_bf16_bits, make_config

pytestmark = pytest.mark.gpu

ATOL = 1e-4
NEAR = 1e-3


def _check(H_gpu, ch_gpu, H_ref, ch_ref, tau):
    H_gpu = np.asarray(H_gpu, np.float64)
    nan_ref = np.isnan(H_ref)
    assert np.array_equal(np.isnan(H_gpu), nan_ref)
    ok = ~nan_ref
    err = np.abs(H_gpu[ok] - H_ref[ok]) / np.maximum(1.0, np.abs(H_ref[ok]))
    assert err.size == 0 or err.max() <= ATOL, f"entropy err {err.max():.3e}"
    far = nan_ref | (np.abs(H_ref - tau) >= NEAR)
    assert np.array_equal(np.asarray(ch_gpu)[far], ch_ref[far])


def _rows(seed, R, V, dtype):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(np.log(0.05), np.log(20.0), size=R)).astype(np.float32)
    x = rng.standard_normal((R, V), dtype=np.float32) * scale[:, None]
    x[np.arange(R), rng.integers(0, V, R)] += np.float32(8.0)
    x[0] = 0.5                                  # uniform row: H = ln V
    x[1] = 0.0
    x[1, V // 3] = 60.0                         # peaked row: H ~ 0
    return x if dtype == "f32" else f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [7, 2049, 20011, 151936])
def test_entropy_rows(dtype, V):
    print(f"entropy dtype={dtype} V={V}", flush=True)
    R = 24
    raw = _rows(V, R, V, dtype)
    logits = padded_logits(raw, (V + 7) // 8 * 8 + 8)
    rng = np.random.default_rng(V + 1)
    rows_per_seq = 3
    B = R // rows_per_seq
    pos = rng.integers(0, rows_per_seq, size=B).astype(np.int32)
    pos[0], pos[1] = 0, -1                      # sequence 1: invalid position
    tau = 2.5
    H, ch = wf.route_entropy(logits, dev(pos), tau, rows_per_seq=rows_per_seq)
    torch.cuda.synchronize()
    sel = np.where(pos >= 0, np.arange(B) * rows_per_seq + pos, -1)
    H_ref, ch_ref = oracle.route_entropy(raw, dtype, sel, tau)
    _check(host(H), host(ch), H_ref, ch_ref, tau)
    assert abs(host(H)[0] - math.log(V)) < 1e-4 * max(1.0, math.log(V))
    # explicit row0 array, rows out of range
    row0 = np.arange(B, dtype=np.int32) * rows_per_seq
    row0[2] = R + 5
    H2, ch2 = wf.route_entropy(logits, dev(pos), tau, row0=dev(row0))
    sel2 = np.where((pos >= 0) & (row0 + pos < R), row0 + pos, -1)
    H2_ref, ch2_ref = oracle.route_entropy(raw, dtype, sel2, tau)
    _check(host(H2), host(ch2), H2_ref, ch2_ref, tau)
    # bitwise reproducible
    H3, _ = wf.route_entropy(logits, dev(pos), tau, rows_per_seq=rows_per_seq)
    assert np.array_equal(host(H), host(H3), equal_nan=True)


def test_entropy_at_accepted_rows_of_routed_workload():
    """Routed bf16 workload: verify, then the entropy policy at each sequence's accepted row."""
    print("entropy on routed_bf16", flush=True)
    batch, _ = make_config("routed_bf16")
    logits = dev(batch.logits)
    offs, choice = dev(batch.offsets), dev(batch.layout_choice)
    al, bo, be, _ = wf.verify_routed(logits, offs, batch.rows, choice, dev(batch.chain_draft),
                                     dev(batch.parent), dev(batch.draft_ids), dev(batch.d2t))
    torch.cuda.synchronize()
    # the oracle's own accepted rows (the GPU path feeds its own verify output)
    t = oracle.row_argmax(batch.logits, "bf16")
    _, _, e_best = oracle.verify_routed(t, batch.offsets, batch.layout_choice, batch.K,
                                        batch.chain_draft, batch.N, batch.parent, batch.draft_ids,
                                        batch.d2t, batch.V)
    assert np.array_equal(host(be), e_best)
    rows = batch.offsets[:-1] + e_best
    sample = [oracle.entropy(batch.logits[r], "bf16") for r in rows[:8]]
    tau = float(np.median(sample))
    H, ch = wf.route_entropy(logits, be, tau, row0=offs)
    H_ref, ch_ref = oracle.route_entropy(batch.logits, "bf16", rows, tau)
    _check(host(H), host(ch), H_ref, ch_ref, tau)


def _routed_entropy_case(batch, logits_dev, tau_from_median=True, mutate=None):
    offsets, choice = batch.offsets.copy(), batch.layout_choice.copy()
    if mutate:
        mutate(offsets, choice)
    t = oracle.row_argmax(batch.logits, batch.dtype)
    e_al, e_bo, e_be = oracle.verify_routed(t, offsets, choice, batch.K, batch.chain_draft,
                                            batch.N, batch.parent, batch.draft_ids, batch.d2t,
                                            batch.V)
    rows = np.where(e_be >= 0, offsets[:-1] + e_be, -1)
    ok_rows = rows[rows >= 0]
    tau = float(np.median([oracle.entropy(batch.logits[r], batch.dtype) for r in ok_rows[:9]]))
    out = wf.verify_routed_entropy(logits_dev, dev(offsets), batch.rows, dev(choice),
                                   dev(batch.chain_draft), dev(batch.parent), dev(batch.draft_ids),
                                   dev(batch.d2t), tau)
    torch.cuda.synchronize()
    al, bo, be, rr, H, nxt = (host(x) for x in out)
    assert np.array_equal(al, e_al) and np.array_equal(bo, e_bo) and np.array_equal(be, e_be)
    covered = np.zeros(batch.rows, bool)
    for b in range(len(choice)):
        if 0 <= offsets[b] <= offsets[b + 1] <= batch.rows:
            covered[offsets[b]:offsets[b + 1]] = True
    assert np.array_equal(rr[covered], t[covered])
    H_ref, ch_ref = oracle.route_entropy(batch.logits, batch.dtype, rows, tau)
    _check(H, nxt, H_ref, ch_ref, tau)
    return H, nxt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_routed_entropy_small(dtype):
    """Fused verify + entropy policy on a ragged mix with ragged vocabulary, and malformed
    sequences (entropy NaN, next choice 0)."""
    from synth import make_routed_batch
    print(f"verify_routed_entropy dtype={dtype}", flush=True)
    V = 3001
    rb = make_routed_batch(61, np.array([0, 1, 1, 0, 0, 1, 0, 1, 1, 0], np.int32), K=16, N=61,
                           V=V, Vd=700, dtype=dtype)
    logits = padded_logits(rb.logits, (V + 7) // 8 * 8 + 8)

    def mutate(offsets, choice):
        choice[3] = 1          # row count no longer matches the choice
    H, nxt = _routed_entropy_case(rb, logits, mutate=mutate)
    assert np.isnan(H[3]) and nxt[3] == 0 and not np.isnan(H[0])


def test_verify_routed_entropy_workload():
    """The 128-sequence routed workload at full size."""
    print("verify_routed_entropy on routed_bf16", flush=True)
    batch, _ = make_config("routed_bf16")
    _routed_entropy_case(batch, dev(batch.logits))
