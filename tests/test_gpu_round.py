"""GPU parity of the fused rounds (whiflash_round_routed = route + verify_routed, and
whiflash_round_chain = route + verify_chain, in fewer launches) against the oracle's route
followed by its verification, and bit-for-bit agreement with the separate GPU calls: router
stage 1 runs the same arithmetic in both (the GEMV tile, the MFMA tile or its lean form
inside the sweep's launch, over the same slices in the same step order), and the finish is
shared code."""

import functools

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import check_router, dev, host, padded_logits
from synth import make_config, make_routed_batch, make_router_inputs

pytestmark = pytest.mark.gpu


def _run(r, rb, logits, b2):
    args = (dev(r.hidden), dev(r.W1), dev(r.b1), dev(r.W2), b2, r.tau, logits, dev(rb.offsets),
            rb.rows, dev(rb.chain_draft), dev(rb.parent), dev(rb.draft_ids), dev(rb.d2t))
    out = [host(x) for x in wf.round_routed(*args)]
    dal, ch = wf.route(dev(r.hidden), dev(r.W1), dev(r.b1), dev(r.W2), b2, r.tau)
    sep = [host(x) for x in wf.verify_routed(logits, dev(rb.offsets), rb.rows, ch,
                                             dev(rb.chain_draft), dev(rb.parent),
                                             dev(rb.draft_ids), dev(rb.d2t))]
    dal_s, ch_s = host(dal), host(ch)
    assert np.array_equal(out[0], dal_s) and np.array_equal(out[1], ch_s)
    assert all(np.array_equal(a, b) for a, b in zip(out[2:6], sep))
    return out


def _oracle(r, rb, b2, out):
    """The oracle's own route, then its routed verification with its own choices; sequences
    within 1e-3 of the threshold may legitimately route differently and are not compared."""
    e_dal, e_ch = oracle.route(r.hidden, r.W1, r.b1, r.W2, b2, r.tau, r.dtype)
    check_router(out[0], out[1], e_dal, e_ch, r.dtype, r.tau)
    far = np.abs(e_dal - r.tau) >= 1e-3
    t = oracle.row_argmax(rb.logits, rb.dtype)
    e = oracle.verify_routed(t, rb.offsets, e_ch, rb.K, rb.chain_draft, rb.N, rb.parent,
                             rb.draft_ids, rb.d2t, rb.V)
    assert np.array_equal(out[5], t)
    for got, exp in zip(out[2:5], e):
        assert np.array_equal(got[far], exp[far])
    return far


# B <= 8 with a GEMV router and 16-byte aligned operands runs router stage 1 and the sweep
# in one launch; (8, 100, 33) has rows of 100 bf16 values (not 16-byte multiples), which
# keeps them in two launches, as B > 8 and the MFMA router do.
@pytest.mark.parametrize("B,d,m", [(12, 256, 64), (40, 2560, 1024), (16, 104, 70), (70, 512, 50),
                                   (1, 256, 64), (3, 2560, 320), (5, 2560, 1024), (8, 100, 33)])
def test_round_small(B, d, m):
    print(f"round B={B} d={d} m={m}", flush=True)
    r = make_router_inputs(B + 5, B, d, m, "bf16")
    layout = np.random.default_rng(B).integers(0, 2, B).astype(np.int32)
    rb = make_routed_batch(B + 6, layout, K=16, N=61, V=3001, Vd=500, dtype="bf16")
    logits = padded_logits(rb.logits, 3016)
    out = _run(r, rb, logits, 0.0)
    _oracle(r, rb, 0.0, out)
    # sequences whose router choice disagrees with their row count come out malformed
    mism = out[1] != layout
    assert np.all(out[2][mism] == 0) and np.all(out[2][~mism] >= 1)


@pytest.mark.parametrize("polarity", ["paper", "literal"])
def test_round_routed_workload(polarity):
    """The routed workload at full size through the benchmark's entry point.  "literal" poses
    it with gains above the threshold verified as DFlash chains: W2, b2 and tau negated, every
    sequence's layout swapped (synth.negate_second_layer)."""
    print(f"round on routed_bf16, {polarity} polarity", flush=True)
    batch, r = make_config("routed_bf16", polarity=polarity)
    out = _run(r, batch, dev(batch.logits), r.b2)
    _oracle(r, batch, r.b2, out)
    assert np.array_equal(out[1], batch.layout_choice) and out[2].min() >= 1
    if polarity == "literal":
        _, paper = make_config("routed_bf16", logits=False)
        p_dal, p_ch = oracle.route(paper.hidden, paper.W1, paper.b1, paper.W2, paper.b2,
                                   paper.tau, paper.dtype)
        # chains are exactly the sequences whose paper-form gain exceeds the threshold
        assert np.array_equal(out[1] == 0, p_dal > paper.tau)
        assert np.all(np.abs(out[0] + p_dal) <= 1e-4 * np.maximum(1.0, np.abs(p_dal)))


# ------------------------------------------------------------------ chain-only round


def _chain_round(r, cb, logits, b1, b2):
    """whiflash_round_chain against route + verify_chain on the GPU and against the oracle."""
    h, W1, W2 = dev(r.hidden), dev(r.W1), dev(r.W2)
    b1d = dev(b1)
    out = [host(x) for x in wf.round_chain(h, W1, b1d, W2, b2, r.tau, logits, dev(cb.draft))]
    dal, ch = (host(x) for x in wf.route(h, W1, b1d, W2, b2, r.tau))
    al, bo, rows = (host(x) for x in wf.verify_chain(logits, dev(cb.draft)))
    assert np.array_equal(out[0], dal) and np.array_equal(out[1], ch)
    assert np.array_equal(out[2], al) and np.array_equal(out[3], bo)
    assert np.array_equal(out[4], rows)
    e_dal, e_ch = oracle.route(r.hidden, r.W1, b1, r.W2, np.float32(b2), r.tau, r.dtype)
    check_router(out[0], out[1], e_dal, e_ch, r.dtype, r.tau)
    t = oracle.row_argmax(cb.logits, cb.dtype)
    e_al, e_bo = oracle.verify_chain(t.reshape(cb.B, cb.K + 1), cb.draft)
    assert np.array_equal(out[4], t)
    assert np.array_equal(out[2], e_al) and np.array_equal(out[3], e_bo)


@functools.lru_cache(maxsize=1)
def _sweep_config():
    return make_config("sweep_bf16")


def test_round_chain_sweep_workload():
    """The 256-chain throughput-sweep workload at full size (MFMA router)."""
    print("round_chain sweep_bf16", flush=True)
    batch, r = _sweep_config()
    _chain_round(r, batch, dev(batch.logits), r.b1, 0.0)


def test_round_chain_sweep_workload_paper_router_width():
    """The same 256 chains with the paper's router width m = d/8 = 320 (WhiFlash paper,
    Appendix A; 0.82M parameters in its Table 6) on the MFMA path: 10 hidden-unit tiles
    of 32, the hidden size cut into 5 slices."""
    print("round_chain sweep_bf16, router 2560 -> 320", flush=True)
    batch, _ = _sweep_config()
    r = make_router_inputs(4, 256, 2560, 320, "bf16")
    _chain_round(r, batch, dev(batch.logits), r.b1, 0.0)


@pytest.mark.parametrize("dtype,B,K,V", [("f32", 3, 5, 2049), ("bf16", 9, 0, 4099),
                                          ("bf16", 40, 16, 20011)])
def test_round_chain_small(dtype, B, K, V):
    """GEMV and MFMA router paths, K = 0, ragged vocabularies, biases set."""
    from synth import make_chain_batch
    print(f"round_chain dtype={dtype} B={B} K={K} V={V}", flush=True)
    r = make_router_inputs(B * 7 + K, B, 96 if B < 16 else 2560, 50 if B < 16 else 1024, dtype)
    b1 = (np.random.default_rng(B).standard_normal(r.m) * 0.5).astype(np.float32)
    cb = make_chain_batch(B + 100, B, K, V, dtype)
    logits = padded_logits(cb.logits, (V + 7) // 8 * 8 + 8)
    _chain_round(r, cb, logits, b1, 0.25)


@pytest.mark.parametrize("hd,ld,B", [("f32", "f32", 1), ("bf16", "bf16", 1), ("f32", "bf16", 2),
                                     ("bf16", "f32", 4), ("bf16", "bf16", 5), ("f32", "f32", 8),
                                     ("bf16", "bf16", 9)])
def test_round_chain_few_sequences(hd, ld, B):
    """Up to 8 sequences on the GEMV router: router stage 1 and the sweep share one launch
    (B = 9 takes two), for every hidden / logits element-type pair."""
    from synth import make_chain_batch
    print(f"round_chain few sequences hidden={hd} logits={ld} B={B}", flush=True)
    r = make_router_inputs(B + 300, B, 2560, 1024, hd)
    b1 = (np.random.default_rng(B + 1).standard_normal(r.m) * 0.5).astype(np.float32)
    V = 20011
    cb = make_chain_batch(B + 301, B, 16, V, ld)
    _chain_round(r, cb, padded_logits(cb.logits, (V + 7) // 8 * 8 + 8), b1, -0.125)


def test_round_chain_batched_chain_config():
    """The 32-chain configuration at full size: K = 16 over 151,936 bf16 logits and the
    2560 -> 1024 bf16 router."""
    print("round_chain batched_chain_bf16", flush=True)
    batch, r = make_config("batched_chain_bf16")
    _chain_round(r, batch, dev(batch.logits), r.b1, 0.0)


@pytest.mark.parametrize("B", [8, 9, 10, 12, 15, 16, 24, 32, 33])
def test_round_chain_mid_batches(B):
    """8 to 33 sequences on 16-byte aligned operands, around the MFMA router's 9-sequence
    switch (below it the GEMV router's tiles share the sweep's launch; from 9 on the MFMA
    router's tiles do, up to the size where it takes a launch of its own)."""
    from synth import make_chain_batch
    print(f"round_chain batch tiles B={B}", flush=True)
    r = make_router_inputs(B + 500, B, 2560, 1024, "bf16")
    b1 = (np.random.default_rng(B + 2).standard_normal(r.m) * 0.5).astype(np.float32)
    V = 20011
    cb = make_chain_batch(B + 501, B, 16, V, "bf16")
    _chain_round(r, cb, padded_logits(cb.logits, (V + 7) // 8 * 8 + 8), b1, 0.0)


@pytest.mark.parametrize("B,ldt,V", [(20, "f32", 20011), (64, "bf16", 30011), (65, "bf16", 30011),
                                      (11, "bf16", 151936)])
def test_round_chain_shared_launch(B, ldt, V):
    """bf16 routers small enough to run their tiles inside the sweep's launch (10 to 64
    sequences on one tile row; 65 spans two and keeps a launch of its own), with float32
    or bf16 logits, ragged and full-width vocabularies."""
    from synth import make_chain_batch
    print(f"round_chain shared launch B={B} logits={ldt} V={V}", flush=True)
    r = make_router_inputs(B + 700, B, 2560, 1024, "bf16")
    b1 = (np.random.default_rng(B + 3).standard_normal(r.m) * 0.5).astype(np.float32)
    cb = make_chain_batch(B + 701, B, 16, V, ldt)
    _chain_round(r, cb, padded_logits(cb.logits, (V + 7) // 8 * 8 + 8), b1, 0.0)


def test_round_routed_shared_launch():
    """A routed round of 40 sequences (router tiles inside the sweep's launch), mixed chains and
    trees over the full vocabulary."""
    print("round_routed shared launch B=40", flush=True)
    r = make_router_inputs(740, 40, 2560, 1024, "bf16")
    layout = np.random.default_rng(40).integers(0, 2, 40).astype(np.int32)
    rb = make_routed_batch(741, layout, K=16, N=61, V=151936, Vd=32000, dtype="bf16")
    out = _run(r, rb, dev(rb.logits), 0.0)
    _oracle(r, rb, 0.0, out)


def test_round_chain_single_sequence_f32():
    """The single-sequence float32 workload at full size: K = 16 over 151,936 float32 logits
    and the 2560 -> 1024 router on one float32 hidden state."""
    print("round_chain single_chain_f32", flush=True)
    batch, r = make_config("single_chain_f32")
    _chain_round(r, batch, dev(batch.logits), r.b1, 0.0)


def test_round_chain_llama_bench_size():
    """The benchmark's Llama-3.1-8B-shape workload at full size: 256 chains of K = 10 over a
    128,256-token vocabulary, router 4096 -> 512 (MFMA path)."""
    from synth import make_chain_batch
    print("round_chain llama shapes, 256 chains", flush=True)
    r = make_router_inputs(6, 256, 4096, 512, "bf16")
    cb = make_chain_batch(6, 256, 10, 128256, "bf16")
    _chain_round(r, cb, dev(cb.logits), r.b1, 0.0)
