"""GPU parity of the HIP path against the CPU oracle at sizes the oracle finishes
quickly: several chunks per row, ragged vocabulary tails (row strides padded to
16 bytes), planted ties, signed zeros, infinities, out-of-domain ids, malformed
trees and routed sequences, empty batches.  Integer results are compared bit
for bit; Delta-AL within the stated tolerance."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import DEV, check_router, dev, host, padded_logits
from synth import make_chain_batch, make_router_inputs, make_routed_batch, make_tree_batch

pytestmark = pytest.mark.gpu

VS = [1, 7, 8, 9, 2047, 2048, 2049, 4099, 6149, 20011]


def _stride(V):
    return (V + 7) // 8 * 8 + 8


def _chain_case(B, K, V, dtype, seed, p=0.8):
    cb = make_chain_batch(seed, B, K, V, dtype, p_match=p)
    logits = padded_logits(cb.logits, _stride(V))
    al, bo, rows = wf.verify_chain(logits, dev(cb.draft))
    torch.cuda.synchronize()
    t = oracle.row_argmax(cb.logits, dtype)
    e_al, e_bo = oracle.verify_chain(t.reshape(B, K + 1), cb.draft)
    assert np.array_equal(host(rows), t)
    assert np.array_equal(host(al), e_al) and np.array_equal(host(bo), e_bo)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", VS)
def test_chain_ragged_vocab(dtype, V):
    print(f"chain dtype={dtype} V={V}", flush=True)
    _chain_case(B=3, K=5, V=V, dtype=dtype, seed=V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_many_rows_and_k0(dtype):
    _chain_case(B=40, K=16, V=30000, dtype=dtype, seed=11)
    _chain_case(B=9, K=0, V=5000, dtype=dtype, seed=12)
    _chain_case(B=2, K=1023, V=300, dtype=dtype, seed=13, p=0.995)


def _raw(x: np.ndarray, dtype):
    from synth import f32_to_bf16_bits
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_ties_zeros_infinities(dtype):
    V = 9000
    rows = []
    r = -np.abs(np.random.default_rng(0).standard_normal(V)) - 1
    a = r.copy(); a[[100, 5000, 8999]] = 3.0; rows.append(a)           # tie across chunks
    a = r.copy(); a[[7000, 3000]] = [-0.0, 0.0]; rows.append(a)         # -0 / +0 tie
    a = r.copy(); a[[6999, 7000]] = [0.0, -0.0]; rows.append(a)
    rows.append(np.full(V, -np.inf))                                     # all -inf
    a = np.full(V, -np.inf); a[V - 1] = -np.inf; a[4321] = -1e30; rows.append(a)
    a = r.copy(); a[[17, 18]] = np.inf; rows.append(a)                   # +inf tie
    a = r.copy(); a[V - 1] = 5.0; rows.append(a)                         # last element
    a = r.copy(); a[0] = 5.0; a[1:8] = 5.0; rows.append(a)               # whole first vector
    a = np.zeros(V); rows.append(a)                                      # all equal
    raw = _raw(np.stack(rows), dtype)
    n = len(rows)
    draft = np.zeros((n, 0), np.int32)
    _, bo, rr = wf.verify_chain(padded_logits(raw, _stride(V)), dev(draft))
    t = oracle.row_argmax(raw, dtype)
    assert np.array_equal(host(rr), t)
    assert list(t[:4]) == [100, 3000, 6999, 0]


def _tree_case(B, N, V, Vd, dtype, seed, mutate=None):
    tb = make_tree_batch(seed, B, N, V, Vd, dtype)
    parent, ids, d2t = tb.parent.copy(), tb.draft_ids.copy(), tb.d2t.copy()
    if mutate:
        mutate(parent, ids, d2t)
    al, bo, be, rows = wf.verify_tree(padded_logits(tb.logits, _stride(V)), dev(parent), dev(ids),
                                      dev(d2t))
    torch.cuda.synchronize()
    t = oracle.row_argmax(tb.logits, dtype)
    e = oracle.verify_tree(t.reshape(B, N), parent, ids, d2t, V)
    assert np.array_equal(host(rows), t)
    assert np.array_equal(host(al), e[0]) and np.array_equal(host(bo), e[1])
    assert np.array_equal(host(be), e[2])
    return host(al)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_random(dtype):
    al = _tree_case(B=12, N=61, V=6149, Vd=1500, dtype=dtype, seed=21)
    assert al.max() > 1


def test_tree_sizes():
    for N in (1, 2, 5, 64, 65, 200, 1024):
        _tree_case(B=3, N=N, V=2049, Vd=900, dtype="bf16", seed=N)


def test_tree_malformed_inputs():
    def mutate(parent, ids, d2t):
        parent[0, 5] = 7          # parent after the node
        parent[1, 3] = -4         # negative parent
        parent[2, 9] = 9          # self loop
        ids[3, 1:6] = -1          # ids outside the draft vocabulary
        ids[4, 1:6] = 10 ** 6
        d2t[:50] = -7             # table entries outside the target vocabulary
        d2t[50:100] = 10 ** 7
    _tree_case(B=6, N=61, V=4099, Vd=600, dtype="bf16", seed=31, mutate=mutate)


def _routed_case(layout, V, dtype, seed, mutate=None):
    rb = make_routed_batch(seed, np.asarray(layout, np.int32), K=16, N=61, V=V, Vd=700, dtype=dtype)
    offsets, choice = rb.offsets.copy(), rb.layout_choice.copy()
    if mutate:
        mutate(offsets, choice)
    total = rb.rows
    al, bo, be, rows = wf.verify_routed(padded_logits(rb.logits, _stride(V)), dev(offsets), total,
                                        dev(choice), dev(rb.chain_draft), dev(rb.parent),
                                        dev(rb.draft_ids), dev(rb.d2t))
    torch.cuda.synchronize()
    t = oracle.row_argmax(rb.logits, dtype)
    e = oracle.verify_routed(t, offsets, choice, 16, rb.chain_draft, 61, rb.parent, rb.draft_ids,
                             rb.d2t, V)
    assert np.array_equal(host(al), e[0]) and np.array_equal(host(bo), e[1])
    assert np.array_equal(host(be), e[2])
    covered = np.zeros(total, bool)
    for b in range(len(choice)):
        lo, hi = offsets[b], offsets[b + 1]
        if 0 <= lo <= hi <= total:
            covered[lo:hi] = True
    assert np.array_equal(host(rows)[covered], t[covered])
    return host(al)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_routed_mixed(dtype):
    layout = [0, 1, 1, 0, 0, 1, 0, 1, 1, 1, 0, 0]
    al = _routed_case(layout, 3001, dtype, seed=41)
    assert al.min() >= 1


def test_routed_malformed():
    def mutate(offsets, choice):
        choice[1] = 1 - choice[1]   # row count no longer matches the choice
        choice[2] = 5               # not a drafter
        offsets[6] = offsets[5] - 1  # decreasing offsets
    layout = [0, 1, 0, 1, 0, 1, 0, 1]
    al = _routed_case(layout, 2500, "bf16", seed=42, mutate=mutate)
    assert al[1] == 0 and al[2] == 0 and al[5] == 0 and al[6] == 0
    assert al[0] >= 1 and al[7] >= 1


def test_empty_batches_are_noops():
    x = torch.zeros((0, 100), dtype=torch.bfloat16, device=DEV)
    wf.verify_chain(x.view(0, 100), torch.zeros((0, 4), dtype=torch.int32, device=DEV))
    h = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    wf.route(h, torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV), None,
             torch.zeros(8, dtype=torch.bfloat16, device=DEV), None, 1.0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,B,d,m", [
    ("f32", 1, 2560, 1024), ("f32", 5, 100, 37), ("bf16", 1, 2560, 320), ("bf16", 7, 96, 50),
    ("bf16", 16, 2560, 1024), ("bf16", 33, 2560, 320), ("bf16", 40, 104, 70), ("f32", 20, 64, 33),
])
def test_router_small(dtype, B, d, m):
    print(f"router dtype={dtype} B={B} d={d} m={m}", flush=True)
    r = make_router_inputs(B * 1000 + d, B, d, m, dtype)
    rng = np.random.default_rng(d)
    b1 = (rng.standard_normal(m) * 0.5).astype(np.float32)
    b2 = np.float32(0.25)
    dal, ch = wf.route(dev(r.hidden), dev(r.W1), dev(b1), dev(r.W2), float(b2), 0.1)
    torch.cuda.synchronize()
    e_dal, e_ch = oracle.route(r.hidden, r.W1, b1, r.W2, b2, 0.1, dtype)
    check_router(host(dal), host(ch), e_dal, e_ch, dtype, 0.1)


# bf16 routers on MFMA tiles whose slicing of the hidden size gives chunk counts per slice
# of 16, 32, 6 and 7 (the last two with a shorter last slice: 2 of 6 and 6 of 7 chunks),
# and 9 (a count the kernel reads at run time).  The routers too large to share the
# sweep's launch with 8 or more chunks per slice run on two wave groups: 16 and 32 chunks
# above, and 8 chunks with a shorter last slice (128 x 3592 -> 1024: slices of 1024
# columns, the fourth holding 520, five chunks, the last of 8 columns) and 10 chunks whose
# last chunk is cut (256 x 2504 -> 1024: the second slice holds 1224 columns).
@pytest.mark.parametrize("B,d,m", [(512, 4096, 512), (512, 4096, 1024), (128, 4096, 640),
                                   (150, 2560, 704), (300, 1152, 1024), (128, 3592, 1024),
                                   (256, 2504, 1024)])
def test_router_mfma_slicings(B, d, m):
    print(f"router MFMA slicing B={B} d={d} m={m}", flush=True)
    r = make_router_inputs(B * 7 + d + m, B, d, m, "bf16")
    b1 = (np.random.default_rng(m).standard_normal(m) * 0.5).astype(np.float32)
    dal, ch = wf.route(dev(r.hidden), dev(r.W1), dev(b1), dev(r.W2), 0.125, 0.1)
    torch.cuda.synchronize()
    e_dal, e_ch = oracle.route(r.hidden, r.W1, b1, r.W2, np.float32(0.125), 0.1, "bf16")
    check_router(host(dal), host(ch), e_dal, e_ch, "bf16", 0.1)


def test_router_deterministic():
    r = make_router_inputs(5, 64, 2560, 1024, "bf16")
    args = (dev(r.hidden), dev(r.W1), None, dev(r.W2), 0.0, 1.0)
    a = host(wf.route(*args)[0])
    b = host(wf.route(*args)[0])
    assert np.array_equal(a, b)


def test_many_rows_small_vocab():
    """Large batches (tens of thousands of rows) with a ragged vocabulary: grid and row
    arithmetic of the full and early-exit paths at sizes far beyond the workloads'."""
    print("many rows", flush=True)
    V = 520                                   # 65 bf16 vectors per row
    cb = make_chain_batch(71, 3000, 16, V, "bf16")
    logits = padded_logits(cb.logits, _stride(V))
    t = oracle.row_argmax(cb.logits, "bf16")
    e_al, e_bo = oracle.verify_chain(t.reshape(3000, 17), cb.draft)
    al, bo, rows = (host(x) for x in wf.verify_chain(logits, dev(cb.draft)))
    assert np.array_equal(rows, t) and np.array_equal(al, e_al) and np.array_equal(bo, e_bo)
    al, bo, _ = (host(x) for x in wf.verify_chain_early_exit(logits, dev(cb.draft)))
    assert np.array_equal(al, e_al) and np.array_equal(bo, e_bo)
    layout = np.arange(1200, dtype=np.int32) % 2
    rb = make_routed_batch(72, layout, K=16, N=61, V=V, Vd=300, dtype="bf16")
    logits = padded_logits(rb.logits, _stride(V))
    t = oracle.row_argmax(rb.logits, "bf16")
    e = oracle.verify_routed(t, rb.offsets, layout, 16, rb.chain_draft, 61, rb.parent,
                             rb.draft_ids, rb.d2t, V)
    args = (logits, dev(rb.offsets), rb.rows, dev(layout), dev(rb.chain_draft), dev(rb.parent),
            dev(rb.draft_ids), dev(rb.d2t))
    for fn in (wf.verify_routed, wf.verify_routed_early_exit):
        al, bo, be, _ = (host(x) for x in fn(*args))
        assert np.array_equal(al, e[0]) and np.array_equal(bo, e[1]) and np.array_equal(be, e[2])
