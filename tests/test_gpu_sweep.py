"""GPU parity of the argmax sweep kernel on its own (whiflash_argmax_sweep): every
chunk's (max, lowest index of the max) against the oracle's greedy argmax applied to
that chunk's entries, bit for bit; and the merge of a row's chunks against the oracle's
argmax of the whole row.  Covers ragged vocabularies (V not a multiple of the vector
width or of the chunk), float32 and bfloat16, padded row strides, maxima tied across
chunk boundaries, rows of -inf, and the 256-chain throughput-sweep workload at full
size (every row merged, sampled rows chunk by chunk)."""

import numpy as np
import pytest
import torch

import drafter_routing_verification_amd as wf
import oracle
from gpu_helpers import dev, host, padded_logits
from synth import make_chain_batch, make_config

pytestmark = pytest.mark.gpu


def _decode(raw_row, dtype):
    return oracle.decode_logits(raw_row, dtype)


def _check_chunks(raw, dtype, vals, idx, rows=None):
    """Chunk records of the listed rows against the oracle on each chunk's entries."""
    R, V = raw.shape
    chunks, elems = wf.argmax_sweep_plan(R, V)
    assert vals.shape == (R, chunks) and idx.shape == (R, chunks)
    for r in (range(R) if rows is None else rows):
        for c in range(chunks):
            lo, hi = c * elems, min(V, (c + 1) * elems)
            t = int(oracle.row_argmax(raw[r:r + 1, lo:hi], dtype)[0]) + lo
            assert idx[r, c] == t, (r, c, idx[r, c], t)
            want = np.float32(_decode(raw[r, lo:hi], dtype).max())
            assert vals[r, c] == want or (np.isneginf(want) and np.isneginf(vals[r, c])), (r, c)


def _merged(vals, idx):
    """Row argmax from chunk records: the largest value, the lowest index among equals
    (chunks are in increasing index order, so the first chunk holding the max wins)."""
    best = vals.max(axis=1, keepdims=True)
    first = np.argmax(vals == best, axis=1)
    return idx[np.arange(len(idx)), first]


def _run(raw, dtype, stride):
    vals, idx = wf.argmax_sweep(padded_logits(raw, stride))
    torch.cuda.synchronize()
    return host(vals), host(idx)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [7, 2049, 20011, 151936])
def test_sweep_chunks_ragged(dtype, V):
    print(f"sweep chunks dtype={dtype} V={V}", flush=True)
    cb = make_chain_batch(V % 97 + 3, 3, 12, V, dtype)        # 39 rows
    raw = cb.logits
    vals, idx = _run(raw, dtype, (V + 7) // 8 * 8 + 8)
    _check_chunks(raw, dtype, vals, idx)
    assert np.array_equal(_merged(vals, idx), oracle.row_argmax(raw, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sweep_ties_and_neg_inf(dtype):
    """Equal maxima planted in several chunks of a row (each chunk reports its own first
    occurrence; the merge keeps the lowest), and rows that are -inf throughout."""
    print(f"sweep ties dtype={dtype}", flush=True)
    V = 20011
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, V)).astype(np.float32)
    chunks, elems = wf.argmax_sweep_plan(8, V)
    for r in range(4):
        for c in range(chunks):
            x[r, min(V - 1, c * elems + (r * 37 + c * 11) % elems)] = 9.0
            x[r, min(V - 1, c * elems + elems - 1)] = 9.0       # last entry of each chunk too
    x[4, :] = -np.inf
    x[5, :] = -np.inf
    x[5, V - 1] = -3.0                                          # only the ragged tail is finite
    x[6, :] = 0.0
    x[6, ::2] = -0.0                                            # -0 and +0 tie
    if dtype == "bf16":
        from synth.workloads import f32_to_bf16_bits
        raw = f32_to_bf16_bits(x)
    else:
        raw = x
    vals, idx = _run(raw, dtype, V + 13)
    _check_chunks(raw, dtype, vals, idx)
    assert np.array_equal(_merged(vals, idx), oracle.row_argmax(raw, dtype))
    assert idx[4, 0] == 0 and np.isneginf(vals[4]).all()


def test_sweep_workload_full_size():
    """The 4,352-row throughput-sweep workload in the launch configuration the benchmark times."""
    print("sweep sweep_bf16 full size", flush=True)
    batch, _ = make_config("sweep_bf16")
    logits = dev(batch.logits)
    vals, idx = (host(t) for t in wf.argmax_sweep(logits))
    assert vals.shape[1] == wf.argmax_sweep_plan(batch.rows, batch.V)[0] == 15
    t = oracle.row_argmax(batch.logits, "bf16")
    assert np.array_equal(_merged(vals, idx), t)
    sample = np.random.default_rng(11).choice(batch.rows, 24, replace=False)
    _check_chunks(batch.logits, "bf16", vals, idx, rows=sample)


@pytest.mark.parametrize("dtype,B", [("bf16", 161), ("bf16", 240), ("f32", 240)])
def test_sweep_large_launch_edges(dtype, B):
    """Launches just past the small-launch limit of 8,192 workgroups, where the first 4,096
    workgroups and the last 512 of each XCD issue their loads in one batch and the rest one
    at a time: 161 chains of 17 rows over 20,011 entries (3 chunks a row, 8,211 workgroups,
    19 streaming ones) and 240 chains (12,240 workgroups, 4,048 streaming), in bfloat16 and
    float32."""
    print(f"sweep large-launch edges dtype={dtype} B={B}", flush=True)
    V = 20011
    cb = make_chain_batch(40 + B, B, 16, V, dtype)
    raw = cb.logits
    chunks, _ = wf.argmax_sweep_plan(raw.shape[0], V)
    assert raw.shape[0] * chunks > 8192
    vals, idx = _run(raw, dtype, V + 5)
    assert np.array_equal(_merged(vals, idx), oracle.row_argmax(raw, dtype))
    sample = np.random.default_rng(B).choice(raw.shape[0], 48, replace=False)
    _check_chunks(raw, dtype, vals, idx, rows=sample)


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 20011), ("bf16", 2049)])
def test_stream_read_sink(dtype, V):
    """The measurement aid reads what the sweep reads: its sink is the XOR of the 32-bit words of
    row 0's first chunk (whole 16-byte vectors only)."""
    print(f"stream read dtype={dtype} V={V}", flush=True)
    cb = make_chain_batch(7, 4, 8, V, dtype)
    raw = cb.logits
    sink = host(wf.stream_read(padded_logits(raw, (V + 7) // 8 * 8 + 8)))
    torch.cuda.synchronize()
    _, elems = wf.argmax_sweep_plan(raw.shape[0], V)
    per = 8 if dtype == "bf16" else 4
    n = min(elems, V // per * per)
    words = np.ascontiguousarray(raw[0, :n]).view(np.uint32)
    want = np.bitwise_xor.reduce(words) if len(words) else np.uint32(0)
    assert np.uint32(sink[0]) == np.uint32(want)
