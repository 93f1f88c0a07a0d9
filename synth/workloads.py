"""Seeded generators for the five verify-and-route workloads.

Shapes follow the pages: a 151,936-token target vocabulary, a 2,560-wide final
hidden state and a fixed 32,000-token EAGLE-3 draft vocabulary (WhiFlash
EAGLE-3 drafter card, "Technical Specifications"); a DFlash block of 16 draft
tokens and an EAGLE-3 tree of 60 draft tokens with depth 8 and top-k 10
(WhiFlash paper, Appendix A, Table 7).

Recipe (the same for every workload):
  * logits: float32 draws from N(0, 1), +8.0 added at one planted target id per
    row, then rounded to nearest-even bfloat16 where the workload is bf16;
  * chain drafts: draft[i] equals the planted id of row i with probability p,
    otherwise a uniform id different from it;
  * trees: node 0 is the root; node u >= 1 picks its parent uniformly among the
    earlier nodes whose depth is below the depth limit and that have fewer than
    the child limit; sibling draft ids are distinct; for an internal node, with
    probability p the planted id of its row is the target id of one of its
    children (uniform), else a uniform id that no child carries; a leaf's
    planted id is uniform;
  * d2t: the first Vd entries of a seeded permutation of the target vocabulary
    (absolute, injective target ids);
  * router: hidden ~ N(0, 1), W1 ~ N(0, 1/d), W2 ~ N(0, 1/m), b1 = 0, b2 = 0 or
    the stored calibration of the routed workload.

Every random stream is ``numpy.random.default_rng([seed, stream, round, seq])``
so sequences can be drawn independently and in any order.
No function here computes an argmax, an acceptance length or a router output.
"""

from __future__ import annotations

import json
from dataclasses import dataclass, field
from pathlib import Path

import numpy as np

V_QWEN3 = 151_936
D_QWEN3 = 2_560
VD_EAGLE3 = 32_000
ROUTER_M = 1_024
TAU = 1.0
PLANT_BOOST = 8.0

# Stream ids of the seeded generators.
_S_LOGITS = 1
_S_CHAIN = 2
_S_TREE = 3
_S_D2T = 4
_S_WEIGHTS = 5
_S_HIDDEN = 6

_CALIBRATION = Path(__file__).resolve().parent.parent / "tests" / "golden" / "routed_calibration.json"


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to nearest-even bfloat16; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def _materialise(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _planted_logits(seed: int, rnd: int, seq: int, planted: np.ndarray, V: int, dtype: str) -> np.ndarray:
    """Rows of N(0,1) noise with +8 at the planted id of each row."""
    rows = planted.shape[0]
    x = _rng(seed, _S_LOGITS, rnd, seq).standard_normal((rows, V), dtype=np.float32)
    x[np.arange(rows), planted] += np.float32(PLANT_BOOST)
    return _materialise(x, dtype)


def _other_id(rng: np.random.Generator, V: int, avoid: int) -> int:
    if V == 1:
        return avoid  # a one-token vocabulary has no other id
    o = int(rng.integers(0, V - 1))
    return o + 1 if o >= avoid else o


# --------------------------------------------------------------------------- chain


@dataclass
class ChainBatch:
    B: int
    K: int
    V: int
    dtype: str
    draft: np.ndarray        # int32 [B, K] target ids
    planted: np.ndarray      # int32 [B, K+1]
    logits: np.ndarray | None = None  # [B*(K+1), V] float32 or uint16 (bf16 bits)

    @property
    def rows(self) -> int:
        return self.B * (self.K + 1)


def make_chain_batch(seed: int, B: int, K: int, V: int = V_QWEN3, dtype: str = "bf16",
                     p_match: float = 0.8, rnd: int = 0, logits: bool = True) -> ChainBatch:
    planted = np.empty((B, K + 1), np.int32)
    draft = np.empty((B, K), np.int32)
    for b in range(B):
        g = _rng(seed, _S_CHAIN, rnd, b)
        planted[b] = g.integers(0, V, size=K + 1)
        for i in range(K):
            if g.random() < p_match:
                draft[b, i] = planted[b, i]
            else:
                draft[b, i] = _other_id(g, V, int(planted[b, i]))
    out = ChainBatch(B, K, V, dtype, draft, planted)
    if logits:
        out.logits = np.concatenate(
            [_planted_logits(seed, rnd, b, planted[b], V, dtype) for b in range(B)], axis=0
        ) if B else np.empty((0, V), np.float32 if dtype == "f32" else np.uint16)
    return out


# --------------------------------------------------------------------------- tree


def make_d2t(seed: int, V: int = V_QWEN3, Vd: int = VD_EAGLE3) -> np.ndarray:
    return _rng(seed, _S_D2T).permutation(V)[:Vd].astype(np.int32)


def _random_tree(g: np.random.Generator, N: int, depth_max: int, children_max: int, Vd: int):
    if children_max > Vd:
        # siblings carry distinct draft ids, so a node cannot have more children than ids exist
        raise ValueError(f"children_max={children_max} exceeds the draft vocabulary Vd={Vd}")
    parent = np.full(N, -1, np.int32)
    depth = np.zeros(N, np.int32)
    nchild = np.zeros(N, np.int32)
    draft_ids = np.full(N, -1, np.int32)
    used: dict[int, set] = {}
    for u in range(1, N):
        elig = np.flatnonzero((depth[:u] < depth_max) & (nchild[:u] < children_max))
        p = int(elig[g.integers(len(elig))])
        parent[u] = p
        depth[u] = depth[p] + 1
        nchild[p] += 1
        sib = used.setdefault(p, set())
        while True:
            did = int(g.integers(0, Vd))
            if did not in sib:
                break
        sib.add(did)
        draft_ids[u] = did
    return parent, draft_ids, depth


@dataclass
class TreeBatch:
    B: int
    N: int
    V: int
    Vd: int
    dtype: str
    parent: np.ndarray       # int32 [B, N]; parent[:,0] = -1
    draft_ids: np.ndarray    # int32 [B, N] draft-vocab ids; [:,0] = -1 (root)
    d2t: np.ndarray          # int32 [Vd]
    planted: np.ndarray      # int32 [B, N]
    depth: np.ndarray        # int32 [B, N] (generator bookkeeping)
    logits: np.ndarray | None = None

    @property
    def rows(self) -> int:
        return self.B * self.N


def _tree_sequence(seed: int, rnd: int, b: int, N: int, V: int, d2t: np.ndarray,
                   p_match: float, depth_max: int, children_max: int):
    g = _rng(seed, _S_TREE, rnd, b)
    parent, draft_ids, depth = _random_tree(g, N, depth_max, children_max, d2t.shape[0])
    planted = np.empty(N, np.int32)
    for u in range(N):
        kids = np.flatnonzero(parent == u)
        kid_tok = [int(d2t[draft_ids[v]]) for v in kids]
        if len(kids) and g.random() < p_match:
            planted[u] = kid_tok[int(g.integers(len(kids)))]
        else:
            while True:
                cand = int(g.integers(0, V))
                if cand not in kid_tok:
                    break
            planted[u] = cand
    return parent, draft_ids, depth, planted


def make_tree_batch(seed: int, B: int, N: int = 61, V: int = V_QWEN3, Vd: int = VD_EAGLE3,
                    dtype: str = "bf16", p_match: float = 0.7, depth_max: int = 8,
                    children_max: int = 10, rnd: int = 0, logits: bool = True) -> TreeBatch:
    if children_max >= V:
        # a row whose children's tokens cover the whole vocabulary has no missing token to plant
        raise ValueError(f"children_max={children_max} must be below the vocabulary V={V}")
    d2t = make_d2t(seed, V, Vd)
    parent = np.empty((B, N), np.int32)
    draft_ids = np.empty((B, N), np.int32)
    depth = np.empty((B, N), np.int32)
    planted = np.empty((B, N), np.int32)
    for b in range(B):
        parent[b], draft_ids[b], depth[b], planted[b] = _tree_sequence(
            seed, rnd, b, N, V, d2t, p_match, depth_max, children_max)
    out = TreeBatch(B, N, V, Vd, dtype, parent, draft_ids, d2t, planted, depth)
    if logits:
        out.logits = np.concatenate(
            [_planted_logits(seed, rnd, b, planted[b], V, dtype) for b in range(B)], axis=0)
    return out


# --------------------------------------------------------------------------- router


@dataclass
class RouterInputs:
    B: int
    d: int
    m: int
    dtype: str
    hidden: np.ndarray   # [B, d] float32 or uint16 (bf16 bits)
    W1: np.ndarray       # [m, d] same dtype
    b1: np.ndarray       # float32 [m]
    W2: np.ndarray       # [m] same dtype
    b2: float            # float32 value
    tau: float = TAU


def make_router_inputs(seed: int, B: int, d: int = D_QWEN3, m: int = ROUTER_M,
                       dtype: str = "bf16", rnd: int = 0, b2: float = 0.0) -> RouterInputs:
    gw = _rng(seed, _S_WEIGHTS)
    W1 = gw.standard_normal((m, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    W2 = gw.standard_normal(m, dtype=np.float32) * np.float32(1.0 / np.sqrt(m))
    h = _rng(seed, _S_HIDDEN, rnd).standard_normal((B, d), dtype=np.float32)
    return RouterInputs(B, d, m, dtype, _materialise(h, dtype), _materialise(W1, dtype),
                        np.zeros(m, np.float32), _materialise(W2, dtype), float(np.float32(b2)))


def negate_second_layer(r: RouterInputs) -> RouterInputs:
    """The same router with W2, b2 and tau negated (sign flips only, exact in bf16 and f32).

    Its gain is the negated gain and its threshold the negated threshold, so a
    sequence with gain g takes choice 1 iff -g > -tau, i.e. iff g < tau.  This is
    how the routed workload is posed under the reading that sends gains above
    the threshold to the DFlash chain, with the library's fixed convention
    (choice 1 = EAGLE-3 iff gain > threshold) left unchanged.
    """
    if r.dtype == "bf16":
        W2 = (np.asarray(r.W2, np.uint16) ^ np.uint16(0x8000)).astype(np.uint16)
    else:
        W2 = -np.asarray(r.W2, np.float32)
    return RouterInputs(r.B, r.d, r.m, r.dtype, r.hidden, r.W1, r.b1, W2,
                        float(-np.float32(r.b2)), float(-np.float32(r.tau)))


# --------------------------------------------------------------------------- routed


def routed_calibration() -> dict:
    """Stored b2 and per-sequence layout for the routed workload (written by the oracle)."""
    with open(_CALIBRATION) as f:
        return json.load(f)


@dataclass
class RoutedBatch:
    B: int
    K: int
    N: int
    V: int
    Vd: int
    dtype: str
    layout_choice: np.ndarray  # int32 [B]: 1 = tree rows, 0 = chain rows
    offsets: np.ndarray        # int32 [B+1]
    chain_draft: np.ndarray    # int32 [B, K]   (rows of tree sequences unused)
    parent: np.ndarray         # int32 [B, N]   (rows of chain sequences unused)
    draft_ids: np.ndarray      # int32 [B, N]
    d2t: np.ndarray
    planted: list = field(default_factory=list)
    router: RouterInputs | None = None
    logits: np.ndarray | None = None

    @property
    def rows(self) -> int:
        return int(self.offsets[-1])


def make_routed_batch(seed: int, layout_choice: np.ndarray, K: int = 16, N: int = 61,
                      V: int = V_QWEN3, Vd: int = VD_EAGLE3, dtype: str = "bf16",
                      p_chain: float = 0.8, p_tree: float = 0.7, rnd: int = 0,
                      logits: bool = True) -> RoutedBatch:
    """Ragged packed batch: sequence b has K+1 chain rows (layout 0) or N tree rows (layout 1)."""
    layout_choice = np.asarray(layout_choice, np.int32)
    B = layout_choice.shape[0]
    d2t = make_d2t(seed, V, Vd)
    offsets = np.zeros(B + 1, np.int32)
    chain_draft = np.full((B, K), -1, np.int32)
    parent = np.full((B, N), -1, np.int32)
    draft_ids = np.full((B, N), -1, np.int32)
    planted = []
    for b in range(B):
        if layout_choice[b] == 1:
            pa, di, _, pl = _tree_sequence(seed, rnd, b, N, V, d2t, p_tree, 8, 10)
            parent[b], draft_ids[b] = pa, di
        else:
            g = _rng(seed, _S_CHAIN, rnd, b)
            pl = g.integers(0, V, size=K + 1).astype(np.int32)
            for i in range(K):
                chain_draft[b, i] = pl[i] if g.random() < p_chain else _other_id(g, V, int(pl[i]))
        planted.append(pl)
        offsets[b + 1] = offsets[b] + pl.shape[0]
    out = RoutedBatch(B, K, N, V, Vd, dtype, layout_choice, offsets, chain_draft, parent,
                      draft_ids, d2t, planted)
    if logits:
        out.logits = np.concatenate(
            [_planted_logits(seed, rnd, b, planted[b], V, dtype) for b in range(B)], axis=0)
    return out


# --------------------------------------------------------------------------- configs

# The five workloads, by name (seeds 0-4).
CONFIGS = {
    "single_chain_f32": dict(seed=0, kind="chain", B=1, K=16, dtype="f32", router=True),
    "batched_chain_bf16": dict(seed=1, kind="chain", B=32, K=16, dtype="bf16", router=True),
    "tree_bf16": dict(seed=2, kind="tree", B=8, N=61, dtype="bf16", router=False),
    "routed_bf16": dict(seed=3, kind="routed", B=128, K=16, N=61, dtype="bf16", router=True),
    "sweep_bf16": dict(seed=4, kind="chain", B=256, K=16, dtype="bf16", router=True, rounds=100),
}


def make_config(name: str, rnd: int = 0, logits: bool = True, V: int = V_QWEN3,
                polarity: str = "paper"):
    """Returns (batch, router_inputs_or_None) for one of the five workloads.

    polarity applies to the routed workload only.  "paper": a gain above the
    threshold picks the EAGLE-3 tree (WhiFlash paper, section 3.3.2, decision
    rule pi(h_t, tau_neural)).  "literal": a gain above the threshold is
    verified as a DFlash chain; the router comes from negate_second_layer and
    every sequence swaps its layout (same hidden states, exact 64/64 split, same
    1e-3 margin)."""
    c = CONFIGS[name]
    seed = c["seed"]
    if c["kind"] == "chain":
        batch = make_chain_batch(seed, c["B"], c["K"], V, c["dtype"], 0.8, rnd, logits)
        router = make_router_inputs(seed, c["B"], dtype=c["dtype"], rnd=rnd)
        return batch, router
    if c["kind"] == "tree":
        return make_tree_batch(seed, c["B"], c["N"], V, VD_EAGLE3, c["dtype"], 0.7, 8, 10,
                               rnd, logits), None
    if polarity not in ("paper", "literal"):
        raise ValueError(f"unknown polarity {polarity!r}")
    cal = routed_calibration()
    router = make_router_inputs(seed, c["B"], dtype=c["dtype"], rnd=rnd, b2=cal["b2"])
    layout = np.asarray(cal["choice"], np.int32)
    if polarity == "literal":
        router = negate_second_layer(router)
        layout = 1 - layout
    batch = make_routed_batch(seed, layout, c["K"], c["N"], V, VD_EAGLE3, c["dtype"], 0.8, 0.7,
                              rnd, logits)
    batch.router = router
    return batch, router


def make_hidden_rows(seed: int, rows: int, d: int = D_QWEN3, dtype: str = "bf16") -> np.ndarray:
    """Final hidden states for every verified row: N(0, 1), one seeded stream."""
    x = _rng(seed, _S_HIDDEN, 1_000_003).standard_normal((rows, d), dtype=np.float32)
    return _materialise(x, dtype)
