"""Plain CPU definitions of the WhiFlash per-round route + greedy verify + emit step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources (cited by page title and section):
  [paper]  "WhiFlash: Accelerating Speculative Decoding with Token-Level
           Cross-Paradigm Routing" (arXiv 2606.07710).
  [router] model card "Qwen3-4B-NeuralRouter-df-e3".
  [eagle]  model card "Qwen3-4B-EAGLE3".

Readings taken where the pages leave a step open are listed beside the code
that takes them.  Floating-point work is done in float64 from the exact input
values; integer work is exact.
"""

from __future__ import annotations

import math

import numpy as np

MALFORMED_AL = 0
MALFORMED_BONUS = -1


# ----------------------------------------------------------------------------- logits


def decode_logits(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored logits.

    bfloat16 is the upper half of an IEEE binary32 word, so placing its 16 bits
    in the high half of a 32-bit word gives the same number exactly.
    """
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN, as they should
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def row_argmax(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Greedy target token of every logits row: the lowest index holding the row maximum.

    Greedy verification accepts a draft token when it equals the target's most
    likely token ([router] "Evaluation": greedy decoding; [paper] §3.3.1 notes
    that greedy decoding needs no softmax).  Definition used here, per row x:
    t = min{ i : x[i] == max_k x[k] } under IEEE equality, so -0 and +0 tie and
    ties go to the lowest index.  Precondition: no NaN (the pages are silent on
    NaN logits).
    """
    raw = np.asarray(raw)
    out = np.empty(raw.shape[0], np.int64)
    for r in range(raw.shape[0]):
        x = decode_logits(raw[r], dtype)
        if np.isnan(x).any():
            raise ValueError(f"row {r} holds NaN; the greedy argmax is undefined")
        top = x.max()
        out[r] = np.flatnonzero(x == top)[0]
    return out


# ----------------------------------------------------------------------------- router


def gelu(z: np.ndarray) -> np.ndarray:
    """Gaussian Error Linear Unit z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)).

    [paper] Appendix A "Neural Router Architecture" names GELU (Hendrycks and
    Gimpel) without a formula; the exact-erf form is taken.
    """
    erf = np.vectorize(math.erf, otypes=[np.float64])
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def route(hidden, W1, b1, W2, b2, tau: float, dtype: str):
    """Neural router and hardware-aware threshold.

    [paper] §3.3.2: the router f_theta maps the final-layer hidden state h_t to
    a scalar predicted gain Delta-AL = f_theta(h_t), and the decision rule
    pi(h_t, tau_neural) picks the autoregressive drafter m_a (EAGLE-3) when
    Delta-AL > tau_neural, else the diffusion drafter m_d (DFlash).
    [paper] Appendix A: linear d -> m, GELU, dropout, linear m -> 1.
    Readings: dropout is the identity at inference; b1 and b2 are present (the
    parameter counts of the paper's router table include them), None meaning 0;
    the threshold is strict, so Delta-AL == tau picks DFlash.
    Returns (delta_al float64 [B], choice int32 [B]) with choice 1 = EAGLE-3 tree,
    0 = DFlash chain.
    """
    h = decode_logits(hidden, dtype).reshape(np.asarray(hidden).shape)
    w1 = decode_logits(W1, dtype).reshape(np.asarray(W1).shape)
    w2 = decode_logits(W2, dtype).reshape(-1)
    m = w1.shape[0]
    bias1 = np.zeros(m) if b1 is None else np.asarray(b1, np.float32).astype(np.float64)
    bias2 = 0.0 if b2 is None else float(np.float32(b2))
    z = h @ w1.T + bias1                 # layer 1: [B, m]
    g = gelu(z)                          # GELU; dropout = identity
    delta_al = g @ w2 + bias2            # layer 2: [B]
    choice = (delta_al > float(np.float32(tau))).astype(np.int32)
    return delta_al, choice


def route_gather(hidden_rows, rows, W1, b1, W2, b2, tau: float, dtype: str):
    """The neural router fed from the hidden state at each sequence's final accepted position.

    [paper] §3.3.2: the policy takes the target's final-layer hidden state at
    the current decoding step; with speculative decoding that is the state at
    the final accepted position (§3.3.1 uses the same position).  rows[b] is
    the packed row of that position; an index outside [0, total_rows) gives
    Delta-AL = NaN and choice 0.  Returns (delta_al float64 [B], choice int32 [B]).
    """
    hidden_rows = np.asarray(hidden_rows)
    rows = np.asarray(rows, np.int64)
    total = hidden_rows.shape[0]
    B = rows.shape[0]
    dal = np.full(B, np.nan)
    choice = np.zeros(B, np.int32)
    ok = (rows >= 0) & (rows < total)
    if ok.any():
        d_ok, c_ok = route(hidden_rows[rows[ok]], W1, b1, W2, b2, tau, dtype)
        dal[ok], choice[ok] = d_ok, c_ok
    return dal, choice


def entropy(raw_row: np.ndarray, dtype: str) -> float:
    """Entropy (nats) of the target's next-token distribution from one logits row.

    [paper] §3.3.1 "Runtime-Informed Policy": H_t = -sum_x p(x) log p(x) over
    the vocabulary at the final accepted position; under greedy decoding p is
    the softmax of the logits (temperature 1).  Computed in float64 as
    p = exp(x - max) / sum exp(x - max), with 0 log 0 = 0.  Precondition:
    finite logits.
    """
    x = decode_logits(raw_row, dtype)
    if not np.isfinite(x).all():
        raise ValueError("entropy needs finite logits")
    e = np.exp(x - x.max())
    p = e / e.sum()
    nz = p[p > 0]
    return float(-(nz * np.log(nz)).sum())


def route_entropy(raw: np.ndarray, dtype: str, rows, tau: float):
    """WhiFlash-Entropy decision for each sequence from the row at its final accepted position.

    [paper] §3.3.1, decision rule pi(H_t, tau_entropy): the autoregressive
    drafter m_a (EAGLE-3, choice 1) when H_t > tau_entropy, else the diffusion
    drafter m_d (DFlash, choice 0).  rows[b] is the packed row index of that
    position; an index outside [0, total_rows) gives H = NaN and choice 0.
    Returns (H float64 [B], choice int32 [B]).
    """
    raw = np.asarray(raw)
    total = raw.shape[0]
    B = len(rows)
    H = np.full(B, np.nan)
    choice = np.zeros(B, np.int32)
    thr = float(np.float32(tau))
    for b in range(B):
        r = int(rows[b])
        if 0 <= r < total:
            H[b] = entropy(raw[r], dtype)
            choice[b] = 1 if H[b] > thr else 0
    return H, choice


# ----------------------------------------------------------------------------- verify


def verify_chain(t: np.ndarray, draft: np.ndarray):
    """DFlash block acceptance under greedy verification.

    [paper] §3.2: the drafted block goes back to the target for parallel
    verification, and decoding continues from the last accepted token; §4
    "Metrics": acceptance length counts the tokens accepted per verification
    round.  Reading: row i of a sequence's K+1 rows is the target's prediction
    after the first i draft tokens; the accepted prefix is the longest run
    draft[0..n-1] == t[0..n-1], and the target's own token t[n] is emitted as
    the bonus, so AL = n + 1.
    t: int [B, K+1] row argmaxes; draft: int [B, K].  Returns (AL, bonus) int32 [B].
    """
    t = np.asarray(t)
    draft = np.asarray(draft)
    B, K = draft.shape
    al = np.empty(B, np.int32)
    bonus = np.empty(B, np.int32)
    for b in range(B):
        n = 0
        while n < K and int(draft[b, n]) == int(t[b, n]):
            n += 1
        al[b] = n + 1
        bonus[b] = t[b, n]
    return al, bonus


def tree_accepted(t, parent, draft_ids, d2t, V):
    """Accepted nodes of one tree, and their depths.

    Same reading as verify_tree ([paper] §3.2; [eagle] "Model Description"):
    node 0 is accepted at depth 0; in index order, node u >= 1 is accepted iff
    0 <= parent[u] = p < u, p is accepted, draft_ids[u] lies in the draft
    vocabulary, its table entry lies in the target vocabulary, and that target
    id equals t[p]; its depth is then depth[p] + 1.
    t, parent, draft_ids: int [N]; d2t: int [Vd].  Returns (bool [N], int [N]).
    """
    N = len(parent)
    Vd = len(d2t)
    accepted = [False] * N
    depth = [0] * N
    accepted[0] = True
    for u in range(1, N):
        p = int(parent[u])
        if not (0 <= p < u):
            continue                      # malformed parent: node unreachable
        did = int(draft_ids[u])
        if not (0 <= did < Vd):
            continue                      # id outside the draft vocabulary
        tok = int(d2t[did])
        if not (0 <= tok < V):
            continue                      # table entry outside the target vocabulary
        if accepted[p] and tok == int(t[p]):
            accepted[u] = True
            depth[u] = depth[p] + 1
    return np.array(accepted, bool), np.array(depth, np.int64)


def _tree_one(t, parent, draft_ids, d2t, V):
    accepted, depth = tree_accepted(t, parent, draft_ids, d2t, V)
    best = min((u for u in range(len(parent)) if accepted[u]), key=lambda u: (-depth[u], u))
    return int(depth[best]) + 1, int(t[best]), best


def verify_tree(t: np.ndarray, parent: np.ndarray, draft_ids: np.ndarray, d2t: np.ndarray, V: int):
    """EAGLE-3 tree acceptance under greedy verification, with the d2t remap.

    [paper] §3.2: the autoregressive drafter returns a tree of candidate tokens
    for parallel verification; [eagle] "Model Description": the drafter proposes
    ids of a fixed 32K draft vocabulary, mapped to target ids.  Readings: node 0
    is the root (the last verified token) and row u is the target's prediction
    after node u; node u >= 1 is accepted iff its parent p = parent[u] satisfies
    0 <= p < u, p is accepted, and d2t[draft_ids[u]] == t[p] (ids outside the
    draft vocabulary or table entries outside the target vocabulary never
    match); the kept path ends at the deepest accepted node, lowest index on
    ties; AL = its depth + 1 and the bonus is the target's token at it.
    Returns (AL, bonus, best_node) int32 [B].
    """
    t = np.asarray(t)
    B, N = np.asarray(parent).shape
    al = np.empty(B, np.int32)
    bonus = np.empty(B, np.int32)
    best = np.empty(B, np.int32)
    for b in range(B):
        al[b], bonus[b], best[b] = _tree_one(t[b], parent[b], draft_ids[b], d2t, V)
    return al, bonus, best


def verify_routed(t_rows: np.ndarray, offsets: np.ndarray, choice: np.ndarray, K: int,
                  chain_draft: np.ndarray, N: int, parent: np.ndarray, draft_ids: np.ndarray,
                  d2t: np.ndarray, V: int):
    """Per-sequence dispatch of a ragged batch to chain or tree acceptance.

    [paper] §3.3: the router is invoked once per speculation round and selects,
    per sequence and step, which drafter's candidates are verified.  Sequence b
    owns packed rows [offsets[b], offsets[b+1]).  choice 0 (DFlash) needs K+1
    rows, choice 1 (EAGLE-3) needs N rows; any other combination, or offsets
    outside [0, total_rows] or decreasing, is malformed: AL = 0, bonus = -1,
    best_node = -1.  For chain sequences best_node is the index of the last
    accepted chain position (AL - 1).
    Returns (AL, bonus, best_node) int32 [B].
    """
    t_rows = np.asarray(t_rows)
    total = t_rows.shape[0]
    B = len(choice)
    al = np.full(B, MALFORMED_AL, np.int32)
    bonus = np.full(B, MALFORMED_BONUS, np.int32)
    best = np.full(B, -1, np.int32)
    for b in range(B):
        lo, hi, c = int(offsets[b]), int(offsets[b + 1]), int(choice[b])
        if not (0 <= lo <= hi <= total):
            continue
        if c == 0 and hi - lo == K + 1:
            a, bo = verify_chain(t_rows[lo:hi][None, :], np.asarray(chain_draft[b])[None, :K])
            al[b], bonus[b], best[b] = a[0], bo[0], a[0] - 1
        elif c == 1 and hi - lo == N:
            a, bo, be = verify_tree(t_rows[lo:hi][None, :], np.asarray(parent[b])[None, :],
                                    np.asarray(draft_ids[b])[None, :], d2t, V)
            al[b], bonus[b], best[b] = a[0], bo[0], be[0]
    return al, bonus, best


# ----------------------------------------------------------------------------- lazy catch-up


def catchup_update(cur, accept_len, nxt, backlog):
    """Backlog bookkeeping of lazy catch-up for one round.

    [paper] §3.4 "Lazy Catch-up": the inactive drafter's KV cache is not
    updated; tokens accepted while a drafter is inactive are its backlog, and
    when a switch to it is committed it prefills that backlog in one batch.
    Per sequence: this round's accepted tokens are added to the backlog of the
    drafter that was not used (1 - cur); if the next round's drafter differs
    (a switch), the incoming drafter's backlog is its catch-up length and is
    reset to 0.  cur or nxt outside {0, 1} (e.g. a malformed sequence) leaves
    the sequence unchanged with no switch.
    backlog: int [B, 2] (column 0 DFlash, column 1 EAGLE-3), not modified.
    Returns (new_backlog [B, 2], switch [B], catchup [B]) int32.
    """
    cur = np.asarray(cur)
    B = cur.shape[0]
    out = np.array(backlog, dtype=np.int64).reshape(B, 2)
    switch = np.zeros(B, np.int32)
    catchup = np.zeros(B, np.int32)
    for b in range(B):
        c, n, a = int(cur[b]), int(nxt[b]), int(accept_len[b])
        if c not in (0, 1) or n not in (0, 1):
            continue
        out[b, 1 - c] += max(a, 0)
        if n != c:
            switch[b] = 1
            catchup[b] = out[b, n]
            out[b, n] = 0
    return out.astype(np.int32), switch, catchup
