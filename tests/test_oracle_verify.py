"""Pins of the oracle's chain, tree and routed acceptance.

Pinned against: brute-force enumeration of every matching prefix (chain) and of
every root path (tree) on exhaustive tiny inputs; the invariants the method
fixes (1 <= AL <= K+1, all-match gives K+1, first-position mismatch gives 1,
lossless emission equals the target's own greedy tokens); tree-as-chain
equivalence; star trees; malformed and out-of-domain inputs.
"""

import itertools

import numpy as np

from oracle import verify_chain, verify_routed, verify_tree, MALFORMED_AL, MALFORMED_BONUS


# ------------------------------------------------------------------ chain


def _chain_brute(t, draft):
    K = len(draft)
    # longest j such that the first j drafts equal the first j target tokens
    best = max(j for j in range(K + 1) if list(draft[:j]) == list(t[:j]))
    return best + 1, t[best]


def test_chain_exhaustive_small():
    V = 3
    for K in range(0, 4):
        for t in itertools.product(range(V), repeat=K + 1):
            for draft in itertools.product(list(range(V)) + [-1, V], repeat=K):
                al, bo = verify_chain(np.array([t]), np.array([draft], np.int64).reshape(1, K))
                e_al, e_bo = _chain_brute(t, draft)
                assert (al[0], bo[0]) == (e_al, e_bo), (t, draft)


def test_chain_invariants_and_lossless():
    rng = np.random.default_rng(3)
    for _ in range(500):
        K = int(rng.integers(0, 20))
        t = rng.integers(0, 5, size=K + 1)
        draft = np.where(rng.random(K) < 0.7, t[:K], rng.integers(0, 5, size=K))
        al, bo = verify_chain(t[None], draft[None])
        al, bo = int(al[0]), int(bo[0])
        assert 1 <= al <= K + 1
        emitted = list(draft[: al - 1]) + [bo]
        # lossless: the emitted tokens are exactly the target's own greedy tokens
        assert emitted == list(t[:al])
    t = np.arange(17)
    assert verify_chain(t[None], t[None, :16])[0][0] == 17            # all match
    d = t[:16].copy()
    d[0] += 1
    assert tuple(x[0] for x in verify_chain(t[None], d[None])) == (1, 0)  # first mismatch


# ------------------------------------------------------------------ tree


def _tree_brute(t, parent, tok):
    """Enumerate every root path; a path is kept when every non-root node on it matches."""
    N = len(parent)
    best_len, best_node = 0, 0
    for u in range(N):
        path, v, ok = [], u, True
        while v != 0:
            p = parent[v]
            if not (0 <= p < v):
                ok = False
                break
            path.append(v)
            v = p
        if not ok:
            continue
        if all(tok[w] == t[parent[w]] for w in path):
            if len(path) > best_len or (len(path) == best_len and u < best_node):
                best_len, best_node = len(path), u
    return best_len + 1, t[best_node], best_node


def _all_parent_arrays(N):
    return itertools.product(*[range(u) for u in range(1, N)])


def test_tree_exhaustive_small():
    V = 4
    d2t = np.arange(V, dtype=np.int32)  # identity table: draft id == target id
    t = np.array([0, 1, 2, 3, 0, 1], np.int32)
    for N in range(1, 6):
        for pa in _all_parent_arrays(N):
            parent = np.array((-1,) + pa, np.int32)
            for pattern in itertools.product([0, 1], repeat=N - 1):
                tok = np.full(N, -1, np.int32)
                for u in range(1, N):
                    want = t[parent[u]]
                    tok[u] = want if pattern[u - 1] else (want + 1) % V
                al, bo, be = verify_tree(t[None, :N], parent[None], tok[None], d2t, V)
                assert (al[0], bo[0], be[0]) == _tree_brute(t[:N], parent, tok), (parent, tok)


def test_tree_as_chain_equals_chain():
    rng = np.random.default_rng(11)
    V = 6
    d2t = np.arange(V, dtype=np.int32)
    for _ in range(300):
        K = int(rng.integers(0, 12))
        t = rng.integers(0, V, size=K + 1).astype(np.int32)
        draft = np.where(rng.random(K) < 0.75, t[:K], rng.integers(0, V, size=K)).astype(np.int32)
        parent = np.arange(-1, K, dtype=np.int32)            # node u's parent is u-1
        ids = np.concatenate([[-1], draft]).astype(np.int32)  # node u carries draft[u-1]
        al_t, bo_t, be_t = verify_tree(t[None], parent[None], ids[None], d2t, V)
        al_c, bo_c = verify_chain(t[None], draft[None])
        assert (al_t[0], bo_t[0], be_t[0]) == (al_c[0], bo_c[0], al_c[0] - 1)


def test_star_tree_accepts_at_most_one():
    V = 10
    d2t = np.arange(V, dtype=np.int32)
    N = 8
    parent = np.array([-1] + [0] * (N - 1), np.int32)
    ids = np.array([-1, 1, 2, 3, 4, 5, 6, 7], np.int32)
    t = np.zeros(N, np.int32)
    for root_tok in range(V):
        t[0] = root_tok
        al, bo, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
        assert al[0] <= 2
        if 1 <= root_tok <= 7:
            assert (al[0], be[0]) == (2, root_tok)
        else:
            assert (al[0], be[0], bo[0]) == (1, 0, root_tok)


def test_tree_out_of_domain_never_matches():
    V, Vd = 5, 4
    d2t = np.array([0, 1, 9, -3], np.int32)   # entries 2 and 3 fall outside the target vocab
    t = np.array([1, 0, 9, 0, 0], np.int32)
    parent = np.array([-1, 0, 0, 0, 0], np.int32)
    for did in [-1, Vd, 2, 3]:
        ids = np.array([-1, did, did, did, did], np.int32)
        al, _, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
        assert (al[0], be[0]) == (1, 0)
    ids = np.array([-1, 1, 1, 1, 1], np.int32)
    al, _, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
    assert (al[0], be[0]) == (2, 1)                 # lowest index among equally deep nodes


def test_tree_malformed_parent_unreachable():
    V = 4
    d2t = np.arange(V, dtype=np.int32)
    t = np.array([1, 2, 3, 0], np.int32)
    ids = np.array([-1, 1, 2, 3], np.int32)
    ok = np.array([-1, 0, 1, 2], np.int32)
    assert verify_tree(t[None], ok[None], ids[None], d2t, V)[0][0] == 4
    for bad in ([-1, 0, 2, 2], [-1, 0, 1, 3], [-1, 0, -5, 2], [-1, 1, 1, 2]):
        al, _, be = verify_tree(t[None], np.array(bad, np.int32)[None], ids[None], d2t, V)
        assert al[0] < 4


def test_generated_trees_respect_depth_bound():
    from synth import make_tree_batch
    from oracle import row_argmax
    tb = make_tree_batch(5, B=6, N=61, V=2000, Vd=500, dtype="bf16")
    t = row_argmax(tb.logits, "bf16").reshape(6, 61)
    al, bo, be = verify_tree(t, tb.parent, tb.draft_ids, tb.d2t, 2000)
    assert np.all(al >= 1) and np.all(al <= 9)
    assert np.all(al == tb.depth[np.arange(6), be] + 1)
    assert np.array_equal(bo, t[np.arange(6), be])


# ------------------------------------------------------------------ routed


def test_routed_dispatch_and_malformed():
    V = 6
    K, N = 2, 3
    d2t = np.arange(V, dtype=np.int32)
    # seq0 chain (3 rows), seq1 tree (3 rows), seq2 chain but 3-row tree layout claim, seq3 bad choice
    t_rows = np.array([1, 2, 3, 4, 5, 0, 1, 1, 1, 2, 2, 2], np.int32)
    offsets = np.array([0, 3, 6, 9, 12], np.int32)
    choice = np.array([0, 1, 0, 7], np.int32)
    chain_draft = np.array([[1, 2], [0, 0], [1, 9], [0, 0]], np.int32)
    parent = np.array([[-1, 0, 1]] * 4, np.int32)
    ids = np.array([[-1, 4, 5]] * 4, np.int32)
    al, bo, be = verify_routed(t_rows, offsets, choice, K, chain_draft, N, parent, ids, d2t, V)
    assert (al[0], bo[0], be[0]) == (3, 3, 2)
    assert (al[1], bo[1], be[1]) == (3, 0, 2)
    assert (al[2], bo[2], be[2]) == (2, 1, 1)
    assert (al[3], bo[3], be[3]) == (MALFORMED_AL, MALFORMED_BONUS, -1)
    bad = np.array([0, 3, 2, 9, 12], np.int32)     # decreasing offsets
    al, bo, be = verify_routed(t_rows, bad, choice[:4], K, chain_draft, N, parent, ids, d2t, V)
    assert al[1] == MALFORMED_AL and al[2] == MALFORMED_AL
    over = np.array([0, 3, 6, 9, 15], np.int32)    # past total_rows
    al, _, _ = verify_routed(t_rows, over, choice, K, chain_draft, N, parent, ids, d2t, V)
    assert al[3] == MALFORMED_AL and al[0] == 3


# ------------------------------------------------------------------ accepted-node sets


def _accepted_by_path(t, parent, ids, d2t, V, u):
    """Node u is accepted iff every edge on its walk up to the root is well formed and matches."""
    while u != 0:
        p = int(parent[u])
        if not (0 <= p < u):
            return False
        did = int(ids[u])
        if not (0 <= did < len(d2t)) or not (0 <= int(d2t[did]) < V) or int(d2t[did]) != int(t[p]):
            return False
        u = p
    return True


def test_tree_accepted_matches_root_path_walk():
    from oracle import tree_accepted
    rng = np.random.default_rng(21)
    V, Vd = 4, 5
    d2t = np.array([0, 1, 2, 3, 7], np.int32)      # id 4 maps outside the target vocabulary
    for _ in range(2000):
        N = int(rng.integers(1, 12))
        parent = np.array([-1] + [int(rng.integers(-1, u + 1)) for u in range(1, N)], np.int32)
        ids = rng.integers(-1, Vd + 1, size=N).astype(np.int32)
        t = rng.integers(0, V, size=N).astype(np.int32)
        acc, depth = tree_accepted(t, parent, ids, d2t, V)
        for u in range(N):
            assert acc[u] == _accepted_by_path(t, parent, ids, d2t, V, u)
        al, bo, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
        assert acc[be[0]] and depth[be[0]] == al[0] - 1 == depth[acc].max()


def test_tree_accepted_duplicate_siblings_both_accepted():
    from oracle import tree_accepted
    V = 6
    d2t = np.arange(V, dtype=np.int32)
    parent = np.array([-1, 0, 0, 1, 2], np.int32)
    ids = np.array([-1, 3, 3, 5, 5], np.int32)     # siblings 1 and 2 carry the same token
    t = np.array([3, 5, 5, 0, 0], np.int32)
    acc, depth = tree_accepted(t, parent, ids, d2t, V)
    assert acc.tolist() == [True, True, True, True, True]
    assert depth.tolist() == [0, 1, 1, 2, 2]
    al, bo, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
    assert (al[0], be[0]) == (3, 3)                # deepest, lowest index among equals


def test_tree_accepted_of_a_chain_is_its_accepted_prefix():
    from oracle import tree_accepted
    rng = np.random.default_rng(22)
    V = 5
    d2t = np.arange(V, dtype=np.int32)
    for _ in range(300):
        K = int(rng.integers(0, 10))
        t = rng.integers(0, V, size=K + 1).astype(np.int32)
        draft = np.where(rng.random(K) < 0.7, t[:K], rng.integers(0, V, size=K)).astype(np.int32)
        parent = np.arange(-1, K, dtype=np.int32)
        ids = np.concatenate([[-1], draft]).astype(np.int32)
        acc, _ = tree_accepted(t, parent, ids, d2t, V)
        al, _ = verify_chain(t[None], draft[None])
        assert acc.tolist() == [i < al[0] for i in range(K + 1)]


# ------------------------------------------------------------------ d2t remap, exact cases
#
# Draft ids index a fixed 32K draft vocabulary and are mapped to target ids by
# the d2t table before they are compared with the target's tokens (Qwen3-4B-EAGLE3
# card, "Model Description" and "Technical Specifications").  The trees below use
# tables far from the identity, and every expected value was derived by hand.
# Each case also states what two wrong readings would give (comparing the draft
# id itself, or looking the id up in the inverse table), so a mistake of either
# kind changes AL, bonus and best node at once.


def test_tree_d2t_reversed_table_exact():
    V = Vd = 8
    d2t = np.array([7, 6, 5, 4, 3, 2, 1, 0], np.int32)       # d2t[i] = 7 - i
    parent = np.array([-1, 0, 1, 0, 3], np.int32)
    ids = np.array([-1, 2, 6, 5, 1], np.int32)               # target ids 5, 1, 2, 6
    t = np.array([5, 1, 4, 6, 0], np.int32)
    # Remapped: node 1 (5 == t[0]) and node 2 (1 == t[1]) are accepted, node 3
    # (2 != t[0]) is not, so node 4 is unreachable.  Deepest node 2 at depth 2:
    # AL 3, bonus t[2] = 4.
    al, bo, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
    assert (al[0], bo[0], be[0]) == (3, 4, 2)
    # Wrong reading (no remap): node 3's raw id 5 == t[0] would win at depth 1
    # (AL 2, bonus 6, best 3).  The table here is its own inverse, so the next
    # case covers the inverted lookup.
    assert (al[0], bo[0], be[0]) != (2, 6, 3)


def test_tree_d2t_injective_into_larger_vocab_exact():
    V, Vd = 10, 6
    d2t = np.array([3, 0, 7, 4, 1, 8], np.int32)             # (7 i + 3) mod 10, not an involution
    parent = np.array([-1, 0, 0, 1, 3, 2], np.int32)
    ids = np.array([-1, 2, 0, 4, 5, 1], np.int32)            # target ids 7, 3, 1, 8, 0
    t = np.array([7, 1, 0, 8, 2, 9], np.int32)
    # Remapped: node 1 (7 == t[0]), node 3 (1 == t[1]) and node 4 (8 == t[3])
    # are accepted; node 2 (3 != t[0]) is not, so node 5 is unreachable even
    # though its target id 0 equals t[2].  Deepest node 4 at depth 3: AL 4,
    # bonus t[4] = 2.
    al, bo, be = verify_tree(t[None], parent[None], ids[None], d2t, V)
    assert (al[0], bo[0], be[0]) == (4, 2, 4)
    # No remap: raw ids 2 and 0 under the root both differ from t[0] = 7 (AL 1).
    # Inverse lookup: id 2 is not a table entry and id 0 is entry 1 != 7 (AL 1).
    # Through the routed dispatch, the same tree behind a chain sequence gives
    # the same result.
    t_rows = np.concatenate([np.array([7, 7, 7], np.int32), t])
    offsets = np.array([0, 3, 9], np.int32)
    choice = np.array([0, 1], np.int32)
    chain_draft = np.array([[7, 7], [0, 0]], np.int32)
    al, bo, be = verify_routed(t_rows, offsets, choice, 2, chain_draft, 6,
                               np.stack([parent, parent]), np.stack([ids, ids]), d2t, V)
    assert al.tolist() == [3, 4] and bo.tolist() == [7, 2] and be.tolist() == [2, 4]
