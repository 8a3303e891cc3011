"""Pins for the oracle's Markov-head edge scores and the parent-conditioned best-first build
(CPU only).

The head scores candidate y at position s as l_s(y) = bases(y) + <W1[x_{s-1}], W2[y]>, with
x_{s-1} the previous token (SpecPilot summary, Prerequisites > parallel drafters and
lattices); in a tree the previous token is the parent's.  Each test fixes the oracle against
something other than its own code: a hand-worked case, the special cases that reduce to a
library log-softmax or to the unconditioned build, a brute-force enumeration of every root
path, and invariants of the conditioning.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import log_softmax

import oracle


def _markov_inputs(rng, B, P, K, V=50, R=4, distinct=True):
    bases = rng.normal(0, 2, size=(B, P, K)).astype(np.float32)
    tok = np.stack([np.stack([rng.permutation(V)[:K] for _ in range(P)]) for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, V, size=B).astype(np.int32)
    W1 = rng.normal(0, 1 / math.sqrt(R), size=(V, R)).astype(np.float32)
    W2 = rng.normal(0, 1 / math.sqrt(R), size=(V, R)).astype(np.float32)
    return bases, tok, root, W1, W2


def test_hand_worked_edge():
    """K = 2, R = 1, zero bases, W1[x] = 1 for the root token, W2 = (ln 2, 0) for the two
    candidates: the logits are (ln 2, 0), so p = (2/3, 1/3) and the edge log-probs are
    (ln 2/3, ln 1/3).  At position 1 the parent token of row pr = 0 is candidate 0, whose
    W1 is 0: both children get ln 1/2."""
    bases = np.zeros((1, 2, 2), np.float32)
    tok = np.array([[[1, 2], [1, 2]]], np.int32)
    root = np.array([0], np.int32)
    W1 = np.array([[1.0], [0.0], [3.0]], np.float32)
    W2 = np.array([[0.0], [math.log(2.0)], [0.0]], np.float32)
    e = oracle.markov_edge_logp(bases, tok, root, W1, W2)
    np.testing.assert_allclose(e[0, 0, 0], [math.log(2 / 3), math.log(1 / 3)], rtol=0, atol=1e-7)
    np.testing.assert_allclose(e[0, 0, 1], e[0, 0, 0], rtol=0, atol=0)  # position 0: the root, any row
    np.testing.assert_allclose(e[0, 1, 0], [math.log(0.5), math.log(0.5)], rtol=0, atol=1e-15)
    # row pr = 1: the parent is candidate 1 (token 2, W1 = 3): logits (3 ln 2, 0) -> (8/9, 1/9)
    np.testing.assert_allclose(e[0, 1, 1], [math.log(8 / 9), math.log(1 / 9)], rtol=0, atol=2e-7)


def test_zero_w1_is_the_plain_log_softmax():
    """W1 = 0: no conditioning; every row of a position is the log-softmax of its bases."""
    rng = np.random.default_rng(1)
    bases, tok, root, _, W2 = _markov_inputs(rng, 2, 3, 5)
    e = oracle.markov_edge_logp(bases, tok, root, np.zeros_like(W2), W2)
    for b in range(2):
        for s in range(3):
            ref = log_softmax(bases[b, s].astype(np.float64))
            for pr in range(5):
                np.testing.assert_allclose(e[b, s, pr], ref, rtol=1e-13, atol=1e-13)


def test_rows_are_distributions_and_condition_on_the_parent_token():
    """Every row exponentiates to a distribution; changing W1 of one token changes exactly the
    rows whose previous token it is (position 0: the root token; position s: candidate pr of
    position s-1), and changing W2 of one token only the entries of that candidate."""
    rng = np.random.default_rng(2)
    B, P, K = 2, 4, 6
    bases, tok, root, W1, W2 = _markov_inputs(rng, B, P, K)
    e = oracle.markov_edge_logp(bases, tok, root, W1, W2)
    np.testing.assert_allclose(np.exp(e).sum(-1), 1.0, rtol=0, atol=1e-12)
    x = int(tok[1, 1, 3])  # the previous token of rows (b=1, s=2, pr=3)
    W1b = W1.copy()
    W1b[x] += 0.5
    e2 = oracle.markov_edge_logp(bases, tok, root, W1b, W2)
    prev = np.zeros((B, P, K), np.int64)
    prev[:, 0, :] = root[:, None]
    prev[:, 1:, :] = tok[:, :-1, :]
    changed = np.any(e2 != e, axis=-1)
    np.testing.assert_array_equal(changed, prev == x)
    y = int(tok[0, 2, 1])
    W2b = W2.copy()
    W2b[y] += 0.5
    e3 = oracle.markov_edge_logp(bases, tok, root, W1, W2b)
    # the candidate's own entry moves against the rest of its row (log-softmax), and only
    # rows that hold the candidate change
    holds = np.zeros((B, P, K), bool)
    holds[:, :, :] = np.any(tok == y, axis=-1)[:, :, None]
    np.testing.assert_array_equal(np.any(e3 != e, axis=-1), holds)


def _lattice_cond(rng, B, P, K):
    logits = rng.normal(0, 2, size=(B, P, K, K))
    edge = (logits - np.log(np.exp(logits).sum(-1, keepdims=True))).astype(np.float32)
    tok = np.stack([np.stack([rng.permutation(1000)[:K] for _ in range(P)]) for _ in range(B)]).astype(np.int32)
    return edge, tok


def test_unconditioned_rows_give_the_plain_build():
    """Rows that ignore the parent (every pr row of a position the same) build the tree of the
    plain lattice, field for field."""
    rng = np.random.default_rng(3)
    for P, K, N in ((3, 4, 20), (4, 3, 64), (16, 16, 64), (2, 5, 40)):
        logits = rng.normal(0, 2, size=(3, P, K))
        lp = -np.sort(-(logits - np.log(np.exp(logits).sum(-1, keepdims=True))), axis=-1).astype(np.float32)
        tok = np.stack([np.stack([rng.permutation(1000)[:K] for _ in range(P)]) for _ in range(3)]).astype(np.int32)
        root = np.arange(3, dtype=np.int32)
        edge = np.repeat(lp[:, :, None, :], K, axis=2)
        a = oracle.build_tree_cond(edge, tok, root, N)
        b = oracle.build_tree(lp, tok, root, N)
        for f in ("parent", "depth", "rank", "token", "anc", "n_nodes"):
            np.testing.assert_array_equal(a[f], b[f])
        np.testing.assert_array_equal(np.nan_to_num(a["score"], nan=7.0), np.nan_to_num(b["score"], nan=7.0))


def _all_paths(edge_b, P, K):
    """Every trie node as (rank path, fp64 score summed root to leaf with the edge log-prob of
    each step conditioned on the previous rank)."""
    nodes = []
    for d in range(1, P + 1):
        for path in itertools.product(range(K), repeat=d):
            s = 0.0
            for pos, r in enumerate(path):
                pr = path[pos - 1] if pos >= 1 else 0
                s = s + float(np.float64(edge_b[pos, pr, r]))
            nodes.append((path, s))
    return nodes


@pytest.mark.parametrize("P,K,N", [(1, 4, 3), (2, 3, 8), (3, 3, 25), (4, 3, 64), (3, 4, 40), (4, 2, 30)])
def test_brute_force_top_n(P, K, N):
    """Continuous random conditioned scores (no ties a.s.): the tree is the top-N trie nodes
    by path score, inserted in descending order, with their scores."""
    rng = np.random.default_rng(100 * P + 10 * K + N)
    edge, tok = _lattice_cond(rng, 3, P, K)
    tree = oracle.build_tree_cond(edge, tok, np.arange(3), N)
    for b in range(3):
        expect = sorted(_all_paths(edge[b], P, K), key=lambda x: -x[1])[:N]
        n = int(tree["n_nodes"][b])
        paths = {0: ()}
        for i in range(1, n):
            paths[i] = paths[int(tree["parent"][b, i])] + (int(tree["rank"][b, i]),)
        got = [paths[i] for i in range(1, n)]
        assert got == [p for p, _ in expect]
        np.testing.assert_array_equal(tree["score"][b, 1:n], [s for _, s in expect])
        for i in range(1, n):  # tokens are the lattice candidates of the node's rank and depth
            d, r = int(tree["depth"][b, i]), int(tree["rank"][b, i])
            assert tree["token"][b, i] == tok[b, d - 1, r]


def test_ties_go_to_the_smaller_parent_then_rank():
    """Every edge tied: the order is breadth-first, parents by slot, children by rank."""
    P, K, N = 3, 3, 30
    edge = np.full((1, P, K, K), np.float32(-math.log(K)), np.float32)
    tok = np.arange(P * K, dtype=np.int32).reshape(1, P, K)
    tree = oracle.build_tree_cond(edge, tok, np.zeros(1, np.int32), N)
    bfs = [()]
    for d in range(1, P + 1):
        bfs += list(itertools.product(range(K), repeat=d))
    n = int(tree["n_nodes"][0])
    paths = {0: ()}
    for i in range(1, n):
        paths[i] = paths[int(tree["parent"][0, i])] + (int(tree["rank"][0, i]),)
    assert [paths[i] for i in range(n)] == bfs[:n]


def test_minus_inf_edges_are_candidates():
    """-inf edge log-probs in conditioned rows: every finite trie node first, by descending
    path score; then the -inf ones, all tied, breadth-first over the remaining frontier in
    (parent slot, rank) order (a queue, each new node's children joining at the back)."""
    import collections
    rng = np.random.default_rng(21)
    P, K, N = 3, 4, 64
    edge, tok = _lattice_cond(rng, 2, P, K)
    edge[0, :, :, 2:] = -np.inf         # half of every row masked
    edge[1, 1, 1:, :] = -np.inf         # position 1 masked under every parent but rank 0
    tree = oracle.build_tree_cond(edge, tok, np.arange(2), N)
    for b in range(2):
        allp = _all_paths(edge[b], P, K)
        finite = sorted((x for x in allp if np.isfinite(x[1])), key=lambda x: -x[1])
        n = int(tree["n_nodes"][b])
        assert n == 1 + min(N, len(allp))
        paths = {0: ()}
        for i in range(1, n):
            paths[i] = paths[int(tree["parent"][b, i])] + (int(tree["rank"][b, i]),)
        got = [paths[i] for i in range(1, n)]
        m = min(N, len(finite))
        assert got[:m] == [p for p, _ in finite[:m]]
        slot_path = {i: paths[i] for i in range(m + 1)}
        inserted = set(slot_path.values())
        queue = collections.deque(sorted((sl, r) for sl, path in slot_path.items() if len(path) < P
                                         for r in range(K) if path + (r,) not in inserted))
        expect = []
        while len(expect) < N - m and queue:
            sl, r = queue.popleft()
            path = slot_path[sl] + (r,)
            slot_path[m + 1 + len(expect)] = path
            if len(path) < P:
                queue.extend((m + 1 + len(expect), rr) for rr in range(K))
            expect.append(path)
        assert got[m:] == expect
