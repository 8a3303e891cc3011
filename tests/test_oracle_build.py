"""Pins for the oracle's best-first tree build (CPU only).

Each check is fixed by the definition of best-first construction over a drafter lattice
(SpecPilot summary, Prerequisites > draft-tree verification; Technical novelty) or by
combinatorics, never by re-running the oracle's own code path.
"""
import collections
import itertools
import math

import numpy as np
import pytest

import oracle


def _lattice(rng, B, P, K, distinct=True):
    logits = rng.normal(0, 2, size=(B, P, K))
    logp = logits - np.log(np.exp(logits).sum(-1, keepdims=True))
    logp = -np.sort(-logp, axis=-1)
    tok = np.stack([np.stack([rng.permutation(1000)[:K] for _ in range(P)]) for _ in range(B)])
    return logp.astype(np.float32), tok.astype(np.int32)


def _all_trie_nodes(logp_b, P, K):
    """Every trie node as (rank path, fp64 score summed root to leaf)."""
    nodes = []
    for d in range(1, P + 1):
        for path in itertools.product(range(K), repeat=d):
            s = 0.0
            for pos, r in enumerate(path):
                s = s + float(np.float64(logp_b[pos, r]))
            nodes.append((path, s))
    return nodes


def _rank_paths(tree, b):
    n = int(tree["n_nodes"][b])
    paths = {0: ()}
    for i in range(1, n):
        paths[i] = paths[int(tree["parent"][b, i])] + (int(tree["rank"][b, i]),)
    return [paths[i] for i in range(n)]


@pytest.mark.parametrize("P,K,N", [(1, 4, 3), (2, 3, 5), (3, 3, 20), (4, 4, 64), (4, 2, 30), (3, 4, 17)])
def test_brute_force_top_n(P, K, N):
    """With continuous random scores (no ties a.s.) the best-first tree is the top-N trie
    nodes by score, inserted in descending score order."""
    rng = np.random.default_rng(P * 100 + K * 10 + N)
    logp, tok = _lattice(rng, 3, P, K)
    tree = oracle.build_tree(logp, tok, np.arange(3), N)
    for b in range(3):
        allnodes = sorted(_all_trie_nodes(logp[b], P, K), key=lambda x: -x[1])
        expect = allnodes[:N]
        got = _rank_paths(tree, b)[1:]
        assert got == [p for p, _ in expect]
        np.testing.assert_array_equal(tree["score"][b, 1:len(got) + 1], [s for _, s in expect])


@pytest.mark.parametrize("P,K,N", [(3, 3, 20), (2, 4, 20), (4, 2, 30), (3, 2, 14)])
def test_uniform_lattice_is_bfs(P, K, N):
    """All candidates equally likely: every tie is broken by (parent index, rank), which
    yields the breadth-first order of the K-ary trie (depth-major, lexicographic)."""
    logp = np.full((1, P, K), -math.log(K), np.float32)
    tok = np.arange(P * K, dtype=np.int32).reshape(1, P, K)
    tree = oracle.build_tree(logp, tok, np.array([7]), N)
    bfs = [p for d in range(1, P + 1) for p in itertools.product(range(K), repeat=d)]
    expect = bfs[:N]
    assert _rank_paths(tree, 0)[1:] == expect


def test_k1_is_chain():
    rng = np.random.default_rng(1)
    for P, N in [(8, 4), (8, 8), (8, 24), (16, 64)]:
        logp = np.zeros((1, P, 1), np.float32)
        tok = rng.integers(0, 100, size=(1, P, 1)).astype(np.int32)
        tree = oracle.build_tree(logp, tok, np.array([5]), N)
        n = min(N, P)
        assert tree["n_nodes"][0] == n + 1
        np.testing.assert_array_equal(tree["parent"][0, 1:n + 1], np.arange(n))
        np.testing.assert_array_equal(tree["depth"][0, :n + 1], np.arange(n + 1))
        np.testing.assert_array_equal(tree["token"][0, 1:n + 1], tok[0, :n, 0])


def test_dominant_top1_is_greedy_chain():
    """A peaked lattice with N <= P gives the stock greedy chain of rank-0 candidates."""
    rng = np.random.default_rng(2)
    P, K, N = 8, 16, 8
    logits = rng.normal(0, 1, size=(1, P, K))
    logits[..., 0] += 30.0
    logp = logits - np.log(np.exp(logits).sum(-1, keepdims=True))
    order = np.argsort(-logp, axis=-1)
    logp = np.take_along_axis(logp, order, -1).astype(np.float32)
    tok = rng.integers(0, 1000, size=(1, P, K)).astype(np.int32)
    tree = oracle.build_tree(logp, tok, np.array([0]), N)
    np.testing.assert_array_equal(tree["parent"][0, 1:], np.arange(N))
    np.testing.assert_array_equal(tree["rank"][0, 1:], 0)


@pytest.mark.parametrize("P,K,N", [(2, 2, 10), (1, 3, 8), (3, 2, 64), (2, 3, 12)])
def test_exhausted_trie(P, K, N):
    rng = np.random.default_rng(3)
    logp, tok = _lattice(rng, 2, P, K)
    tree = oracle.build_tree(logp, tok, np.array([1, 2]), N)
    size = sum(K ** d for d in range(1, P + 1))
    assert (tree["n_nodes"] == min(N, size) + 1).all()


def test_invariants_on_config_shaped_lattices():
    """Prefix closure, parent < child, depth/token/score/ancestor consistency and
    non-increasing scores (log-probs are <= 0) on 8x16 and 16x16 lattices."""
    rng = np.random.default_rng(4)
    for P, K, N in [(8, 16, 24), (16, 16, 64), (4, 4, 8)]:
        logp, tok = _lattice(rng, 4, P, K)
        tree = oracle.build_tree(logp, tok, np.arange(4), N)
        for b in range(4):
            n = int(tree["n_nodes"][b])
            assert n == N + 1
            assert tree["parent"][b, 0] == -1 and tree["depth"][b, 0] == 0 and tree["anc"][b, 0] == 0
            for i in range(1, n):
                p = int(tree["parent"][b, i])
                d = int(tree["depth"][b, i])
                r = int(tree["rank"][b, i])
                assert 0 <= p < i
                assert d == tree["depth"][b, p] + 1 and 1 <= d <= P
                assert 0 <= r < K
                assert tree["token"][b, i] == tok[b, d - 1, r]
                assert tree["score"][b, i] == tree["score"][b, p] + np.float64(logp[b, d - 1, r])
                assert int(tree["anc"][b, i]) == int(tree["anc"][b, p]) | (1 << (i - 1))
                assert tree["score"][b, i] <= tree["score"][b, i - 1] or i == 1
            # each (parent, rank) appears at most once; siblings appear in rank order
            pairs = [(int(tree["parent"][b, i]), int(tree["rank"][b, i])) for i in range(1, n)]
            assert len(set(pairs)) == len(pairs)
            for p in set(x for x, _ in pairs):
                ranks = [r for x, r in pairs if x == p]
                assert ranks == list(range(len(ranks)))


def _lazy_build(logp_b, N):
    """Best-first with a lazy frontier (each inserted node offers only its lowest-rank
    un-inserted child), the form the GPU kernel uses; valid when ranks are sorted."""
    P, K = logp_b.shape
    score, depth, nxt = [0.0], [0], [0]
    order = []
    while len(order) < N:
        best = None
        for p in range(len(score)):
            if depth[p] < P and nxt[p] < K:
                s = score[p] + float(np.float64(logp_b[depth[p], nxt[p]]))
                if best is None or s > best[0]:
                    best = (s, p)
        if best is None:
            break
        s, p = best
        order.append((p, nxt[p]))
        nxt[p] += 1
        score.append(s)
        depth.append(depth[p] + 1)
        nxt.append(0)
    return order


@pytest.mark.parametrize("seed", range(6))
def test_lazy_frontier_equals_full_frontier(seed):
    rng = np.random.default_rng(seed)
    P, K, N = [(8, 16, 24), (16, 16, 64), (4, 4, 8), (3, 3, 30), (2, 5, 64), (16, 2, 64)][seed]
    logp, tok = _lattice(rng, 2, P, K)
    if seed == 3:
        logp[:] = np.float32(-math.log(K))          # all ties
    tree = oracle.build_tree(logp, tok, np.arange(2), N)
    for b in range(2):
        n = int(tree["n_nodes"][b])
        full = [(int(tree["parent"][b, i]), int(tree["rank"][b, i])) for i in range(1, n)]
        assert _lazy_build(logp[b], N) == full


def test_minus_inf_log_probs_are_candidates():
    """-inf log-probs (masked candidates) are candidates like any other: every finite trie
    node comes first, in descending score order; then the -inf ones, all tied, in the tie order
    (smaller parent slot, then smaller rank), which is breadth-first over the remaining
    frontier: a queue, each new node's children joining at the back.  The tree is as large as
    the budget or the trie allows."""
    rng = np.random.default_rng(77)
    P, K, N = 3, 4, 64                  # a trie of 84 nodes
    logp, tok = _lattice(rng, 3, P, K)
    logp[0, :, 2:] = -np.inf            # half of every position masked
    logp[1, 1, 1:] = -np.inf            # position 1 masked but for rank 0
    # finite log-probs whose sums fall below -FLT_MAX (-inf once rounded to fp32)
    logp[2] = -np.sort(rng.uniform(1e38, 3.4e38, size=(P, K)), axis=-1).astype(np.float32)
    tree = oracle.build_tree(logp, tok, np.arange(3), N)
    for b in range(3):
        allnodes = _all_trie_nodes(logp[b], P, K)
        finite = sorted((x for x in allnodes if np.isfinite(x[1])), key=lambda x: -x[1])
        got = _rank_paths(tree, b)[1:]
        assert int(tree["n_nodes"][b]) == 1 + min(N, len(allnodes))
        m = min(N, len(finite))
        assert got[:m] == [p for p, _ in finite[:m]]
        slot_path = {0: ()}
        for i, path in enumerate(got[:m]):
            slot_path[i + 1] = path
        inserted = set(slot_path.values())
        queue = collections.deque(sorted((sl, r) for sl, path in slot_path.items() if len(path) < P
                                         for r in range(K) if path + (r,) not in inserted))
        expect = []
        while len(expect) < N - m and queue:
            sl, r = queue.popleft()
            path = slot_path[sl] + (r,)
            slot = m + 1 + len(expect)
            expect.append(path)
            slot_path[slot] = path
            if len(path) < P:
                queue.extend((slot, rr) for rr in range(K))
        assert got[m:] == expect
        sc = tree["score"][b, 1:len(got) + 1]
        assert np.all(np.isfinite(sc[:m])) and np.all(sc[m:] == -np.inf)
        assert np.all(np.diff(sc[:m]) <= 0)
