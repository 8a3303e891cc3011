"""Pins for the oracle's batch-wide best-first build under a shared node budget (CPU only).

SpecPilot summary, Technical novelty (batching: one node budget shared by the batch, and a
number of draft positions chosen per request).  Each check is fixed by the definition of a
best-first pass over the union of the requests' frontiers, or by combinatorics: brute force
over whole tiny tries, the breadth-first order of a uniform lattice, the per-request special
cases, and the budget arithmetic.
"""
import itertools
import math

import numpy as np
import pytest

import oracle

from .test_oracle_build import _lattice, _rank_paths


def _trie(logp_b, depth_cap, K):
    """Every node of one request's trie up to depth_cap: (rank path, fp64 root-to-leaf score)."""
    nodes = []
    for d in range(1, depth_cap + 1):
        for path in itertools.product(range(K), repeat=d):
            s = 0.0
            for pos, r in enumerate(path):
                s = s + float(np.float64(logp_b[pos, r]))
            nodes.append((path, s))
    return nodes


def _greedy_take(ordered, B, N, G):
    """Walk (request, path) items in pop order, keeping at most N per request and G in all."""
    got = [[] for _ in range(B)]
    total = 0
    for b, path in ordered:
        if total == G:
            break
        if len(got[b]) < N:
            got[b].append(path)
            total += 1
    return got


@pytest.mark.parametrize("B,P,K,N,G,positions", [
    (3, 3, 3, 8, 10, [3, 2, 1]),
    (4, 4, 2, 6, 13, [4, 4, 2, 3]),
    (2, 3, 4, 20, 25, None),
    (5, 2, 3, 4, 40, [2, 1, 2, 0, 2]),
    (3, 4, 3, 64, 7, None),
])
def test_brute_force_shared_top_g(B, P, K, N, G, positions):
    """Distinct scores (K >= 2, continuous draws): the batch takes its trie nodes in
    descending score order, skipping a request once it holds N, until G are taken; each
    request inserts its own nodes in that order."""
    rng = np.random.default_rng(B * 1000 + P * 100 + K * 10 + G)
    logp, tok = _lattice(rng, B, P, K)
    caps = [P] * B if positions is None else positions
    every = [(s, b, path) for b in range(B) for path, s in _trie(logp[b], caps[b], K)]
    every.sort(key=lambda x: -x[0])
    expect = _greedy_take([(b, path) for _, b, path in every], B, N, G)
    tree = oracle.build_tree_shared(logp, tok, np.arange(B), N, G, positions)
    for b in range(B):
        assert _rank_paths(tree, b)[1:] == expect[b]
        assert int(tree["n_nodes"][b]) == 1 + len(expect[b])


@pytest.mark.parametrize("B,P,K,N,G", [(3, 3, 2, 10, 11), (2, 2, 3, 12, 9), (4, 3, 2, 3, 12),
                                       (3, 2, 2, 6, 100)])
def test_uniform_lattice_is_depth_then_request_then_bfs(B, P, K, N, G):
    """All candidates equally likely: scores depend on depth only, so the pass takes depth 1
    of request 0, of request 1, ..., then depth 2 of each request in turn, each depth in
    breadth-first (lexicographic) order: this pins the cross-request tie rule."""
    logp = np.full((B, P, K), -math.log(K), np.float32)
    tok = np.tile(np.arange(P * K, dtype=np.int32).reshape(1, P, K), (B, 1, 1))
    order = [(b, path) for d in range(1, P + 1) for b in range(B)
             for path in itertools.product(range(K), repeat=d)]
    expect = _greedy_take(order, B, N, G)
    tree = oracle.build_tree_shared(logp, tok, np.arange(B), N, G)
    for b in range(B):
        assert _rank_paths(tree, b)[1:] == expect[b]


@pytest.mark.parametrize("seed", range(3))
def test_unbounded_budget_is_independent_builds(seed):
    """With a budget no batch can reach, every request gets its own best-first tree of N
    drafts over its own positions."""
    rng = np.random.default_rng(40 + seed)
    B, P, K, N = 4, 5, 4, 30
    logp, tok = _lattice(rng, B, P, K)
    positions = [5, 3, 2, 4]
    shared = oracle.build_tree_shared(logp, tok, np.arange(B), N, 10 ** 6, positions)
    for b in range(B):
        own = oracle.build_tree(logp[b:b + 1, :positions[b]], tok[b:b + 1, :positions[b]],
                                np.array([b]), N)
        n = int(own["n_nodes"][0])
        assert int(shared["n_nodes"][b]) == n
        for name in ("parent", "depth", "rank", "token", "score", "anc"):
            np.testing.assert_array_equal(shared[name][b, :n], own[name][0, :n])


@pytest.mark.parametrize("seed", range(4))
def test_each_request_is_a_best_first_prefix(seed):
    """Whatever the budget leaves a request, its tree is that request's own best-first tree
    of that size; the batch holds min(G, what the requests can hold) drafts; and no
    candidate left to a request that is not full beats the last node the batch took."""
    rng = np.random.default_rng(60 + seed)
    B, P, K, N = 6, 6, 5, 24
    logp, tok = _lattice(rng, B, P, K)
    positions = rng.integers(1, P + 1, size=B)
    G = int(rng.integers(10, 80))
    tree = oracle.build_tree_shared(logp, tok, np.arange(B), N, G, positions)
    n = tree["n_nodes"].astype(int)
    room = [min(N, sum(K ** d for d in range(1, int(positions[b]) + 1))) for b in range(B)]
    assert (n - 1).sum() == min(G, sum(room))
    last = min(tree["score"][b, n[b] - 1] for b in range(B) if n[b] > 1)
    for b in range(B):
        own = oracle.build_tree(logp[b:b + 1, :positions[b]], tok[b:b + 1, :positions[b]],
                                np.array([b]), n[b] - 1)
        for name in ("parent", "depth", "rank", "token", "score", "anc"):
            np.testing.assert_array_equal(tree[name][b, :n[b]], own[name][0, :n[b]])
        if n[b] - 1 < room[b]:
            used = {(int(tree["parent"][b, i]), int(tree["rank"][b, i])) for i in range(1, n[b])}
            for i in range(n[b]):
                d = int(tree["depth"][b, i])
                if d >= positions[b]:
                    continue
                for r in range(K):
                    if (i, r) not in used:
                        assert tree["score"][b, i] + float(np.float64(logp[b, d, r])) <= last


def test_degenerate_budgets():
    rng = np.random.default_rng(3)
    logp, tok = _lattice(rng, 3, 3, 3)
    t0 = oracle.build_tree_shared(logp, tok, np.array([5, 6, 7]), 8, 0)
    np.testing.assert_array_equal(t0["n_nodes"], [1, 1, 1])
    np.testing.assert_array_equal(t0["token"][:, 0], [5, 6, 7])
    t1 = oracle.build_tree_shared(logp, tok, np.array([5, 6, 7]), 8, 5, positions=[0, 0, 3])
    np.testing.assert_array_equal(t1["n_nodes"], [1, 1, 6])
    t2 = oracle.build_tree_shared(logp, tok, np.array([5, 6, 7]), 0, 5)
    np.testing.assert_array_equal(t2["n_nodes"], [1, 1, 1])
