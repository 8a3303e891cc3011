"""Property-based pins for the oracle on small random shapes (CPU only, hypothesis).

Each property is fixed by a definition or by mathematics, not by the oracle's own code:
  * best-first construction (SpecPilot summary, Prerequisites > draft-tree verification;
    Technical novelty): the tree is closed under parents, pops come in non-increasing
    score order, no unused child of an inserted node beats the last pop, and with
    distinct scores the tree is exactly the top-N trie nodes by score;
  * greedy acceptance (same page, Prerequisites > speculative decoding and > draft-tree
    verification): the accepted path matches the target on every edge, cannot be
    extended, takes the smallest matching slot at every step, and with distinct sibling
    tokens is the deepest matching root path found by enumeration;
  * the shared node budget (same page, Technical novelty, batching): the batch holds its
    first G trie nodes by score, each request capped at N and at its own positions;
  * the gated delta rule along the tree (same page, Prerequisites > hybrid recurrent
    architecture): a node's output equals the WY / UT closed form solved with a library
    linear solve, the tree verify of a node equals the chain verify over its root path
    rows, and the commit equals the verify state of the deepest accepted node.
"""
import itertools

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

from .test_oracle_accept import _brute_force, _tree_from_parents
from .test_oracle_build import _all_trie_nodes, _lattice, _rank_paths
from .test_oracle_verify import _data, _path, _random_tree, _wy_outputs

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


def _trie_size(P, K):
    return sum(K ** d for d in range(1, P + 1))


# --------------------------------------------------------------------------------------
# best-first build
# --------------------------------------------------------------------------------------
@SETTINGS
@given(P=st.integers(1, 4), K=st.integers(2, 4), N=st.integers(1, 40), seed=st.integers(0, 2**31 - 1))
def test_build_is_top_n_with_distinct_scores(P, K, N, seed):
    """K >= 2 so that every log-prob is strictly negative and no two trie nodes tie."""
    rng = np.random.default_rng(seed)
    logp, tok = _lattice(rng, 1, P, K)
    tree = oracle.build_tree(logp, tok, np.array([3]), N)
    ranked = sorted(_all_trie_nodes(logp[0], P, K), key=lambda x: -x[1])
    expect = ranked[:N]
    got = _rank_paths(tree, 0)[1:]
    assert int(tree["n_nodes"][0]) == 1 + min(N, _trie_size(P, K))
    assert got == [p for p, _ in expect]


@SETTINGS
@given(P=st.integers(1, 4), K=st.integers(1, 4), N=st.integers(1, 40), seed=st.integers(0, 2**31 - 1),
       levels=st.integers(1, 4))
def test_build_invariants_with_ties(P, K, N, seed, levels):
    """Log-probs drawn from a few quantised levels so that many paths tie."""
    rng = np.random.default_rng(seed)
    logp = -0.5 * rng.integers(0, levels, size=(1, P, K)).astype(np.float32)
    tok = rng.integers(0, 50, size=(1, P, K)).astype(np.int32)
    tree = oracle.build_tree(logp, tok, np.array([11]), N)
    n = int(tree["n_nodes"][0])
    assert n == 1 + min(N, _trie_size(P, K))
    par, dep, rank = tree["parent"][0], tree["depth"][0], tree["rank"][0]
    score, token, anc = tree["score"][0], tree["token"][0], tree["anc"][0]
    assert par[0] == -1 and dep[0] == 0 and token[0] == 11 and score[0] == 0.0
    used = {0: set()}
    for i in range(1, n):
        p = int(par[i])
        assert 0 <= p < i                                   # closed under parents
        assert dep[i] == dep[p] + 1 and 1 <= dep[i] <= P
        assert token[i] == tok[0, dep[i] - 1, rank[i]]
        assert score[i] == score[p] + float(np.float64(logp[0, dep[i] - 1, rank[i]]))
        assert rank[i] not in used[p]                       # each child inserted once
        used[p].add(int(rank[i]))
        used[i] = set()
        assert int(anc[i]) == int(anc[p]) | (1 << (i - 1))
        if i >= 2:
            assert score[i] <= score[i - 1]                 # pops never increase
    # no child left out of the tree beats the last node in
    if n - 1 == N:
        last = score[n - 1]
        for i in range(n):
            if dep[i] < P:
                for r in range(K):
                    if r not in used[i]:
                        assert score[i] + float(np.float64(logp[0, dep[i], r])) <= last


# --------------------------------------------------------------------------------------
# greedy acceptance
# --------------------------------------------------------------------------------------
@st.composite
def _tree_and_target(draw, distinct_siblings):
    n = draw(st.integers(1, 30))
    parent = [-1] + [draw(st.integers(0, i - 1)) for i in range(1, n)]
    vocab = draw(st.integers(2, 6))
    token = [-1]
    kids = {}
    for i in range(1, n):
        p = parent[i]
        if distinct_siblings:
            t = vocab * len(kids.get(p, [])) + draw(st.integers(0, vocab - 1))
        else:
            t = draw(st.integers(0, vocab - 1))
        kids.setdefault(p, []).append(i)
        token.append(t)
    target = [draw(st.integers(0, 3 * vocab)) for _ in range(n)]
    return parent, token, np.array([target])


@SETTINGS
@given(data=_tree_and_target(distinct_siblings=True))
def test_accept_is_deepest_matching_path(data):
    parent, token, target = data
    tree = _tree_from_parents(parent, token)
    acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=len(parent))
    best = _brute_force(tree, target[0])
    assert acc_len[0] == len(best)
    assert list(acc_node[0, :len(best)]) == best
    assert list(acc_tok[0, :len(best)]) == [token[c] for c in best[1:]] + [target[0, best[-1]]]
    assert (acc_node[0, len(best):] == -1).all() and (acc_tok[0, len(best):] == -1).all()


@SETTINGS
@given(data=_tree_and_target(distinct_siblings=False))
def test_accept_greedy_walk_with_duplicate_tokens(data):
    parent, token, target = data
    n = len(parent)
    tree = _tree_from_parents(parent, token)
    acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=n)
    path = [int(x) for x in acc_node[0, :int(acc_len[0])]]
    assert path[0] == 0 and 1 <= len(path) <= max(tree["depth"][0]) + 1
    for a, c in zip(path, path[1:]):
        matching = [x for x in range(1, n) if parent[x] == a and token[x] == target[0, a]]
        assert matching and c == min(matching)             # smallest matching slot
    u = path[-1]
    assert not any(parent[x] == u and token[x] == target[0, u] for x in range(1, n))
    assert acc_tok[0, len(path) - 1] == target[0, u]       # bonus token


# --------------------------------------------------------------------------------------
# gated delta rule along the tree, and the commit
# --------------------------------------------------------------------------------------
@SETTINGS
@given(n=st.integers(1, 24), d=st.integers(1, 9), max_depth=st.integers(1, 12),
       seed=st.integers(0, 2**31 - 1))
def test_verify_equals_wy_closed_form(n, d, max_depth, seed):
    rng = np.random.default_rng(seed)
    parent, _ = _random_tree(rng, n, max_depth=max_depth)
    q, k, v, alpha, beta, h0 = _data(rng, n, 1, d, d)
    _, o = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    o_wy = _wy_outputs(parent, q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], h0[0])
    np.testing.assert_allclose(o[:, 0], o_wy, rtol=1e-9, atol=1e-10)


@SETTINGS
@given(n=st.integers(1, 20), H=st.integers(1, 3), dk=st.integers(1, 6), dv=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1))
def test_tree_node_equals_chain_over_its_path(n, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, beta, h0 = _data(rng, n, H, dk, dv)
    st_t, o_t = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    i = int(rng.integers(0, n))
    rows = _path(parent, i)
    m = len(rows)
    st_c, o_c = oracle.verify_request(np.arange(-1, m - 1), m, q[rows], k[rows], v[rows],
                                      alpha[rows], beta[rows], h0)
    np.testing.assert_allclose(st_t[i], st_c[-1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o_t[i], o_c[-1], rtol=1e-12, atol=1e-13)


@SETTINGS
@given(L=st.integers(1, 2), B=st.integers(1, 3), n=st.integers(1, 12), H=st.integers(1, 2),
       d=st.integers(1, 5), seed=st.integers(0, 2**31 - 1))
def test_commit_is_state_of_deepest_accepted(L, B, n, H, d, seed):
    rng = np.random.default_rng(seed)
    parents = [_random_tree(rng, n)[0] for _ in range(B)]
    tree = {"parent": np.stack(parents), "n_nodes": np.full(B, n)}
    q, k, v, alpha, beta, h0s = zip(*[_data(rng, n, H, d, d) for _ in range(L * B)])
    shape = lambda xs: np.stack(xs).reshape((L, B) + xs[0].shape)
    q, k, v, alpha, beta, h0 = map(shape, (q, k, v, alpha, beta, h0s))
    deepest = rng.integers(0, n, size=B)
    acc_node = np.full((B, n + 1), -1)
    acc_len = np.zeros(B, int)
    for b in range(B):
        p = _path(parents[b], int(deepest[b]))
        acc_node[b, :len(p)] = p
        acc_len[b] = len(p)
    _, hnorm, kept = oracle.verify(tree, q, k, v, alpha, beta, h0, keep_states_of=deepest)
    new = oracle.commit(acc_node, acc_len, k, v, alpha, beta, h0)
    np.testing.assert_allclose(new, kept, rtol=1e-12, atol=1e-13)
    for l, b in itertools.product(range(L), range(B)):
        np.testing.assert_allclose(np.sqrt((new[l, b] ** 2).sum(axis=(-2, -1))),
                                   hnorm[l, b, int(deepest[b])], rtol=1e-12)


# --------------------------------------------------------------------------------------
# batch-wide best-first build under a shared budget
# --------------------------------------------------------------------------------------
@SETTINGS
@given(B=st.integers(1, 5), P=st.integers(1, 3), K=st.integers(2, 4), N=st.integers(1, 20),
       G=st.integers(0, 60), seed=st.integers(0, 2**31 - 1), data=st.data())
def test_shared_build_is_top_g_of_the_batch(B, P, K, N, G, seed, data):
    """Distinct scores: the batch's trees hold exactly its first G trie nodes in descending
    score order (a request stops at N), each request in its own insertion order."""
    positions = data.draw(st.lists(st.integers(0, P), min_size=B, max_size=B))
    rng = np.random.default_rng(seed)
    logp, tok = _lattice(rng, B, P, K)
    every = []
    for b in range(B):
        for path, s in _all_trie_nodes(logp[b], positions[b], K):
            every.append((s, b, path))
    every.sort(key=lambda x: -x[0])
    got_b = [[] for _ in range(B)]
    total = 0
    for s, b, path in every:
        if total == G:
            break
        if len(got_b[b]) < N:
            got_b[b].append(path)
            total += 1
    tree = oracle.build_tree_shared(logp, tok, np.arange(B), N, G, positions)
    for b in range(B):
        assert _rank_paths(tree, b)[1:] == got_b[b]
