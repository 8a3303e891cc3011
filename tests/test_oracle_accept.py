"""Pins for the oracle's greedy acceptance (CPU only).

Acceptance takes the longest root path whose draft tokens equal the target argmax at
their parents, plus one bonus token; tau is in [1, depth + 1] (SpecPilot summary,
Prerequisites > speculative decoding and > draft-tree verification).
"""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, generate, resolve_target
from workloads.generate import target_probs


def _tree_from_parents(parent, token):
    n = len(parent)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    return {"parent": np.array([parent]), "token": np.array([token]), "n_nodes": np.array([n]),
            "depth": np.array([depth])}


def _brute_force(tree, target):
    """Enumerate every root path; keep those whose every edge matches; the accepted path
    is the deepest (unique when sibling tokens are distinct)."""
    n = int(tree["n_nodes"][0])
    par, tok = tree["parent"][0], tree["token"][0]
    best = [0]
    for i in range(n):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = par[j]
        path = path[::-1]
        if all(tok[c] == target[par[c]] for c in path[1:]) and len(path) > len(best):
            best = path
    return best


def test_against_brute_force_on_random_trees():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(1, 30))
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        # sibling tokens distinct: token = 10 * (rank among siblings) + small noise-free id
        token = [-1] * n
        seen = {}
        for i in range(1, n):
            seen.setdefault(parent[i], 0)
            token[i] = 3 * seen[parent[i]] + int(rng.integers(0, 3))
            seen[parent[i]] += 1
        tree = _tree_from_parents(parent, token)
        target = rng.integers(0, 12, size=(1, n))
        acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=n)
        best = _brute_force(tree, target[0])
        assert acc_len[0] == len(best)
        assert list(acc_node[0, :len(best)]) == best
        assert list(acc_tok[0, :len(best) - 1]) == [token[c] for c in best[1:]]
        assert acc_tok[0, len(best) - 1] == target[0, best[-1]]
        depth = tree["depth"][0]
        assert 1 <= acc_len[0] <= depth.max() + 1


def test_all_match_and_no_match():
    parent = [-1, 0, 1, 2, 3, 0, 5, 1]
    token = [-1, 10, 11, 12, 13, 20, 21, 30]
    tree = _tree_from_parents(parent, token)
    # target equals the chain 0->1->2->3->4 everywhere: tau = 5, bonus = target[4]
    target = np.array([[10, 11, 12, 13, 99, 0, 0, 0]])
    acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=4)
    assert acc_len[0] == 5
    assert list(acc_tok[0]) == [10, 11, 12, 13, 99]
    assert list(acc_node[0]) == [0, 1, 2, 3, 4]
    # no draft matches: tau = 1, the bonus is the root's target
    target = np.array([[55, 11, 12, 13, 99, 0, 0, 0]])
    acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=4)
    assert acc_len[0] == 1
    assert list(acc_tok[0]) == [55, -1, -1, -1, -1]
    assert list(acc_node[0]) == [0, -1, -1, -1, -1]
    # branch switch: root target 20 picks slot 5, then slot 6
    target = np.array([[20, 11, 12, 13, 99, 21, 7, 0]])
    acc_len, acc_tok, acc_node = oracle.accept(tree, target, P=4)
    assert acc_len[0] == 3 and list(acc_node[0, :3]) == [0, 5, 6] and list(acc_tok[0, :3]) == [20, 21, 7]


def test_lowest_index_on_duplicate_sibling_tokens():
    parent = [-1, 0, 0, 2]
    token = [-1, 5, 5, 6]
    tree = _tree_from_parents(parent, token)
    acc_len, _, acc_node = oracle.accept(tree, np.array([[5, 6, 6, 1]]), P=3)
    assert acc_len[0] == 2 and list(acc_node[0, :2]) == [0, 1]


@pytest.mark.parametrize("cfg_name", ["tiny", "one_layer"])
def test_expected_tau_closed_form(cfg_name):
    """Target choices are i.i.d. per slot, so the probability that the accepted path passes
    through node n is the product over its edges of P(target at the parent = token of the
    child) = p(rank of child) + p(uniform) / V.  Hence
    E[tau] = 1 + sum over draft nodes of that product; the sample mean over many draws must
    agree within 4 standard errors."""
    cfg = CONFIGS[cfg_name]
    w = generate(cfg, seed=0)
    tree = oracle.build_tree(w.lat_logp, w.lat_tok, w.root_tok, cfg.N)
    probs = target_probs(cfg, cfg.p_top1)
    n = int(tree["n_nodes"][0])
    reach = np.ones(n)
    for i in range(1, n):
        edge = probs[int(tree["rank"][0, i])] + probs[cfg.K] / cfg.V
        reach[i] = reach[int(tree["parent"][0, i])] * edge
    expect = 1.0 + reach[1:].sum()
    rng = np.random.default_rng(123)
    draws = 4000
    cdf = np.cumsum(probs)
    cdf[-1] = 1.0
    taus = np.empty(draws)
    for t in range(draws):
        choice = np.searchsorted(cdf, rng.random(size=(1, n)), side="right").clip(0, cfg.K).astype(np.int32)
        uni = rng.integers(0, cfg.V, size=(1, n)).astype(np.int32)
        target = resolve_target(tree["depth"], tree["n_nodes"], w.lat_tok, choice, uni)
        taus[t] = oracle.accept(tree, target, cfg.P)[0][0]
    se = taus.std(ddof=1) / np.sqrt(draws)
    assert abs(taus.mean() - expect) < 4 * se, (taus.mean(), expect, se)
