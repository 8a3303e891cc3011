"""Pins for the oracle's gated-delta-rule tree verify and commit (CPU only).

The recurrence is h = alpha (I - beta k k^T) h_parent + beta k v^T, o = h^T q (SpecPilot
summary, Prerequisites > hybrid recurrent architecture).  Each test fixes the oracle
against something other than its own code: closed forms of special cases, an
explicit-matrix composition of affine maps, the WY / UT-transform closed form solved with
a library linear solver, and invariances of the update.
"""
import numpy as np
import pytest

import oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _random_tree(rng, n, max_depth=None):
    parent = [-1]
    depth = [0]
    for i in range(1, n):
        cands = [p for p in range(i) if max_depth is None or depth[p] < max_depth]
        p = int(rng.choice(cands))
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.array(parent), np.array(depth)


def _path(parent, i):
    out = []
    while i >= 0:
        out.append(i)
        i = parent[i]
    return out[::-1]


def _data(rng, n, H, dk, dv, unit_k=True):
    q = _unit(rng.normal(size=(n, H, dk)))
    k = rng.normal(size=(n, H, dk))
    k = _unit(k) if unit_k else k
    v = rng.normal(size=(n, H, dv))
    alpha = rng.uniform(0.2, 0.99, size=(n, H))
    beta = rng.uniform(0.05, 1.0, size=(n, H))
    h0 = rng.normal(0, 0.3, size=(H, dk, dv))
    return q, k, v, alpha, beta, h0


def test_hand_worked_2x2():
    """d=2 by hand: h0 = I, k = e1, v = (2, 3), alpha = 0.5, beta = 1 gives
    h = 0.5 (I - e1 e1^T) + e1 (2, 3) = [[2, 3], [0, 0.5]] and, for q = e2, o = (0, 0.5)."""
    h0 = np.eye(2)
    h, o = oracle.gdn_step(h0, np.array([0.0, 1.0]), np.array([1.0, 0.0]), np.array([2.0, 3.0]),
                           np.array(0.5), np.array(1.0))
    np.testing.assert_array_equal(h, [[2.0, 3.0], [0.0, 0.5]])
    np.testing.assert_array_equal(o, [0.0, 0.5])
    # a second step along the chain with k = e2, v = (-1, 4), alpha = 0.25, beta = 0.5:
    # h2 = 0.25 (h - 0.5 e2 (e2^T h)) + 0.5 e2 (-1, 4) = [[0.5, 0.75], [-0.5, 2.0625]]
    h2, o2 = oracle.gdn_step(h, np.array([1.0, 0.0]), np.array([0.0, 1.0]), np.array([-1.0, 4.0]),
                             np.array(0.25), np.array(0.5))
    np.testing.assert_allclose(h2, [[0.5, 0.75], [-0.5, 2.0625]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o2, [0.5, 0.75], rtol=0, atol=1e-15)


def test_readout_is_transpose_product():
    """o = h^T q: with q = e_i the output is row i of h (pins the transposition)."""
    rng = np.random.default_rng(0)
    h = rng.normal(size=(5, 7))
    for i in range(5):
        q = np.zeros(5)
        q[i] = 1.0
        np.testing.assert_array_equal(oracle.gdn_readout(h, q), h[i])


def test_identity_gates():
    """alpha = 1, beta = 0: every node's state is h0 and o_i = h0^T q_i."""
    rng = np.random.default_rng(1)
    n, H, d = 17, 3, 8
    parent, _ = _random_tree(rng, n)
    q, k, v, _, _, h0 = _data(rng, n, H, d, d)
    st, o = oracle.verify_request(parent, n, q, k, v, np.ones((n, H)), np.zeros((n, H)), h0)
    for i in range(n):
        np.testing.assert_array_equal(st[i], h0)
        np.testing.assert_allclose(o[i], np.einsum("hij,hi->hj", h0, q[i]), rtol=1e-14, atol=1e-14)


def test_decay_only():
    """beta = 0: h_i = (product of alpha along the root path of i) h0."""
    rng = np.random.default_rng(2)
    n, H, d = 21, 2, 6
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, _, h0 = _data(rng, n, H, d, d)
    st, _ = oracle.verify_request(parent, n, q, k, v, alpha, np.zeros((n, H)), h0)
    for i in range(n):
        g = np.prod(alpha[_path(parent, i)], axis=0)
        np.testing.assert_allclose(st[i], g[:, None, None] * h0, rtol=1e-13, atol=1e-15)


def test_beta_one_replaces_key_direction():
    """beta = 1 with unit k: k_i^T h_i = v_i^T exactly (up to rounding), whatever alpha;
    for x orthogonal to k_i, x^T h_i = alpha_i x^T h_parent."""
    rng = np.random.default_rng(3)
    n, H, d = 15, 2, 8
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, _, h0 = _data(rng, n, H, d, d)
    st, _ = oracle.verify_request(parent, n, q, k, v, alpha, np.ones((n, H)), h0)
    for i in range(n):
        hp = h0 if i == 0 else st[parent[i]]
        for h in range(H):
            np.testing.assert_allclose(k[i, h] @ st[i, h], v[i, h], rtol=1e-12, atol=1e-12)
            x = rng.normal(size=d)
            x -= (x @ k[i, h]) * k[i, h]
            np.testing.assert_allclose(x @ st[i, h], alpha[i, h] * (x @ hp[h]), rtol=1e-11, atol=1e-12)


def test_orthonormal_chain_closed_form():
    """alpha = beta = 1 along a chain with orthonormal keys: the k-directions are replaced
    and the rest kept, h_m = (I - sum k k^T) h0 + sum k v^T."""
    rng = np.random.default_rng(4)
    d, m = 10, 6
    Qm, _ = np.linalg.qr(rng.normal(size=(d, d)))
    keys = Qm[:, :m].T
    v = rng.normal(size=(m, d))
    h0 = rng.normal(size=(d, d))
    parent = np.arange(-1, m - 1)
    st, _ = oracle.verify_request(parent, m, _unit(rng.normal(size=(m, 1, d))), keys[:, None, :],
                                  v[:, None, :], np.ones((m, 1)), np.ones((m, 1)), h0[None])
    expect = (np.eye(d) - keys.T @ keys) @ h0 + keys.T @ v
    np.testing.assert_allclose(st[-1, 0], expect, rtol=1e-12, atol=1e-12)


def test_affine_map_composition_brute_force():
    """Each node's state equals the composition, along its root path, of the affine maps
    h -> A_s h + b_s with A_s = alpha_s (I - beta_s k_s k_s^T) and b_s = beta_s k_s v_s^T,
    evaluated with explicit d x d matrices (independent of traversal order)."""
    rng = np.random.default_rng(5)
    n, H, d = 40, 2, 7
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, beta, h0 = _data(rng, n, H, d, d, unit_k=False)
    st, o = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    for i in range(n):
        for h in range(H):
            M = np.eye(d)
            c = np.zeros((d, d))
            for s in _path(parent, i):
                A = alpha[s, h] * (np.eye(d) - beta[s, h] * np.outer(k[s, h], k[s, h]))
                M = A @ M
                c = A @ c + beta[s, h] * np.outer(k[s, h], v[s, h])
            hs = M @ h0[h] + c
            np.testing.assert_allclose(st[i, h], hs, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(o[i, h], hs.T @ q[i, h], rtol=1e-11, atol=1e-12)


def _wy_outputs(parent, q, k, v, alpha, beta, h0):
    """Tree form of the WY / UT-transform closed form, solved with numpy.linalg.solve.

    With gamma_t the product of alpha over the root path of t and A[t, s] the ancestor
    indicator, the pseudo-values U solve (I + Lm) U = diag(beta) (V - diag(gamma) K h0)
    where Lm[t, s] = beta_t (gamma_t / gamma_s) k_t.k_s for strict ancestors s, and
    o_t = gamma_t h0^T q_t + sum over s ancestor-or-self of (gamma_t/gamma_s)(q_t.k_s) u_s.
    """
    n = len(parent)
    anc = np.zeros((n, n), bool)
    for t in range(n):
        for s in _path(parent, t):
            anc[t, s] = True
    gam = np.array([np.prod(alpha[_path(parent, t)]) for t in range(n)])
    ratio = gam[:, None] / gam[None, :]
    strict = anc & ~np.eye(n, dtype=bool)
    Lm = np.where(strict, beta[:, None] * ratio * (k @ k.T), 0.0)
    R = beta[:, None] * (v - gam[:, None] * (k @ h0))
    U = np.linalg.solve(np.eye(n) + Lm, R)
    Mm = np.where(anc, ratio * (q @ k.T), 0.0)
    return gam[:, None] * (q @ h0) + Mm @ U


@pytest.mark.parametrize("seed", range(4))
def test_wy_closed_form(seed):
    rng = np.random.default_rng(10 + seed)
    n, d = [(9, 8), (25, 16), (65, 12), (30, 5)][seed]
    parent, _ = _random_tree(rng, n, max_depth=[4, 8, 16, 30][seed])
    q, k, v, alpha, beta, h0 = _data(rng, n, 1, d, d)
    _, o = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    o_wy = _wy_outputs(parent, q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], h0[0])
    np.testing.assert_allclose(o[:, 0], o_wy, rtol=1e-10, atol=1e-11)


def test_homogeneity_and_column_permutation():
    rng = np.random.default_rng(6)
    n, H, d = 20, 2, 9
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, beta, h0 = _data(rng, n, H, d, d)
    st, o = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    st2, o2 = oracle.verify_request(parent, n, q, k, 2.5 * v, alpha, beta, 2.5 * h0)
    np.testing.assert_allclose(st2, 2.5 * st, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o2, 2.5 * o, rtol=1e-12, atol=1e-13)
    perm = rng.permutation(d)
    st3, o3 = oracle.verify_request(parent, n, q, k, v[..., perm], alpha, beta, h0[..., perm])
    np.testing.assert_allclose(st3, st[..., perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o3, o[..., perm], rtol=1e-13, atol=1e-14)


def test_norm_bound():
    """||I - beta k k^T||_2 <= 1 for unit k and beta in [0, 1], so
    ||h_i||_F <= alpha_i ||h_parent||_F + beta_i ||v_i||."""
    rng = np.random.default_rng(7)
    n, H, d = 30, 3, 8
    parent, _ = _random_tree(rng, n)
    q, k, v, alpha, beta, h0 = _data(rng, n, H, d, d)
    st, _ = oracle.verify_request(parent, n, q, k, v, alpha, beta, h0)
    for i in range(n):
        hp = h0 if i == 0 else st[parent[i]]
        lhs = np.linalg.norm(st[i], axis=(-2, -1))
        rhs = alpha[i] * np.linalg.norm(hp, axis=(-2, -1)) + beta[i] * np.linalg.norm(v[i], axis=-1)
        assert (lhs <= rhs * (1 + 1e-12)).all()


def test_commit_equals_node_state():
    """The committed state is the deepest accepted node's state (verify snapshots) and the
    chain recurrence over the accepted rows."""
    rng = np.random.default_rng(8)
    L, B, n, H, d = 2, 3, 12, 2, 6
    parents = [_random_tree(rng, n)[0] for _ in range(B)]
    tree = {"parent": np.stack(parents), "n_nodes": np.full(B, n)}
    q = _unit(rng.normal(size=(L, B, n, H, d)))
    k = _unit(rng.normal(size=(L, B, n, H, d)))
    v = rng.normal(size=(L, B, n, H, d))
    alpha = rng.uniform(0.3, 1, size=(L, B, n, H))
    beta = rng.uniform(0, 1, size=(L, B, n, H))
    h0 = rng.normal(size=(L, B, H, d, d))
    deepest = rng.integers(0, n, size=B)
    acc_node = np.full((B, n + 1), -1)
    acc_len = np.zeros(B, int)
    for b in range(B):
        p = _path(parents[b], int(deepest[b]))
        acc_node[b, :len(p)] = p
        acc_len[b] = len(p)
    _, _, kept = oracle.verify(tree, q, k, v, alpha, beta, h0, keep_states_of=deepest)
    new = oracle.commit(acc_node, acc_len, k, v, alpha, beta, h0)
    np.testing.assert_allclose(new, kept, rtol=1e-12, atol=1e-13)


def _commit_unrolled(k, v, alpha, beta, h0):
    """The accepted path's updates in unrolled form (the form the commit kernels evaluate):
    with G_x the product of alpha_0..alpha_x and R(x, y) = alpha_{y+1} ... alpha_x,
    S_{x-1}^T k_x = G_{x-1} h0^T k_x + sum_{y<x} R(x-1, y) (k_x . k_y) c_y,
    c_x = beta_x (v_x - alpha_x S_{x-1}^T k_x), and the final state is
    G h0 + sum_y R(tau-1, y) k_y c_y^T.  k, v: [tau][d]; alpha, beta: [tau]; h0: [dk][dv]."""
    tau = len(alpha)
    R = lambda x, y: float(np.prod(alpha[y + 1:x + 1]))  # empty product = 1
    d = k @ h0                      # [tau][dv]: k_x . h0[:, j]
    gram = k @ k.T
    c = np.zeros_like(v)
    G = 1.0
    for x in range(tau):
        ks = G * d[x] + sum(R(x - 1, y) * gram[x, y] * c[y] for y in range(x))
        c[x] = beta[x] * (v[x] - alpha[x] * ks)
        G *= alpha[x]
    return G * h0 + sum(R(tau - 1, y) * np.outer(k[y], c[y]) for y in range(tau))


@pytest.mark.parametrize("tau,d", [(1, 4), (2, 6), (5, 8), (17, 16)])
def test_commit_unrolled_form(tau, d):
    """The unrolled form equals the oracle's row-by-row commit along the same path, for unit
    and for unnormalised keys (the identity does not need |k| = 1)."""
    rng = np.random.default_rng(100 + tau)
    for unit_k in (True, False):
        n = tau
        _, k, v, alpha, beta, h0 = _data(rng, n, 1, d, d, unit_k=unit_k)
        acc_node = np.arange(tau)[None, :]
        acc_len = np.array([tau])
        ref = oracle.commit(acc_node, acc_len, k[None, None], v[None, None], alpha[None, None],
                            beta[None, None], h0[None, None])[0, 0, 0]
        got = _commit_unrolled(k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], h0[0])
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def _stock_chain(rows_q, rows_k, rows_v, rows_a, rows_b, h0_head):
    """The stock sequential recurrence over a row sequence of one head, written out here on its
    own (expanded form: h <- a h - a b k (k^T h) + b k v^T, then o = h^T q), independent of the
    oracle's code: states and outputs after every row."""
    h = np.array(h0_head, dtype=np.float64)
    states, outs = [], []
    for q_, k_, v_, a_, b_ in zip(rows_q, rows_k, rows_v, rows_a, rows_b):
        kh = np.einsum("i,ij->j", k_, h)
        h = a_ * h - (a_ * b_) * np.einsum("i,j->ij", k_, kh) + b_ * np.einsum("i,j->ij", k_, v_)
        states.append(h.copy())
        outs.append(np.einsum("ij,i->j", h, q_))
    return states, outs


def test_chain_tree_equals_sequence():
    """A chain-shaped tree (node i's parent is i-1) verifies like the stock sequential
    recurrence over the same rows, and a node of a branching tree like the stock recurrence over
    the rows of its root path; the recurrence is the separate loop above."""
    rng = np.random.default_rng(9)
    n, H, d = 12, 2, 8
    q, k, v, alpha, beta, h0 = _data(rng, n, H, d, d)
    st, o = oracle.verify_request(np.arange(-1, n - 1), n, q, k, v, alpha, beta, h0)
    assert st.shape == (n, H, d, d) and o.shape == (n, H, d)
    for hh in range(H):
        states, outs = _stock_chain(q[:, hh], k[:, hh], v[:, hh], alpha[:, hh], beta[:, hh], h0[hh])
        for i in range(n):
            np.testing.assert_allclose(st[i, hh], states[i], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(o[i, hh], outs[i], rtol=1e-12, atol=1e-13)
    # a branching tree: node 5's root path is 0-2-5, node 7's is 0-1-3-6-7
    parent = np.array([-1, 0, 0, 1, 2, 2, 3, 6])
    st_t, o_t = oracle.verify_request(parent, 8, q[:8], k[:8], v[:8], alpha[:8], beta[:8], h0)
    for node, rows in ((5, [0, 2, 5]), (7, [0, 1, 3, 6, 7])):
        for hh in range(H):
            states, outs = _stock_chain(q[rows, hh], k[rows, hh], v[rows, hh], alpha[rows, hh], beta[rows, hh],
                                        h0[hh])
            np.testing.assert_allclose(st_t[node, hh], states[-1], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(o_t[node, hh], outs[-1], rtol=1e-12, atol=1e-13)
