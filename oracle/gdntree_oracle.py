"""Plain fp64 CPU oracle for lossless draft-tree verification on a Gated-DeltaNet target.

TEST INFRASTRUCTURE ONLY.  This module is imported solely by the test suite, by the
smoke check of the package entry file and by the benchmark's CPU-baseline leg.  The
library's product path never imports, links or executes anything here, and this module
imports nothing from the library: the two share no code.

Sources (the pages this follows; "SpecPilot summary" is the paper summary page for
"SpecPilot: Autonomous Algorithm Discovery and Systems Optimization for Speculative
Decoding", paper.rainbus.top/paper/2611.02501):
  * Greedy lossless acceptance: the longest draft prefix equal to the target argmax is
    accepted plus one bonus token, tau in [1, m+1] (SpecPilot summary, Prerequisites >
    speculative decoding).
  * Draft-tree verification: one target pass over a tree where every node sees only its
    ancestors; accept the longest root path matching the target argmax plus a bonus
    token; DDTree-style construction adds nodes greedily by path log-probability up to N
    (SpecPilot summary, Prerequisites > draft-tree verification).  The best-first tree
    scores edges by log p(child | parent) and may be wider than the drafter block
    (SpecPilot summary, Technical novelty).
  * Parent-conditioned edge scores (a DSpark-style Markov head): the logit of candidate y
    at position s is l_s(y) = bases(y) + <W1[x_{s-1}], W2[y]>, conditioned on the previous
    token x_{s-1} (SpecPilot summary, Prerequisites > parallel drafters and lattices).
  * Gated DeltaNet: h_t = alpha_t (I - beta_t k_t k_t^T) h_{t-1} + beta_t k_t v_t^T,
    o_t = h_t^T q_t; tree verification recomputes states along root paths instead of
    snapshotting every node (SpecPilot summary, Prerequisites > hybrid recurrent
    architecture; Technical novelty).

Readings where the pages leave a step open (each listed in the design notes):
  * N counts draft nodes only; slot 0 is the root (the pending last token) and the verify
    pass processes N+1 rows, the root first, starting from the committed state h0.
  * A node's score is the sum of the lattice log-probs of the ranks along its path,
    accumulated root to leaf in fp64 (score_child = score_parent + float64(logp)).
  * Ties in the best-first pop go to the smaller parent index, then the smaller rank; the
    node index is the insertion order.
  * If the trie holds fewer than N nodes the build stops early.
  * If several children of the current node match the target, the smallest index wins.
  * With a budget shared by the batch, G counts draft nodes over all requests (roots not
    counted), N stays the per-request cap, and ties across requests go to the smaller
    request index.
  * Outputs carry no 1/sqrt(d_k) scale: o = h^T q exactly.
  * Markov head: a position's candidate set stays the lattice's K tokens; only their scores
    depend on the previous token, which is the parent node's token (the root token at
    position 0).  bases(y) is the drafter's base logit of candidate y at that position.
    The edge log-prob is the log-softmax of l_s over the position's K candidates.

Every function is a direct transcription of the definition; nothing is blocked, fused or
reordered.  This oracle keeps every per-node state of one (layer, request) while it
verifies (the snapshot method the pages avoid on the GPU, harmless on the CPU).
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------------------
# (a) best-first tree construction
# --------------------------------------------------------------------------------------
def build_tree(lat_logp: np.ndarray, lat_tok: np.ndarray, root_tok: np.ndarray, N: int) -> dict:
    """Best-first draft tree over a drafter lattice, one per request.

    SpecPilot summary, Prerequisites > draft-tree verification (greedy addition by path
    log-prob up to N nodes) and Technical novelty (edges scored by log p(child|parent)).

    lat_logp: f32 [B][P][K] candidate log-probs per position; lat_tok: int [B][P][K];
    root_tok: int [B]; N: draft-node budget.
    Returns arrays of shape [B][N+1] (slots >= n_nodes[b] hold -1 / 0 / NaN fillers):
    parent, depth, rank, token (int64), score (f64), anc (uint64: bit j-1 set iff draft
    slot j is an ancestor-or-self), and n_nodes [B] (root included).
    """
    B, P, K = lat_logp.shape
    out = {
        "parent": np.full((B, N + 1), -1, np.int64),
        "depth": np.full((B, N + 1), -1, np.int64),
        "rank": np.full((B, N + 1), -1, np.int64),
        "token": np.full((B, N + 1), -1, np.int64),
        "score": np.full((B, N + 1), np.nan),
        "anc": np.zeros((B, N + 1), np.uint64),
        "n_nodes": np.zeros(B, np.int64),
    }
    for b in range(B):
        parent, depth, rank, token, score, anc = [-1], [0], [-1], [int(root_tok[b])], [0.0], [0]
        # the full frontier: every child (p, r) of every inserted node p not yet inserted
        frontier = [(0, r) for r in range(K)] if P > 0 else []
        while len(parent) - 1 < N and frontier:
            def key(c):
                p, r = c
                s = score[p] + float(np.float64(lat_logp[b, depth[p], r]))
                return (-s, p, r)
            best = min(frontier, key=key)
            frontier.remove(best)
            p, r = best
            i = len(parent)
            d = depth[p] + 1
            parent.append(p)
            depth.append(d)
            rank.append(r)
            token.append(int(lat_tok[b, d - 1, r]))
            score.append(score[p] + float(np.float64(lat_logp[b, d - 1, r])))
            anc.append(anc[p] | (1 << (i - 1)))
            if d < P:
                frontier.extend((i, rr) for rr in range(K))
        n = len(parent)
        out["parent"][b, :n] = parent
        out["depth"][b, :n] = depth
        out["rank"][b, :n] = rank
        out["token"][b, :n] = token
        out["score"][b, :n] = score
        out["anc"][b, :n] = np.array(anc, dtype=np.uint64)
        out["n_nodes"][b] = n
    return out


def build_tree_shared(lat_logp: np.ndarray, lat_tok: np.ndarray, root_tok: np.ndarray, N: int,
                      G: int, positions=None) -> dict:
    """Best-first draft trees for a whole batch under one shared node budget.

    SpecPilot summary, Technical novelty (batching: the node budget is shared across the
    batch, and each request gets its own number of draft positions).  One best-first pass
    runs over the union of every request's frontier: it adds the candidate with the
    largest path log-prob until the batch holds G draft nodes or no candidate is left.  A
    request that holds N draft nodes offers no more candidates (its tree keeps N+1 slots),
    and request b draws children only from its first positions[b] lattice positions
    (all P when positions is None; values are clipped to [0, P]).

    Ties: the smaller request index, then the smaller parent slot, then the smaller rank.
    Node indices within a request are its insertion order.  Returns the arrays of
    build_tree, with every request's tree in its own [N+1] slots.
    """
    B, P, K = lat_logp.shape
    pos = np.full(B, P) if positions is None else np.clip(np.asarray(positions), 0, P)
    out = {
        "parent": np.full((B, N + 1), -1, np.int64),
        "depth": np.full((B, N + 1), -1, np.int64),
        "rank": np.full((B, N + 1), -1, np.int64),
        "token": np.full((B, N + 1), -1, np.int64),
        "score": np.full((B, N + 1), np.nan),
        "anc": np.zeros((B, N + 1), np.uint64),
        "n_nodes": np.zeros(B, np.int64),
    }
    trees = [{"parent": [-1], "depth": [0], "rank": [-1], "token": [int(root_tok[b])],
              "score": [0.0], "anc": [0]} for b in range(B)]
    # the full frontier of the batch: (request, parent slot, rank)
    frontier = [(b, 0, r) for b in range(B) if pos[b] > 0 and N > 0 for r in range(K)]
    total = 0
    while total < G and frontier:
        def key(c):
            b, p, r = c
            t = trees[b]
            s = t["score"][p] + float(np.float64(lat_logp[b, t["depth"][p], r]))
            return (-s, b, p, r)
        best = min(frontier, key=key)
        frontier.remove(best)
        b, p, r = best
        t = trees[b]
        i = len(t["parent"])
        d = t["depth"][p] + 1
        t["parent"].append(p)
        t["depth"].append(d)
        t["rank"].append(r)
        t["token"].append(int(lat_tok[b, d - 1, r]))
        t["score"].append(t["score"][p] + float(np.float64(lat_logp[b, d - 1, r])))
        t["anc"].append(t["anc"][p] | (1 << (i - 1)))
        total += 1
        if d < pos[b]:
            frontier.extend((b, i, rr) for rr in range(K))
        if i == N:  # the request is full: withdraw its remaining candidates
            frontier = [c for c in frontier if c[0] != b]
    for b, t in enumerate(trees):
        n = len(t["parent"])
        for name in ("parent", "depth", "rank", "token", "score"):
            out[name][b, :n] = t[name]
        out["anc"][b, :n] = np.array(t["anc"], dtype=np.uint64)
        out["n_nodes"][b] = n
    return out


def markov_edge_logp(bases: np.ndarray, lat_tok: np.ndarray, root_tok: np.ndarray, W1: np.ndarray,
                     W2: np.ndarray) -> np.ndarray:
    """Parent-conditioned edge log-probs of a DSpark-style Markov head.

    SpecPilot summary, Prerequisites > parallel drafters and lattices: the head scores
    candidate y at position s as l_s(y) = bases(y) + <W1[x_{s-1}], W2[y]>, where x_{s-1} is
    the previous token.  In a draft tree the previous token of a child at position s is its
    parent's token: the root token for s = 0, otherwise the lattice candidate of the parent's
    rank at position s-1.

    bases: f32 [B][P][K] base logits of the lattice candidates; lat_tok: int [B][P][K];
    root_tok: int [B]; W1, W2: [V][R] embeddings of the previous and of the candidate token.
    Returns fp64 [B][P][K][K]: [b][s][pr][r] = l_s(lat_tok[b,s,r] | x) minus the
    log-sum-exp of l_s over the position's K candidates, with x = root_tok[b] for s = 0
    (every pr row the same) and x = lat_tok[b,s-1,pr] for s >= 1.
    """
    B, P, K = bases.shape
    out = np.empty((B, P, K, K))
    for b in range(B):
        for s in range(P):
            for pr in range(K):
                x = int(root_tok[b]) if s == 0 else int(lat_tok[b, s - 1, pr])
                w1 = np.asarray(W1[x], np.float64)
                logits = np.array([float(bases[b, s, r]) + float(np.dot(w1, np.asarray(W2[int(lat_tok[b, s, r])],
                                                                                     np.float64)))
                                   for r in range(K)])
                m = logits.max()
                out[b, s, pr] = logits - (m + np.log(np.sum(np.exp(logits - m))))
    return out


def build_tree_cond(edge_logp: np.ndarray, lat_tok: np.ndarray, root_tok: np.ndarray, N: int) -> dict:
    """Best-first draft tree whose edge log-probs depend on the parent (a Markov-head lattice).

    SpecPilot summary, Technical novelty (edges scored by log p(child | parent)) and
    Prerequisites > draft-tree verification (greedy addition by path log-prob up to N).
    The same construction as build_tree, except that the log-prob of child rank r of node
    p is edge_logp[b, depth(p), pr, r] with pr = rank(p) (the parent's candidate at its own
    position), and pr = 0 for the root's children.

    edge_logp: f32 [B][P][K][K]; lat_tok: int [B][P][K]; root_tok: int [B]; N: budget.
    Ties: the smaller parent slot, then the smaller rank.  Returns the arrays of build_tree.
    """
    B, P, K = lat_tok.shape
    out = {
        "parent": np.full((B, N + 1), -1, np.int64),
        "depth": np.full((B, N + 1), -1, np.int64),
        "rank": np.full((B, N + 1), -1, np.int64),
        "token": np.full((B, N + 1), -1, np.int64),
        "score": np.full((B, N + 1), np.nan),
        "anc": np.zeros((B, N + 1), np.uint64),
        "n_nodes": np.zeros(B, np.int64),
    }
    for b in range(B):
        parent, depth, rank, token, score, anc = [-1], [0], [-1], [int(root_tok[b])], [0.0], [0]
        frontier = [(0, r) for r in range(K)] if P > 0 else []

        def edge(p, r):
            return float(np.float64(edge_logp[b, depth[p], rank[p] if depth[p] >= 1 else 0, r]))

        while len(parent) - 1 < N and frontier:
            best = min(frontier, key=lambda c: (-(score[c[0]] + edge(*c)), c[0], c[1]))
            frontier.remove(best)
            p, r = best
            i = len(parent)
            d = depth[p] + 1
            s_new = score[p] + edge(p, r)
            parent.append(p)
            depth.append(d)
            rank.append(r)
            token.append(int(lat_tok[b, d - 1, r]))
            score.append(s_new)
            anc.append(anc[p] | (1 << (i - 1)))
            if d < P:
                frontier.extend((i, rr) for rr in range(K))
        n = len(parent)
        out["parent"][b, :n] = parent
        out["depth"][b, :n] = depth
        out["rank"][b, :n] = rank
        out["token"][b, :n] = token
        out["score"][b, :n] = score
        out["anc"][b, :n] = np.array(anc, dtype=np.uint64)
        out["n_nodes"][b] = n
    return out


# --------------------------------------------------------------------------------------
# (b) gated delta rule along the tree
# --------------------------------------------------------------------------------------
def gdn_update(h_prev: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
               beta: np.ndarray) -> np.ndarray:
    """One gated-delta-rule state update, batched over leading axes.

    SpecPilot summary, Prerequisites > hybrid recurrent architecture:
        h = alpha (I - beta k k^T) h_prev + beta k v^T.
    h_prev: [..., dk, dv]; k: [..., dk]; v: [..., dv]; alpha, beta: [...].
    """
    a = alpha[..., None, None]
    b = beta[..., None, None]
    kT_h = (k[..., None, :] @ h_prev)[..., 0, :]                 # k^T h_prev   [..., dv]
    return a * (h_prev - b * k[..., :, None] * kT_h[..., None, :]) + b * k[..., :, None] * v[..., None, :]


def gdn_readout(h: np.ndarray, q: np.ndarray) -> np.ndarray:
    """o = h^T q (same passage); h: [..., dk, dv], q: [..., dk] -> [..., dv]."""
    return (q[..., None, :] @ h)[..., 0, :]


def gdn_step(h_prev, q, k, v, alpha, beta):
    """Update then readout: returns (h, o)."""
    h = gdn_update(h_prev, k, v, alpha, beta)
    return h, gdn_readout(h, q)


def verify_request(parent: np.ndarray, n: int, q, k, v, alpha, beta, h0):
    """Every node's state and output for one (layer, request).

    Node states are computed in insertion order from the parent's state, the root from h0
    (SpecPilot summary, Prerequisites > hybrid recurrent architecture and draft-tree
    verification: each node depends only on its ancestors).
    q, k, v: [N+1][H][d]; alpha, beta: [N+1][H]; h0: [H][dk][dv] (all fp64).
    Returns states [n][H][dk][dv] and outputs [n][H][dv].
    """
    H, dk, dv = h0.shape
    states = np.empty((n, H, dk, dv))
    outs = np.empty((n, H, dv))
    for i in range(n):
        hp = h0 if i == 0 else states[parent[i]]
        states[i], outs[i] = gdn_step(hp, q[i], k[i], v[i], alpha[i], beta[i])
    return states, outs


def verify(tree: dict, q, k, v, alpha, beta, h0, keep_states_of=None):
    """Tree verify for every layer and request.

    q, k, v: [L][B][N+1][H][d]; alpha, beta: [L][B][N+1][H]; h0: [L][B][H][dk][dv] (fp64).
    Returns o [L][B][N+1][H][dv] (NaN in unused slots) and hnorm [L][B][N+1][H], the
    Frobenius norm of each node's fp64 state (the scale of the parity tolerance).
    ``keep_states_of``: optional [B] array of node indices whose states are also returned
    as a [L][B][H][dk][dv] array.
    """
    L, B, R, H, _ = q.shape
    dv = v.shape[-1]
    o = np.full((L, B, R, H, dv), np.nan)
    hnorm = np.full((L, B, R, H), np.nan)
    kept = None if keep_states_of is None else np.empty_like(h0)
    for l in range(L):
        for b in range(B):
            n = int(tree["n_nodes"][b])
            st, ou = verify_request(tree["parent"][b], n, q[l, b], k[l, b], v[l, b],
                                    alpha[l, b], beta[l, b], h0[l, b])
            o[l, b, :n] = ou
            hnorm[l, b, :n] = np.sqrt((st ** 2).sum(axis=(-2, -1)))
            if kept is not None:
                kept[l, b] = st[int(keep_states_of[b])]
    return (o, hnorm) if kept is None else (o, hnorm, kept)


# --------------------------------------------------------------------------------------
# (c) greedy acceptance and accepted-path commit
# --------------------------------------------------------------------------------------
def accept(tree: dict, target: np.ndarray, P: int):
    """Longest root path whose tokens equal the target argmax, plus one bonus token.

    SpecPilot summary, Prerequisites > speculative decoding (greedy acceptance plus bonus,
    tau in [1, m+1]) and > draft-tree verification (longest matching root path).
    target: [B][N+1], the target's argmax after each slot's node.
    Returns acc_len [B] (= tau), acc_tok [B][P+1] (accepted draft tokens then the bonus,
    padded with -1) and acc_node [B][P+1] (root, then the accepted nodes, padded -1).
    """
    B = target.shape[0]
    acc_len = np.zeros(B, np.int64)
    acc_tok = np.full((B, P + 1), -1, np.int64)
    acc_node = np.full((B, P + 1), -1, np.int64)
    for b in range(B):
        n = int(tree["n_nodes"][b])
        u, path = 0, [0]
        while True:
            nxt = [c for c in range(1, n)
                   if tree["parent"][b, c] == u and tree["token"][b, c] == target[b, u]]
            if not nxt:
                break
            u = min(nxt)
            path.append(u)
        toks = [int(tree["token"][b, c]) for c in path[1:]] + [int(target[b, u])]
        acc_len[b] = len(path)
        acc_tok[b, :len(toks)] = toks
        acc_node[b, :len(path)] = path
    return acc_len, acc_tok, acc_node


def commit(acc_node: np.ndarray, acc_len: np.ndarray, k, v, alpha, beta, h0):
    """New recurrent state of every (layer, request, head): the state at the deepest
    accepted node, recomputed from h0 along root -> accepted path with the gated delta
    rule (SpecPilot summary, Prerequisites > hybrid recurrent architecture: states are
    recomputed along root paths rather than snapshotted).
    k, v: [L][B][N+1][H][d]; alpha, beta: [L][B][N+1][H]; h0: [L][B][H][dk][dv].
    Returns the committed states [L][B][H][dk][dv].
    """
    L, B = h0.shape[:2]
    out = np.empty_like(h0)
    for l in range(L):
        for b in range(B):
            h = h0[l, b]
            for i in acc_node[b, :int(acc_len[b])]:
                h = gdn_update(h, k[l, b, i], v[l, b, i], alpha[l, b, i], beta[l, b, i])
            out[l, b] = h
    return out


def pipeline(lat_logp, lat_tok, root_tok, N, q, k, v, alpha, beta, h0, target_fn, G=None,
             positions=None):
    """build -> verify -> accept -> commit for one batch.

    ``target_fn(tree)`` returns the per-slot target argmax [B][N+1] for the built tree (the
    target model's LM head is outside the method; the caller supplies it).  With ``G`` set,
    the trees come from build_tree_shared (batch budget G, per-request ``positions``).
    """
    P = lat_logp.shape[1]
    if G is None:
        tree = build_tree(lat_logp, lat_tok, root_tok, N)
    else:
        tree = build_tree_shared(lat_logp, lat_tok, root_tok, N, G, positions)
    o, hnorm = verify(tree, q, k, v, alpha, beta, h0)
    target = target_fn(tree)
    acc_len, acc_tok, acc_node = accept(tree, target, P)
    new_state = commit(acc_node, acc_len, k, v, alpha, beta, h0)
    return {"tree": tree, "o": o, "hnorm": hnorm, "target": target, "acc_len": acc_len,
            "acc_tok": acc_tok, "acc_node": acc_node, "state": new_state}
