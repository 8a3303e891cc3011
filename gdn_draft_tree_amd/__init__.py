"""gdn_draft_tree_amd: lossless draft-tree verification against a hybrid Gated-DeltaNet
target, as hand-written gfx950 (MI355X) HIP kernels behind a C ABI (include/gdntree.h).

    tree = gdntree_build(lat_logp, lat_tok, root_tok, N)
    o    = gdntree_verify(tree, q, k, v, alpha, beta, state)          # per GDN layer
    acc  = gdntree_accept_commit(tree, target_argmax, k, v, alpha, beta, state, P)
    # or, split: acc = gdntree_accept(tree, target_argmax, P); gdntree_commit(tree, acc[0], acc[2], ...)
    # a whole batch under one budget of G draft nodes (request b over positions[b] positions):
    tree = gdntree_build_shared(lat_logp, lat_tok, root_tok, N, G, positions)
    # the end of a step fused with the next step's build (optionally under a batch budget):
    acc  = gdntree_accept_commit_build(tree, target_argmax, k, v, alpha, beta, state, P, *next_lattice, N, next_tree)
    # a Markov-head drafter (candidate scores conditioned on the previous token):
    edge = gdntree_markov_edges(bases, lat_tok, root_tok, W1, W2)   # [B][P][K][K]
    tree = gdntree_build_cond(edge, lat_tok, root_tok, N)
    # the commit deferred into the next step's verify (the state read once per step):
    acc  = gdntree_accept_build(tree, target_argmax, P, *next_lattice, N, next_tree)
    o    = gdntree_accept_commit_verify(tree, target_argmax, k, v, alpha, beta, P, next_tree, *next_rows, state)

Importing this package loads libgdntree.so and raises if it has not been built.
"""
from ._binding import (EXPORTED, GDNTREE_BF16, GDNTREE_ERR_ARG, GDNTREE_ERR_DEVICE,  # noqa: F401
                       GDNTREE_ERR_UNSUPPORTED, GDNTREE_F32, GDNTREE_OK, LIB, LIB_PATH, CTree,
                       GdnTreeError, Tree, gdntree_accept, gdntree_accept_build, gdntree_accept_commit,
                       gdntree_accept_commit_build, gdntree_accept_commit_build_shared,
                       gdntree_accept_commit_verify, gdntree_build,
                       gdntree_build_cond, gdntree_build_shared, gdntree_commit, gdntree_commit_build,
                       gdntree_markov_edges, gdntree_status_str, gdntree_verify)
