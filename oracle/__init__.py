"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .gdntree_oracle import (accept, build_tree, build_tree_cond, build_tree_shared, commit, gdn_readout,  # noqa: F401
                             gdn_step, gdn_update, markov_edge_logp, pipeline, verify, verify_request)
