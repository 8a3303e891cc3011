"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .gdntree_oracle import (accept, build_tree, build_tree_shared, commit, gdn_readout, gdn_step,  # noqa: F401
                             gdn_update, pipeline, verify, verify_request)
