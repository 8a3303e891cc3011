"""Seeded synthetic workloads for draft-tree verification.

This package draws inputs only: lattices, synthetic target choices, q/k/v/alpha/beta
rows and initial recurrent states.  It holds none of the method's arithmetic (no
tree building, no recurrence, no acceptance) and imports neither the oracle nor the
HIP library, so both sides of every parity test can consume the same arrays.
"""
from .configs import CONFIGS, Config  # noqa: F401
from .generate import MarkovHead, Workload, generate, markov_head, resolve_target  # noqa: F401
