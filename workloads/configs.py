"""The five workload presets, and the ragged batch under a shared node budget.

Shapes follow the SpecPilot summary (paper.rainbus.top/paper/2611.02501): parallel drafters
propose 8 or 16 masked positions with a top-16 candidate lattice (section "Prerequisites >
parallel drafter"); best-first trees of N=24..64 nodes (sections "Prerequisites > draft-tree
verification" and "Technical novelty"); 48 GDN layers in the hybrid target (section
"Prerequisites > hybrid recurrent architecture"); batches of 16-32 requests (section
"Motivation").  Head size 128 and 32 heads are the usual Gated-DeltaNet head geometry.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    B: int            # requests
    L: int            # independent GDN layers sharing one tree
    H: int            # heads per layer
    D: int            # head dim (d_k = d_v)
    dtype: str        # "f32" or "bf16" for q, k, v, alpha, beta and the output o
    P: int            # drafter positions
    K: int            # candidates per position
    V: int            # vocabulary size
    N: int            # draft-node budget (root not counted)
    # synthetic target model: probability that the target's argmax is the rank-0 candidate
    p_top1: float = 0.85
    # when set, p_top1 is drawn per request from U(lo, hi)
    p_top1_range: tuple | None = None
    # include the geometric rank-r tail (rank r>=1 with prob (1-p)*(2/3)*0.5**r)
    rank_tail: bool = True
    # when set, the trees are built under one batch budget of G draft nodes (N stays the
    # per-request cap), and request b uses positions[b % len(positions)] lattice positions
    G: int | None = None
    positions: tuple | None = None
    notes: str = field(default="", compare=False)

    def positions_for(self, B: int | None = None):
        B = self.B if B is None else B
        return None if self.positions is None else [self.positions[b % len(self.positions)] for b in range(B)]

    @property
    def rows(self) -> int:
        return self.N + 1


CONFIGS: dict[str, Config] = {
    "tiny": Config("tiny", B=1, L=1, H=1, D=64, dtype="f32", P=4, K=4, V=32000, N=8,
                   rank_tail=False,
                   notes="1 request, 1 head, d=64, fp32 everything, 4x4 lattice, N=8"),
    "one_layer": Config("one_layer", B=1, L=1, H=32, D=128, dtype="bf16", P=8, K=16,
                        V=151936, N=24,
                        notes="one GDN layer, batch 1, 8x16 lattice, N=24"),
    "deep": Config("deep", B=1, L=48, H=32, D=128, dtype="bf16", P=16, K=16, V=151936,
                   N=64, notes="48 independent GDN layers, batch 1, 16x16 lattice, N=64"),
    "batched": Config("batched", B=24, L=1, H=32, D=128, dtype="bf16", P=8, K=16,
                      V=151936, N=24,
                      notes="24 requests x one GDN layer, 8x16 lattices, N=24"),
    "ragged": Config("ragged", B=32, L=1, H=32, D=128, dtype="bf16", P=16, K=16,
                     V=151936, N=64, p_top1_range=(0.6, 0.95),
                     notes="32 requests x one GDN layer, 16x16 lattices, N=64, "
                           "per-request top-1 agreement ~ U(0.6, 0.95)"),
    # the ragged batch under a node budget shared by the batch (SpecPilot summary, Technical
    # novelty, batching: a 192-node budget, draft positions 16/12/8 chosen per request)
    "shared": Config("shared", B=32, L=1, H=32, D=128, dtype="bf16", P=16, K=16, V=151936,
                     N=64, p_top1_range=(0.6, 0.95), G=192, positions=(16, 12, 8),
                     notes="32 requests x one GDN layer, 16x16 lattices, one batch budget of 192 "
                           "draft nodes (at most 64 per request), draft positions 16/12/8 by "
                           "request, per-request top-1 agreement ~ U(0.6, 0.95)"),
}
