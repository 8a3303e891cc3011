"""Seeded generator for the synthetic workloads.

Recipe (one named child stream of ``numpy.random.SeedSequence(seed)`` per item, in order):
 1. lattice logits ~ N(0, std 2) [B][P][K] -> log-softmax over K in fp64 -> sorted
    descending -> fp32.
 2. lattice tokens: per (b, p), K distinct ids drawn uniformly from [0, V) without
    replacement (draw order is the rank).
 3. root tokens [B] uniform in [0, V).
 4. per-request top-1 agreement p_b (fixed, or ~U(lo, hi)), then per-slot target choice
    [B][N+1] in {0..K-1 (a lattice rank), K (a uniform token)}.
 5. per-slot uniform target tokens [B][N+1].
 6. q ~ N(0,1) [L][B][N+1][H][D], L2-normalised over D in fp64.
 7. k likewise.
 8. v ~ N(0,1).
 9. g ~ N(0,1) [L][B][N+1][H]; alpha = exp(-softplus(g)).
10. beta = sigmoid(N(0,1)).
11. h0 ~ N(0, std 0.1) [L][B][H][D_k][D_v], fp32.

q, k, v, alpha and beta are then cast to the config dtype (bf16 by round-to-nearest-even
through torch on the CPU, or fp32).  The cast tensors are what both the oracle (widened
exactly to fp64) and the GPU consume.

Markov-head inputs (``markov_head``, for the parent-conditioned lattices), from
``numpy.random.SeedSequence([seed, 0x4D48])`` in three named child streams: base logits
~ N(0, std 2) [B][P][K] sorted descending along K (rank 0 is the selector's top candidate),
then W1 and W2 ~ N(0, std 1/sqrt(R)) [V][R] in fp32, so that <W1[x], W2[y]> has unit std.
They pair with a workload's lattice tokens and root tokens; random matrices stand in for a
trained head.

The synthetic target argmax of tree slot i (the token the target model predicts after the
node in slot i) is the lattice candidate of rank c_i at the node's child position when the
slot's choice c_i is a rank and the node is above the last position, else the slot's
uniform token.  It is resolved from a built tree by ``resolve_target``; this stands in for
the target's LM head, which is outside the verified path.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import CONFIGS, Config

_STREAMS = ("lat_logits", "lat_tokens", "root_tok", "tgt_choice", "tgt_uniform",
            "q", "k", "v", "g", "beta", "h0")


@dataclass
class Workload:
    cfg: Config
    seed: int
    lat_logp: np.ndarray      # f32 [B][P][K], sorted descending along K
    lat_tok: np.ndarray       # i32 [B][P][K], distinct per (b, p)
    root_tok: np.ndarray      # i32 [B]
    p_top1: np.ndarray        # f64 [B]
    tgt_choice: np.ndarray    # i32 [B][N+1], K means "uniform token"
    tgt_uniform: np.ndarray   # i32 [B][N+1]
    q: torch.Tensor           # cfg dtype, CPU, [L][B][N+1][H][D]
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor       # cfg dtype, CPU, [L][B][N+1][H]
    beta: torch.Tensor
    h0: torch.Tensor          # f32, CPU, [L][B][H][D_k][D_v]

    def f64(self, name: str) -> np.ndarray:
        """The named tensor widened exactly to fp64 numpy."""
        return getattr(self, name).to(torch.float64).numpy()


def _rngs(seed: int) -> dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def _target_probs(cfg: Config, p1: float) -> np.ndarray:
    """Probabilities of choices 0..K-1 (lattice ranks) and K (uniform token)."""
    p = np.zeros(cfg.K + 1)
    p[0] = p1
    if cfg.rank_tail and cfg.K > 1:
        r = np.arange(1, cfg.K)
        p[1:cfg.K] = (1.0 - p1) * (2.0 / 3.0) * 0.5 ** r
    p[cfg.K] = 1.0 - p[:cfg.K].sum()
    return p


def target_probs(cfg: Config, p1: float) -> np.ndarray:
    return _target_probs(cfg, p1)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def generate(cfg: Config | str, seed: int = 0, *, B: int | None = None) -> Workload:
    """Draw one workload.  ``B`` overrides the request count (for bounded samples)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if B is not None:
        from dataclasses import replace
        cfg = replace(cfg, B=B)
    g = _rngs(seed)
    Bn, L, H, D, P, K, V, R = cfg.B, cfg.L, cfg.H, cfg.D, cfg.P, cfg.K, cfg.V, cfg.rows

    logits = g["lat_logits"].normal(0.0, 2.0, size=(Bn, P, K))
    m = logits.max(axis=-1, keepdims=True)
    logp = logits - (m + np.log(np.exp(logits - m).sum(axis=-1, keepdims=True)))
    logp = -np.sort(-logp, axis=-1)
    lat_logp = logp.astype(np.float32)

    lat_tok = np.empty((Bn, P, K), dtype=np.int32)
    for b in range(Bn):
        for p in range(P):
            lat_tok[b, p] = g["lat_tokens"].choice(V, size=K, replace=False)

    root_tok = g["root_tok"].integers(0, V, size=Bn).astype(np.int32)

    if cfg.p_top1_range is not None:
        lo, hi = cfg.p_top1_range
        p_top1 = g["tgt_choice"].uniform(lo, hi, size=Bn)
    else:
        p_top1 = np.full(Bn, cfg.p_top1)
    u = g["tgt_choice"].random(size=(Bn, R))
    tgt_choice = np.empty((Bn, R), dtype=np.int32)
    for b in range(Bn):
        cdf = np.cumsum(_target_probs(cfg, float(p_top1[b])))
        cdf[-1] = 1.0
        tgt_choice[b] = np.searchsorted(cdf, u[b], side="right").clip(0, K)
    tgt_uniform = g["tgt_uniform"].integers(0, V, size=(Bn, R)).astype(np.int32)

    def unit_rows(rng):
        x = rng.normal(0.0, 1.0, size=(L, Bn, R, H, D))
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    q = unit_rows(g["q"])
    k = unit_rows(g["k"])
    v = g["v"].normal(0.0, 1.0, size=(L, Bn, R, H, D))
    gg = g["g"].normal(0.0, 1.0, size=(L, Bn, R, H))
    alpha = np.exp(-np.logaddexp(0.0, gg))
    beta = 1.0 / (1.0 + np.exp(-g["beta"].normal(0.0, 1.0, size=(L, Bn, R, H))))
    h0 = g["h0"].normal(0.0, 0.1, size=(L, Bn, H, D, D)).astype(np.float32)

    return Workload(cfg=cfg, seed=seed, lat_logp=lat_logp, lat_tok=lat_tok, root_tok=root_tok,
                    p_top1=p_top1, tgt_choice=tgt_choice, tgt_uniform=tgt_uniform,
                    q=_cast(q, cfg.dtype), k=_cast(k, cfg.dtype), v=_cast(v, cfg.dtype),
                    alpha=_cast(alpha, cfg.dtype), beta=_cast(beta, cfg.dtype),
                    h0=torch.from_numpy(h0))


def resolve_target(depth: np.ndarray, n_nodes: np.ndarray, lat_tok: np.ndarray,
                   tgt_choice: np.ndarray, tgt_uniform: np.ndarray) -> np.ndarray:
    """Synthetic per-slot target argmax [B][N+1] for a built tree.

    ``depth`` is the tree's depth array [B][N+1] and ``n_nodes`` its node counts [B];
    slots at or beyond ``n_nodes`` get their uniform token.
    """
    Bn, P, K = lat_tok.shape
    out = tgt_uniform.copy()
    for b in range(Bn):
        for i in range(int(n_nodes[b])):
            c, d = int(tgt_choice[b, i]), int(depth[b, i])
            if c < K and d < P:
                out[b, i] = lat_tok[b, d, c]
    return out.astype(np.int32)


@dataclass
class MarkovHead:
    bases: np.ndarray  # f32 [B][P][K], sorted descending along K
    W1: np.ndarray     # f32 [V][R], previous-token embeddings
    W2: np.ndarray     # f32 [V][R], candidate embeddings


def markov_head(cfg: Config | str, seed: int = 0, R: int = 32, *, B: int | None = None) -> MarkovHead:
    """Seeded stand-ins for a Markov head over the config's lattice shape (see the recipe)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    Bn = cfg.B if B is None else B
    bases_s, w1_s, w2_s = (np.random.Generator(np.random.PCG64(c))
                           for c in np.random.SeedSequence([seed, 0x4D48]).spawn(3))
    bases = -np.sort(-bases_s.normal(0.0, 2.0, size=(Bn, cfg.P, cfg.K)), axis=-1).astype(np.float32)
    W1 = w1_s.normal(0.0, 1.0 / np.sqrt(R), size=(cfg.V, R)).astype(np.float32)
    W2 = w2_s.normal(0.0, 1.0 / np.sqrt(R), size=(cfg.V, R)).astype(np.float32)
    return MarkovHead(bases, W1, W2)
