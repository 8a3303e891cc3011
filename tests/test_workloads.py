"""The seeded generator produces the documented shapes, dtypes and distributions."""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, generate, resolve_target


@pytest.mark.parametrize("name", ["tiny", "one_layer", "batched"])
def test_shapes_dtypes_and_ranges(name):
    cfg = CONFIGS[name]
    w = generate(cfg, seed=0)
    B, L, H, D, P, K, R = cfg.B, cfg.L, cfg.H, cfg.D, cfg.P, cfg.K, cfg.rows
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    assert w.lat_logp.shape == (B, P, K) and w.lat_logp.dtype == np.float32
    assert w.lat_tok.shape == (B, P, K) and w.lat_tok.dtype == np.int32
    assert (np.diff(w.lat_logp, axis=-1) <= 0).all()
    assert (w.lat_logp <= 0).all()
    np.testing.assert_allclose(np.exp(w.lat_logp.astype(np.float64)).sum(-1), 1.0, rtol=1e-5)
    for b in range(B):
        for p in range(P):
            assert len(set(w.lat_tok[b, p].tolist())) == K
    assert ((w.lat_tok >= 0) & (w.lat_tok < cfg.V)).all()
    for name_ in ("q", "k", "v"):
        t = getattr(w, name_)
        assert t.shape == (L, B, R, H, D) and t.dtype == dt
    for name_ in ("alpha", "beta"):
        t = getattr(w, name_)
        assert t.shape == (L, B, R, H) and t.dtype == dt
        x = w.f64(name_)
        assert (x > 0).all() and (x < 1).all()
    assert w.h0.shape == (L, B, H, D, D) and w.h0.dtype == torch.float32
    qn = np.linalg.norm(w.f64("q"), axis=-1)
    tol = 1e-6 if cfg.dtype == "f32" else 2 ** -7
    assert np.abs(qn - 1).max() < tol
    assert ((w.tgt_choice >= 0) & (w.tgt_choice <= K)).all()


def test_seeded_determinism():
    a = generate("one_layer", seed=3)
    b = generate("one_layer", seed=3)
    c = generate("one_layer", seed=4)
    assert torch.equal(a.q, b.q) and torch.equal(a.h0, b.h0)
    np.testing.assert_array_equal(a.lat_tok, b.lat_tok)
    assert not torch.equal(a.q, c.q)


def test_ragged_top1_range():
    w = generate("ragged", seed=0, B=8)
    assert ((w.p_top1 >= 0.6) & (w.p_top1 <= 0.95)).all()
    assert len(set(w.p_top1.tolist())) == 8


def test_resolve_target():
    lat_tok = np.arange(2 * 3, dtype=np.int32).reshape(1, 2, 3) + 100
    depth = np.array([[0, 1, 1, 2, -1]])
    choice = np.array([[1, 0, 3, 2, 0]], np.int32)
    uni = np.array([[7, 8, 9, 10, 11]], np.int32)
    t = resolve_target(depth, np.array([4]), lat_tok, choice, uni)
    # slot 0: depth 0, rank 1 -> lat_tok[0][1]; slot 1: depth 1, rank 0 -> lat_tok[1][0];
    # slot 2: uniform choice; slot 3: depth 2 == P -> uniform; slot 4 unused -> uniform
    assert t.tolist() == [[101, 103, 9, 10, 11]]


def test_error_reduction_reports_nan_as_failure():
    """A NaN GPU result must fail the parity bar, not vanish in a max()."""
    import numpy as np
    from tests.gpu_harness import worst
    assert worst([np.array([1e-4, 2e-4]), np.array([3e-4])]) == 3e-4
    assert worst([np.array([1e-4, np.nan])]) == float("inf")
