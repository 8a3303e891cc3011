"""Helpers for GPU parity tests: run the HIP path and the oracle on the same inputs and
compare them to the stated bars (bit-exact trees / acceptance; states and outputs within
2e-3 of the fp64 state's Frobenius norm)."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import torch

import oracle
from workloads import CONFIGS, generate, resolve_target

TOL = 2e-3


def slice_workload(w, H=None, B=None, L=None):
    """A sub-workload with the first H heads / B requests / L layers (heads, requests and
    layers are independent, so this is plumbing, not arithmetic)."""
    H = H or w.cfg.H
    B = B or w.cfg.B
    L = L or w.cfg.L
    sl5 = (slice(0, L), slice(0, B), slice(None), slice(0, H))
    w2 = replace(w, cfg=replace(w.cfg, H=H, B=B, L=L),
                 lat_logp=w.lat_logp[:B].copy(), lat_tok=w.lat_tok[:B].copy(), root_tok=w.root_tok[:B].copy(),
                 p_top1=w.p_top1[:B].copy(), tgt_choice=w.tgt_choice[:B].copy(),
                 tgt_uniform=w.tgt_uniform[:B].copy(),
                 q=w.q[sl5].contiguous(), k=w.k[sl5].contiguous(), v=w.v[sl5].contiguous(),
                 alpha=w.alpha[sl5].contiguous(), beta=w.beta[sl5].contiguous(),
                 h0=w.h0[:L, :B, :H].contiguous())
    return w2


def device_inputs(w, dev="cuda"):
    import gdn_draft_tree_amd as g
    return dict(
        lat_logp=torch.from_numpy(w.lat_logp).to(dev), lat_tok=torch.from_numpy(w.lat_tok).to(dev),
        root_tok=torch.from_numpy(w.root_tok).to(dev),
        q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev), alpha=w.alpha.to(dev), beta=w.beta.to(dev),
        state=w.h0.to(dev))


def run_gpu(w, out_dtype=None, d=None, split=False, shared=None):
    """build -> verify -> (host: synthetic target from the built tree) -> accept_commit, or
    with split=True accept -> commit (the two-call form).  shared=(G, positions or None)
    builds the trees under a batch budget of G draft nodes."""
    import gdn_draft_tree_amd as g
    d = d or device_inputs(w)
    if shared is None:
        tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N)
    else:
        G, positions = shared
        pos = None if positions is None else torch.tensor(np.asarray(positions, np.int32)).cuda()
        tree = g.gdntree_build_shared(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N, G, pos)
    L, B, R, Hh, D = w.q.shape
    # zero-filled, so that converting the whole buffer never reads slots the kernel leaves alone
    o = torch.zeros(L, B, R, Hh, D, dtype=out_dtype or d["q"].dtype, device=d["q"].device)
    g.gdntree_verify(tree, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], o=o, out_dtype=out_dtype)
    torch.cuda.synchronize()
    depth = tree.depth.cpu().numpy()
    n_nodes = tree.n_nodes.cpu().numpy()
    target = resolve_target(depth, n_nodes, w.lat_tok, w.tgt_choice, w.tgt_uniform)
    if split:
        acc = g.gdntree_accept(tree, torch.from_numpy(target).cuda(), w.cfg.P)
        g.gdntree_commit(tree, acc[0], acc[2], d["k"], d["v"], d["alpha"], d["beta"], d["state"], w.cfg.P)
    else:
        acc = g.gdntree_accept_commit(tree, torch.from_numpy(target).cuda(), d["k"], d["v"], d["alpha"],
                                      d["beta"], d["state"], w.cfg.P)
    torch.cuda.synchronize()
    return dict(tree={f: getattr(tree, f).cpu().numpy() for f in
                      ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")},
                o=o.float().cpu().numpy().astype(np.float64), target=target,
                acc_len=acc[0].cpu().numpy(), acc_tok=acc[1].cpu().numpy(), acc_node=acc[2].cpu().numpy(),
                state=d["state"].cpu().numpy().astype(np.float64))


def run_oracle(w, shared=None):
    def target_fn(tree):
        return resolve_target(tree["depth"], tree["n_nodes"], w.lat_tok, w.tgt_choice, w.tgt_uniform)
    G, positions = shared if shared is not None else (None, None)
    return oracle.pipeline(w.lat_logp, w.lat_tok, w.root_tok, w.cfg.N, w.f64("q"), w.f64("k"), w.f64("v"),
                           w.f64("alpha"), w.f64("beta"), w.h0.double().numpy(), target_fn, G=G,
                           positions=positions)


def assert_tree_equal(gt, ot):
    np.testing.assert_array_equal(gt["n_nodes"], ot["n_nodes"])
    for b in range(len(ot["n_nodes"])):
        n = int(ot["n_nodes"][b])
        for f in ("parent", "depth", "rank", "token"):
            np.testing.assert_array_equal(gt[f][b, :n], ot[f][b, :n], err_msg=f"{f} b={b}")
        assert gt["score"][b, :n].tobytes() == ot["score"][b, :n].tobytes(), f"score bits b={b}"
        np.testing.assert_array_equal(gt["anc"][b, :n].view(np.uint64), ot["anc"][b, :n], err_msg=f"anc b={b}")


def worst(errs) -> float:
    """The largest error, with any NaN (a non-finite GPU result) reported as +inf: Python's
    max() would silently skip it."""
    a = np.asarray([np.max(e) for e in errs], dtype=np.float64)
    return float("inf") if np.isnan(a).any() else float(a.max())


def output_errors(g_o, o_ref, hnorm, n_nodes):
    """max over channels of |o_gpu - o_ref| / ||S_ref(t)||_F for every used (l, b, t, h)."""
    errs = []
    for b, n in enumerate(n_nodes):
        n = int(n)
        errs.append(np.abs(g_o[:, b, :n] - o_ref[:, b, :n]).max(-1) / hnorm[:, b, :n])
    return worst(errs)


def state_errors(g_s, s_ref):
    num = np.abs(g_s - s_ref).max(axis=(-2, -1))
    den = np.sqrt((s_ref ** 2).sum(axis=(-2, -1)))
    return worst([num / den])


def check_all(w, out_dtype=None, gpu=None, ref=None, shared=None):
    gpu = gpu or run_gpu(w, out_dtype=out_dtype, shared=shared)
    ref = ref or run_oracle(w, shared=shared)
    assert_tree_equal(gpu["tree"], ref["tree"])
    np.testing.assert_array_equal(gpu["target"], ref["target"])
    oe = output_errors(gpu["o"], ref["o"], ref["hnorm"], ref["tree"]["n_nodes"])
    assert oe <= TOL, f"output error {oe:.3e} > {TOL}"
    np.testing.assert_array_equal(gpu["acc_len"], ref["acc_len"])
    np.testing.assert_array_equal(gpu["acc_tok"], ref["acc_tok"])
    np.testing.assert_array_equal(gpu["acc_node"], ref["acc_node"])
    se = state_errors(gpu["state"], ref["state"])
    assert se <= TOL, f"committed state error {se:.3e} > {TOL}"
    return dict(out_err=oe, state_err=se, gpu=gpu, ref=ref)


def config(name):
    return CONFIGS[name]


def make(name, seed=0, **kw):
    return generate(name, seed=seed, **kw)


# ---------------------------------------------------------------------------------------------
# The oracle on every unit of a full-size configuration, in worker processes (spawned, so that
# no GPU state is inherited; each regenerates the seeded workload itself).
_UNIT_CACHE: dict = {}


def _oracle_unit(job):
    """Worker: the oracle's pipeline on request b, layers [l0, l1), of a generated workload.
    Returns the tree, acceptance, outputs, state norms and committed states of that request."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import generate as gen
    from workloads import resolve_target as rt
    name, seed, b, l0, l1, scale_h0 = job
    key = (name, seed)
    if key not in _UNIT_CACHE:
        _UNIT_CACHE.clear()
        _UNIT_CACHE[key] = gen(name, seed=seed)
    w = _UNIT_CACHE[key]
    sl, ll = slice(b, b + 1), slice(l0, l1)
    x = {f: getattr(w, f)[ll, sl].to(torch.float64).numpy() for f in ("q", "k", "v", "alpha", "beta")}
    h0 = w.h0[ll, sl].double().numpy() * scale_h0
    lat_tok, tch, tun = w.lat_tok[sl], w.tgt_choice[sl], w.tgt_uniform[sl]
    with threadpool_limits(limits=1):
        r = oracle.pipeline(w.lat_logp[sl], lat_tok, w.root_tok[sl], w.cfg.N, x["q"], x["k"], x["v"], x["alpha"],
                            x["beta"], h0, lambda t: rt(t["depth"], t["n_nodes"], lat_tok, tch, tun))
    return dict(tree={k: v[0] for k, v in r["tree"].items()}, target=r["target"][0], acc_len=r["acc_len"][0],
                acc_tok=r["acc_tok"][0], acc_node=r["acc_node"][0], o=r["o"][:, 0].astype(np.float32),
                hnorm=r["hnorm"][:, 0], state=r["state"][:, 0].astype(np.float32),
                state_norm=np.sqrt((r["state"][:, 0] ** 2).sum(axis=(-2, -1))))


def oracle_every_unit(name, seed=0, scale_h0=1.0, workers=None):
    """The oracle on every request (and every layer) of a full configuration, one request per
    task over up to 16 spawned worker processes.  Returns per-request results."""
    import multiprocessing as mp
    import os
    B, L = CONFIGS[name].B, CONFIGS[name].L
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    lchunk = max(1, -(-L * B // workers) // B) if B < workers else L   # split layers when requests are few
    jobs = [(name, seed, b, l0, min(L, l0 + lchunk), scale_h0) for b in range(B) for l0 in range(0, L, lchunk)]
    with mp.get_context("spawn").Pool(min(workers, len(jobs))) as pool:
        parts = pool.map(_oracle_unit, jobs, chunksize=1)
    out = []
    for b in range(B):   # layers of one request back together
        ps = [p for j, p in zip(jobs, parts) if j[2] == b]
        r = dict(ps[0])
        for f in ("o", "hnorm", "state", "state_norm"):
            r[f] = np.concatenate([p[f] for p in ps], axis=0)
        out.append(r)
    return out


def check_every_unit(gpu, refs):
    """Trees, targets and acceptance bit-exact for every request; outputs and committed states
    of every (layer, request, head) within the bar.  Returns (out_err, state_err)."""
    errs_o, errs_s = [], []
    for b, r in enumerate(refs):
        n = int(r["tree"]["n_nodes"])
        for f in ("parent", "depth", "rank", "token"):
            np.testing.assert_array_equal(gpu["tree"][f][b, :n], r["tree"][f][:n], err_msg=f"{f} b={b}")
        assert gpu["tree"]["score"][b, :n].tobytes() == r["tree"]["score"][:n].tobytes(), f"score b={b}"
        np.testing.assert_array_equal(gpu["tree"]["anc"][b, :n].view(np.uint64), r["tree"]["anc"][:n])
        np.testing.assert_array_equal(gpu["target"][b], r["target"])
        assert int(gpu["acc_len"][b]) == int(r["acc_len"]), f"tau b={b}"
        np.testing.assert_array_equal(gpu["acc_tok"][b], r["acc_tok"])
        np.testing.assert_array_equal(gpu["acc_node"][b], r["acc_node"])
        errs_o.append(np.abs(gpu["o"][:, b, :n] - r["o"][:, :n]).max(-1) / r["hnorm"][:, :n])
        errs_s.append(np.abs(gpu["state"][:, b] - r["state"]).max(axis=(-2, -1)) / r["state_norm"])
    return worst(errs_o), worst(errs_s)
