"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.  Trees, targets and acceptance must be bit-exact; outputs and committed states
within 2e-3 of the fp64 state's Frobenius norm (max-abs error over value channels)."""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

from workloads import CONFIGS, Config, generate

from . import gpu_harness as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def test_tiny_full():
    w = generate("tiny", seed=0)
    r = H.check_all(w)
    _say(f"tiny: out_err={r['out_err']:.2e} state_err={r['state_err']:.2e} tau={r['gpu']['acc_len']}")


@pytest.mark.parametrize("name,seed,heads,reqs,layers", [
    ("one_layer", 0, None, None, None),     # 32 heads -> 1-wave workgroups, 4 slices per head
    ("one_layer", 1, None, None, None),
    ("batched", 0, 8, None, None),          # 192 heads -> 2-wave workgroups
    ("batched", 1, 16, None, None),         # 384 heads -> 4-wave workgroups
    ("ragged", 0, 4, None, None),           # N = 64: 65 rows, a ragged last node tile
    ("ragged", 2, 8, 16, None),
    ("deep", 0, 2, None, 48),               # 48 layers share one tree
    ("ragged", 3, None, 24, None),          # 768 heads: more than one head per workgroup
])
def test_configs(name, seed, heads, reqs, layers):
    w = generate(name, seed=seed, B=reqs)
    w = H.slice_workload(w, H=heads, L=layers)
    r = H.check_all(w)
    _say(f"{name} seed={seed} H={w.cfg.H} B={w.cfg.B} L={w.cfg.L}: out_err={r['out_err']:.2e} "
         f"state_err={r['state_err']:.2e} tau={r['gpu']['acc_len'].tolist()}")


@pytest.mark.parametrize("name", ["one_layer", "batched", "ragged", "deep"])
def test_full_size_every_unit(name):
    """Full configuration on the GPU in the bench's launch shape; the oracle (in worker
    processes) checks every (layer, request, head) unit: trees, targets and acceptance of every
    request bit-exact, every output row and committed state within the bar."""
    w = generate(name, seed=0)
    _say(f"{name} full size: GPU pipeline")
    gpu = H.run_gpu(w)
    _say(f"{name} full size: oracle on every unit")
    refs = H.oracle_every_unit(name, seed=0)
    oe, se = H.check_every_unit(gpu, refs)
    _say(f"{name} full size, every unit: out_err={oe:.2e} state_err={se:.2e}")
    assert oe <= H.TOL and se <= H.TOL


@pytest.mark.parametrize("scale", [100.0, 1e-4])
def test_state_scale_far_from_the_rows(scale):
    """A committed state 100x larger or 10^4x smaller than the rows' scale (v ~ N(0, 1)):
    the products stay exact at any scale, so the bar holds relative to each node state."""
    w = H.slice_workload(generate("ragged", seed=4, B=6), H=4)
    w.h0.mul_(scale)
    r = H.check_all(w)
    _say(f"h0 x {scale:g}: out_err={r['out_err']:.2e} state_err={r['state_err']:.2e}")


def test_full_size_state_scaled_up():
    """Every unit of the ragged batch with the committed state 100x larger."""
    w = generate("ragged", seed=1)
    w.h0.mul_(100.0)
    gpu = H.run_gpu(w)
    refs = H.oracle_every_unit("ragged", seed=1, scale_h0=100.0)
    oe, se = H.check_every_unit(gpu, refs)
    _say(f"ragged x100 every unit: out_err={oe:.2e} state_err={se:.2e}")
    assert oe <= H.TOL and se <= H.TOL


@pytest.mark.parametrize("name,heads", [("ragged", 4), ("batched", 8)])
def test_pipelined_steps(name, heads):
    """Four decode steps run as the bench runs them (verify(i), then acceptance + commit of
    step i with the build of step i+1 in one launch, then verify(i+1) on the committed
    states): every step's trees, outputs, acceptance and committed states against the oracle's
    pipeline, each step starting from the oracle's previous committed state."""
    import gdn_draft_tree_amd as g
    import oracle
    from workloads import resolve_target
    steps = [H.slice_workload(generate(name, seed=20 + i, B=8), H=heads) for i in range(4)]
    w0 = steps[0]
    d = [H.device_inputs(w) for w in steps]
    state = d[0]["state"]                     # the committed state carried across steps
    h_ref = w0.h0.double().numpy()
    trees = [g.gdntree_build(d[0]["lat_logp"], d[0]["lat_tok"], d[0]["root_tok"], w0.cfg.N)]
    for i, w in enumerate(steps):
        tree = trees[i]
        o = torch.zeros_like(d[i]["q"])
        g.gdntree_verify(tree, d[i]["q"], d[i]["k"], d[i]["v"], d[i]["alpha"], d[i]["beta"], state, o=o)
        torch.cuda.synchronize()
        depth, nn = tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy()
        target = torch.from_numpy(resolve_target(depth, nn, w.lat_tok, w.tgt_choice, w.tgt_uniform)).cuda()
        if i + 1 < len(steps):
            nxt = g.Tree.empty(w.cfg.B, w.cfg.N, "cuda")
            acc = g.gdntree_accept_commit_build(tree, target, d[i]["k"], d[i]["v"], d[i]["alpha"], d[i]["beta"],
                                                state, w.cfg.P, d[i + 1]["lat_logp"], d[i + 1]["lat_tok"],
                                                d[i + 1]["root_tok"], w.cfg.N, nxt)
            trees.append(nxt)
        else:
            acc = g.gdntree_accept_commit(tree, target, d[i]["k"], d[i]["v"], d[i]["alpha"], d[i]["beta"], state,
                                          w.cfg.P)
        torch.cuda.synchronize()
        ref = oracle.pipeline(w.lat_logp, w.lat_tok, w.root_tok, w.cfg.N, w.f64("q"), w.f64("k"), w.f64("v"),
                              w.f64("alpha"), w.f64("beta"), h_ref,
                              lambda t: resolve_target(t["depth"], t["n_nodes"], w.lat_tok, w.tgt_choice,
                                                       w.tgt_uniform))
        H.assert_tree_equal({f: getattr(tree, f).cpu().numpy() for f in
                             ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")}, ref["tree"])
        oe = H.output_errors(o.float().cpu().numpy().astype(np.float64), ref["o"], ref["hnorm"],
                             ref["tree"]["n_nodes"])
        for x, y in zip(acc, (ref["acc_len"], ref["acc_tok"], ref["acc_node"])):
            np.testing.assert_array_equal(x.cpu().numpy(), y)
        se = H.state_errors(state.cpu().numpy().astype(np.float64), ref["state"])
        _say(f"{name} step {i}: out_err={oe:.2e} state_err={se:.2e} tau={ref['acc_len'].tolist()}")
        assert oe <= H.TOL and se <= H.TOL
        h_ref = ref["state"]                   # the next step starts from the oracle's commit


def test_nan_gate_is_confined_to_its_head():
    """A NaN decay gate at one used slot of one (layer, request, head) stays in that head: every
    other (layer, request, head) gives the oracle's outputs and committed state.  (Inside the head
    the per-node sum is one dense product over the head's nodes, so the NaN reaches every node of
    that head; the oracle's NaNs are the slot's subtree, which the GPU's must cover.)"""
    import oracle
    w = _custom(P=16, K=16, N=64, B=4, H_=4, L=2, seed=6)
    tree = oracle.build_tree(w.lat_logp, w.lat_tok, w.root_tok, w.cfg.N)
    l0, b0, h0_, slot = 1, 2, 3, 5
    w.alpha[l0, b0, slot, h0_] = float("nan")
    gpu = H.run_gpu(w)
    ref = H.run_oracle(w)
    H.assert_tree_equal(gpu["tree"], ref["tree"])
    n = int(tree["n_nodes"][b0])
    anc = tree["anc"][b0].astype(np.uint64)
    sub = [t for t in range(n) if (int(anc[t]) >> (slot - 1)) & 1]   # the slot's subtree
    assert slot in sub
    used = np.zeros(gpu["o"].shape[:4], bool)
    for b, nb in enumerate(ref["tree"]["n_nodes"]):
        used[:, b, :int(nb)] = True
    ok = used.copy()
    ok[l0, b0, :, h0_] = False                                         # every other head
    err = np.abs(gpu["o"] - ref["o"]).max(-1)[ok] / ref["hnorm"][ok]
    assert np.isfinite(gpu["o"][ok]).all() and err.max() <= H.TOL, err.max()
    assert np.isnan(gpu["o"][l0, b0, sub, h0_]).all()                  # the oracle's NaNs are NaN
    # committed states: every other head within the bar; the affected head NaN only if the
    # accepted path went through the slot
    se = np.abs(gpu["state"] - ref["state"]).max(axis=(-2, -1)) / np.sqrt((ref["state"] ** 2).sum(axis=(-2, -1)))
    mask = np.ones(se.shape, bool)
    mask[l0, b0, h0_] = False
    assert np.isfinite(se[mask]).all() and se[mask].max() <= H.TOL
    on_path = slot in ref["acc_node"][b0, :int(ref["acc_len"][b0])].tolist()
    assert np.isnan(gpu["state"][l0, b0, h0_]).any() == on_path
    _say(f"NaN gate at (l={l0}, b={b0}, h={h0_}, slot {slot}): other heads out_err={err.max():.2e}, "
         f"state on the accepted path: {on_path}")


def _custom(P, K, N, B=2, H_=2, D=128, dtype="bf16", L=1, seed=0, V=1000):
    cfg = Config("custom", B=B, L=L, H=H_, D=D, dtype=dtype, P=P, K=K, V=V, N=N)
    return generate(cfg, seed=seed)


def test_uniform_lattice_ties():
    """Every candidate tied: the tie-break (parent slot, then rank) decides the whole tree."""
    w = _custom(P=4, K=4, N=64)
    w.lat_logp[:] = np.float32(-math.log(4))
    H.check_all(w)


def test_k1_chain_and_exhausted_trie():
    H.check_all(_custom(P=16, K=1, N=24))          # chain of 16, n = 17 < N + 1
    H.check_all(_custom(P=2, K=3, N=64, B=3))       # 12-node trie, n = 13


def test_minus_inf_log_probs():
    """Masked (-inf) candidates, and finite log-probs whose fp64 sums round to -inf in fp32:
    trees bit-exact against the oracle, per request and under batch budgets, then the whole
    pipeline on them."""
    w = _custom(P=3, K=4, N=64, B=3)  # tries of 84 nodes
    rng = np.random.default_rng(5)
    w.lat_logp[0, :, 2:] = -np.inf
    w.lat_logp[1, 1, 1:] = -np.inf
    w.lat_logp[2] = -np.sort(rng.uniform(1e38, 3.4e38, size=(3, 4)), axis=-1).astype(np.float32)
    H.check_all(w)
    for G in (20, 100, 180):
        _say(f"-inf lattices under a budget of {G}")
        H.check_all(w, shared=(G, None))


def test_deep_chain_tau_17():
    """A peaked lattice and a target that always agrees with rank 0: depth 16, tau = 17."""
    w = _custom(P=16, K=16, N=64, B=2, H_=4)
    logp = w.lat_logp.astype(np.float64)
    logp[..., 0] = -1e-4
    logp[..., 1:] -= 20.0
    w.lat_logp[:] = np.sort(logp, axis=-1)[..., ::-1].astype(np.float32)
    w.tgt_choice[:] = 0
    r = H.check_all(w)
    assert (r["gpu"]["acc_len"] == 17).all()


def test_poisoned_unused_slots():
    """Slots at or beyond n_nodes hold NaN inputs and a sentinel output; neither may leak."""
    import gdn_draft_tree_amd as g
    w = _custom(P=2, K=3, N=40, B=2, H_=3)           # n = 13 of 41 slots
    n = 13
    for name in ("q", "k", "v", "alpha", "beta"):
        getattr(w, name)[:, :, n:] = float("nan")
    d = H.device_inputs(w)
    o = torch.full((1, 2, 41, 3, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N)
    g.gdntree_verify(tree, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], o=o)
    torch.cuda.synchronize()
    assert int(tree.n_nodes.cpu()[0]) == n
    oc = o.float().cpu()
    assert torch.isfinite(oc[:, :, :n]).all()
    assert (oc[:, :, n:] == 7.0).all()
    H.check_all(w)


@pytest.mark.parametrize("D,dtype,out", [(64, "bf16", None), (128, "f32", None), (64, "f32", None),
                                         (128, "bf16", torch.float32)])
def test_dtypes_and_head_dims(D, dtype, out):
    w = _custom(P=8, K=16, N=64, B=3, H_=4, D=D, dtype=dtype)
    H.check_all(w, out_dtype=out)


def test_layers_and_requests():
    H.check_all(_custom(P=8, K=8, N=24, B=5, H_=3, L=4, seed=3))


def test_determinism_and_launch_shape_independence():
    """Same inputs give bitwise-identical outputs run to run, and a request's outputs do not
    depend on the launch shape (1-wave vs 4-wave workgroups, chosen by the head count)."""
    import gdn_draft_tree_amd as g
    w1 = _custom(P=8, K=16, N=64, B=1, H_=8, seed=5)
    d1 = H.device_inputs(w1)
    t1 = g.gdntree_build(d1["lat_logp"], d1["lat_tok"], d1["root_tok"], 64)
    o1 = g.gdntree_verify(t1, d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], d1["state"])
    o1b = g.gdntree_verify(t1, d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], d1["state"])
    # 32 copies of the request: 256 heads -> 4-wave workgroups
    rep = lambda x: x.repeat_interleave(32, dim=1) if x.dim() >= 2 else x
    d32 = {k_: (rep(v_) if k_ in ("q", "k", "v", "alpha", "beta", "state") else v_) for k_, v_ in d1.items()}
    d32["lat_logp"] = d1["lat_logp"].repeat(32, 1, 1)
    d32["lat_tok"] = d1["lat_tok"].repeat(32, 1, 1)
    d32["root_tok"] = d1["root_tok"].repeat(32)
    t32 = g.gdntree_build(d32["lat_logp"], d32["lat_tok"], d32["root_tok"], 64)
    o32 = g.gdntree_verify(t32, d32["q"].contiguous(), d32["k"].contiguous(), d32["v"].contiguous(),
                           d32["alpha"].contiguous(), d32["beta"].contiguous(), d32["state"].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o1b.view(torch.int16))
    for b in (0, 17, 31):
        assert torch.equal(o32[:, b].view(torch.int16), o1[:, 0].view(torch.int16))


def test_malformed_tree_is_contained():
    """A parent link that is not smaller than its child gives NaN outputs for that request
    only; an out-of-range node count leaves that request's outputs untouched."""
    import gdn_draft_tree_amd as g
    w = _custom(P=4, K=4, N=8, B=3, H_=2)
    d = H.device_inputs(w)
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], 8)
    torch.cuda.synchronize()
    tree.parent[1, 5] = 7
    tree.n_nodes[2] = 99
    o = torch.full((1, 3, 9, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    g.gdntree_verify(tree, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], o=o)
    torch.cuda.synchronize()
    oc = o.float().cpu()
    assert torch.isfinite(oc[:, 0]).all()
    assert torch.isnan(oc[:, 1]).all()
    assert (oc[:, 2] == 3.0).all()


@pytest.mark.parametrize("name,seed,heads,reqs,layers", [
    ("tiny", 0, None, None, None),
    ("ragged", 1, 4, 8, None),
    ("deep", 1, 2, None, 6),
])
def test_split_accept_then_commit(name, seed, heads, reqs, layers):
    """gdntree_accept then gdntree_commit give exactly what gdntree_accept_commit gives (the
    same fp32 arithmetic, bitwise), and so match the oracle."""
    w = H.slice_workload(generate(name, seed=seed, B=reqs), H=heads, L=layers)
    fused = H.run_gpu(w)
    split = H.run_gpu(w, split=True)
    for f in ("acc_len", "acc_tok", "acc_node"):
        np.testing.assert_array_equal(split[f], fused[f])
    assert np.array_equal(split["state"], fused["state"])
    r = H.check_all(w, gpu=split)
    _say(f"split {name}: state_err={r['state_err']:.2e} tau={split['acc_len'].tolist()}")


def test_commit_keeps_state_on_a_bad_path():
    """gdntree_commit leaves a request's state untouched when its path is not a root path of
    its tree (a slot outside the node count, tau 0, a first slot other than the root, a slot
    that is not a child of the previous one) and commits the others."""
    import gdn_draft_tree_amd as g
    from workloads import resolve_target
    w = _custom(P=4, K=4, N=8, B=5, H_=2)
    d = H.device_inputs(w)
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], 8)
    torch.cuda.synchronize()
    depth = tree.depth.cpu().numpy()
    target = resolve_target(depth, tree.n_nodes.cpu().numpy(), w.lat_tok, w.tgt_choice, w.tgt_uniform)
    tgt = torch.from_numpy(target).cuda()
    s_ref = d["state"].clone()
    acc_ref = g.gdntree_accept_commit(tree, tgt, d["k"], d["v"], d["alpha"], d["beta"], s_ref, 4)
    acc_len, acc_tok, acc_node = g.gdntree_accept(tree, tgt, 4)
    torch.cuda.synchronize()
    assert torch.equal(acc_len, acc_ref[0]) and torch.equal(acc_node, acc_ref[2])
    acc_len, acc_node = acc_len.clone(), acc_node.clone()
    acc_node[1, 1] = 99; acc_len[1] = 2                      # slot outside the node count
    acc_len[2] = 0                                           # tau 0
    acc_node[3, 0] = 1                                       # first slot not the root
    deep = [t for t in range(1, 9) if depth[4, t] == 2]      # a slot that is not a child of the root
    assert deep, "the seeded tree has a depth-2 node"
    acc_node[4, 1] = deep[0]; acc_len[4] = 2
    s0 = d["state"].clone()
    g.gdntree_commit(tree, acc_len, acc_node, d["k"], d["v"], d["alpha"], d["beta"], d["state"], 4)
    torch.cuda.synchronize()
    assert torch.equal(d["state"][:, 0], s_ref[:, 0])
    for b in (1, 2, 3, 4):
        assert torch.equal(d["state"][:, b], s0[:, b]), b


@pytest.mark.parametrize("cur,nxt", [
    (dict(P=8, K=16, N=64, B=3, H_=4), dict(P=16, K=16, N=64, B=5, seed=7)),
    (dict(P=4, K=4, N=8, B=2, H_=2, D=64, dtype="f32"), dict(P=8, K=8, N=24, B=1, seed=3)),
])
def test_commit_build_equals_the_two_calls(cur, nxt):
    """One launch of commit + next build gives bitwise what gdntree_commit and gdntree_build
    give separately (and the next tree equals the oracle's)."""
    import gdn_draft_tree_amd as g
    import oracle
    from workloads import resolve_target
    w = _custom(**cur)
    wn = _custom(**nxt)
    d = H.device_inputs(w)
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N)
    torch.cuda.synchronize()
    target = resolve_target(tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy(), w.lat_tok, w.tgt_choice,
                            w.tgt_uniform)
    acc = g.gdntree_accept(tree, torch.from_numpy(target).cuda(), w.cfg.P)
    s_sep = d["state"].clone()
    g.gdntree_commit(tree, acc[0], acc[2], d["k"], d["v"], d["alpha"], d["beta"], s_sep, w.cfg.P)
    nl = (torch.from_numpy(wn.lat_logp).cuda(), torch.from_numpy(wn.lat_tok).cuda(), torch.from_numpy(wn.root_tok).cuda())
    t_sep = g.gdntree_build(*nl, wn.cfg.N)
    t_fused = g.Tree.empty(wn.cfg.B, wn.cfg.N, "cuda")
    g.gdntree_commit_build(tree, acc[0], acc[2], d["k"], d["v"], d["alpha"], d["beta"], d["state"], w.cfg.P,
                           *nl, wn.cfg.N, t_fused)
    torch.cuda.synchronize()
    assert torch.equal(d["state"], s_sep)
    fields = ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")
    fused = {f: getattr(t_fused, f).cpu().numpy() for f in fields}
    sep = {f: getattr(t_sep, f).cpu().numpy() for f in fields}
    sep["anc"] = sep["anc"].view(np.uint64)
    H.assert_tree_equal(fused, sep)                          # used slots, scores bitwise
    H.assert_tree_equal(fused, oracle.build_tree(wn.lat_logp, wn.lat_tok, wn.root_tok, wn.cfg.N))


def test_prepared_calls_equal_direct_calls():
    """A call prepared once (binding's prepare=True) and enqueued twice gives bitwise what the
    direct calls give."""
    import gdn_draft_tree_amd as g
    w = _custom(P=8, K=16, N=64, B=2, H_=3, seed=11)
    d = H.device_inputs(w)
    t_direct = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], 64)
    o_direct = g.gdntree_verify(t_direct, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"])
    t_prep = g.Tree.empty(2, 64, "cuda")
    o_prep = torch.empty_like(o_direct)
    pb = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], 64, out=t_prep, prepare=True)
    pv = g.gdntree_verify(t_prep, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], o=o_prep, prepare=True)
    for _ in range(2):
        o_prep.fill_(0)
        pb()
        pv()
        torch.cuda.synchronize()
        assert torch.equal(t_prep.parent, t_direct.parent) and torch.equal(t_prep.anc, t_direct.anc)
        assert torch.equal(o_prep.view(torch.int16), o_direct.view(torch.int16))


@pytest.mark.parametrize("cur,nxt", [
    (dict(P=8, K=16, N=64, B=3, H_=4), dict(P=16, K=16, N=64, B=5, seed=7)),   # more next requests
    (dict(P=16, K=16, N=64, B=6, H_=2), dict(P=8, K=16, N=24, B=2, seed=9)),   # fewer next requests
    (dict(P=4, K=4, N=8, B=2, H_=2, D=64, dtype="f32"), dict(P=8, K=8, N=24, B=2, seed=3)),
])
def test_accept_commit_build_equals_the_two_calls(cur, nxt):
    """Acceptance, commit and the next build in one launch give bitwise what
    gdntree_accept_commit and gdntree_build give separately."""
    import gdn_draft_tree_amd as g
    from workloads import resolve_target
    w = _custom(**cur)
    wn = _custom(**nxt)
    d = H.device_inputs(w)
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N)
    torch.cuda.synchronize()
    target = torch.from_numpy(resolve_target(tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy(), w.lat_tok,
                                             w.tgt_choice, w.tgt_uniform)).cuda()
    s_sep = d["state"].clone()
    acc_sep = g.gdntree_accept_commit(tree, target, d["k"], d["v"], d["alpha"], d["beta"], s_sep, w.cfg.P)
    nl = (torch.from_numpy(wn.lat_logp).cuda(), torch.from_numpy(wn.lat_tok).cuda(), torch.from_numpy(wn.root_tok).cuda())
    t_sep = g.gdntree_build(*nl, wn.cfg.N)
    t_fused = g.Tree.empty(wn.cfg.B, wn.cfg.N, "cuda")
    acc = tuple(torch.full_like(x, -7) for x in acc_sep)
    g.gdntree_accept_commit_build(tree, target, d["k"], d["v"], d["alpha"], d["beta"], d["state"], w.cfg.P,
                                  *nl, wn.cfg.N, t_fused, acc=acc)
    torch.cuda.synchronize()
    assert torch.equal(d["state"], s_sep)
    for x, y in zip(acc, acc_sep):
        assert torch.equal(x, y)
    fields = ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")
    fused = {f: getattr(t_fused, f).cpu().numpy() for f in fields}
    sep = {f: getattr(t_sep, f).cpu().numpy() for f in fields}
    sep["anc"] = sep["anc"].view(np.uint64)
    H.assert_tree_equal(fused, sep)


@pytest.mark.parametrize("name,B", [("ragged", 24), ("batched", 24)])
def test_repeated_launches_with_shared_cus(name, B):
    """Several launches over more units than resident workgroups (two or three share each
    CU, and a second round follows) give bitwise-identical outputs, every unit within the
    bar against the oracle.  Guards against schedule-dependent corruption that shows only
    when workgroups run side by side."""
    import gdn_draft_tree_amd as g
    w = generate(name, seed=3, B=B)
    ref = H.run_oracle(w)
    d = H.device_inputs(w)
    tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], w.cfg.N)
    outs = []
    for _ in range(3):
        o = g.gdntree_verify(tree, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"])
        torch.cuda.synchronize()
        outs.append(o)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    oe = H.output_errors(outs[0].float().cpu().numpy().astype(np.float64), ref["o"], ref["hnorm"],
                         ref["tree"]["n_nodes"])
    assert oe <= H.TOL, f"output error {oe:.3e}"
    _say(f"{name} B={B}: 3 launches identical, out_err={oe:.2e}")


@pytest.mark.parametrize("name,B,heads,G,positions", [
    ("ragged", 32, 2, 192, "16/12/8"),   # the batch budget of draft rows, positions per request
    ("ragged", 32, 2, 1500, None),       # a budget that leaves some requests at the cap
    ("batched", 24, 2, 200, None),
    ("batched", 24, 1, 0, None),         # roots only
    ("batched", 24, 1, 10 ** 6, "0/8/3"),  # no cut (no selection launch); zero positions
    ("ragged", 64, 1, 1000, None),       # 64 lists x 64 keys, the largest cut
    ("batched", 1, 1, 10, None),         # one request: no merge
    ("batched", 100, 1, 300, "8/5"),     # 100 requests (128 lists)
])
def test_build_shared_full_pipeline(name, B, heads, G, positions):
    """Shared-budget trees bit-exact against the oracle's batch-wide best-first pass; then
    verify, acceptance and commit over those trees against the oracle."""
    w = H.slice_workload(generate(replace(CONFIGS[name], B=B), seed=3), H=heads)
    pos = None
    if positions is not None:
        cyc = [int(x) for x in positions.split("/")]
        pos = [cyc[b % len(cyc)] for b in range(B)]
    _say(f"shared build: {name} B={B} H={heads} G={G} positions={positions}")
    r = H.check_all(w, shared=(G, pos))
    n = r["gpu"]["tree"]["n_nodes"]
    _say(f"  drafts per request {n.min() - 1}..{n.max() - 1}, total {int(n.sum()) - B}, "
         f"out_err={r['out_err']:.2e} state_err={r['state_err']:.2e}")


def test_build_shared_uniform_ties():
    """Every candidate tied in every request: the cross-request rule (smaller request first)
    and the in-request rule decide the whole allocation."""
    w = _custom(P=4, K=4, N=40, B=6)
    w.lat_logp[:] = np.float32(-math.log(4))
    for G in (5, 23, 100, 239):
        H.check_all(w, shared=(G, [4, 2, 3, 4, 1, 4]))


@pytest.mark.parametrize("name,N", [("ragged", 8), ("ragged", 32), ("batched", 16)])
def test_tau_replay_at_smaller_budgets(name, N):
    """The tau(N) replay (build and acceptance alone, a budget below the workload's N, the
    first N + 1 per-slot target draws) against the oracle: trees and acceptance bit-exact."""
    import oracle
    from workloads import resolve_target
    import gdn_draft_tree_amd as g
    w = generate(name, seed=5)
    lp, lt, rt = (torch.from_numpy(x).cuda() for x in (w.lat_logp, w.lat_tok, w.root_tok))
    tree = g.gdntree_build(lp, lt, rt, N)
    torch.cuda.synchronize()
    tgt = resolve_target(tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy(), w.lat_tok,
                         w.tgt_choice[:, :N + 1], w.tgt_uniform[:, :N + 1])
    acc = g.gdntree_accept(tree, torch.from_numpy(np.ascontiguousarray(tgt)).cuda(), w.cfg.P)
    torch.cuda.synchronize()
    ref = oracle.build_tree(w.lat_logp, w.lat_tok, w.root_tok, N)
    H.assert_tree_equal({f: getattr(tree, f).cpu().numpy() for f in
                         ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")}, ref)
    tgt_ref = resolve_target(ref["depth"], ref["n_nodes"], w.lat_tok, w.tgt_choice[:, :N + 1],
                             w.tgt_uniform[:, :N + 1])
    a_len, a_tok, a_node = oracle.accept(ref, tgt_ref, w.cfg.P)
    np.testing.assert_array_equal(acc[0].cpu().numpy(), a_len)
    np.testing.assert_array_equal(acc[1].cpu().numpy(), a_tok)
    np.testing.assert_array_equal(acc[2].cpu().numpy(), a_node)
    _say(f"{name} N={N}: mean tau {a_len.mean():.3f}")



@pytest.mark.parametrize("G,positions", [(192, "16/12/8"), (0, None), (10 ** 6, "4/16")])
def test_accept_commit_build_shared_equals_the_two_calls(G, positions):
    """Acceptance + commit + the next trees under a batch budget in one call equal
    gdntree_accept_commit then gdntree_build_shared, bitwise; the next trees equal the oracle's."""
    import oracle
    import gdn_draft_tree_amd as g
    cur = H.slice_workload(generate("ragged", seed=7), B=32, H=2)
    nxt = generate("ragged", seed=8)
    pos = None if positions is None else [int(x) for x in positions.split("/")]
    pos = None if pos is None else [pos[b % len(pos)] for b in range(32)]
    runs = []
    for fused in (True, False):
        d = H.device_inputs(cur)
        tree = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], cur.cfg.N)
        torch.cuda.synchronize()
        from workloads import resolve_target
        tgt = torch.from_numpy(resolve_target(tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy(), cur.lat_tok,
                                              cur.tgt_choice, cur.tgt_uniform)).cuda()
        nl = [torch.from_numpy(x).cuda() for x in (nxt.lat_logp, nxt.lat_tok, nxt.root_tok)]
        npos = None if pos is None else torch.tensor(pos, dtype=torch.int32).cuda()
        nout = g.Tree.empty(32, nxt.cfg.N, "cuda")
        if fused:
            acc = g.gdntree_accept_commit_build_shared(tree, tgt, d["k"], d["v"], d["alpha"], d["beta"], d["state"],
                                                       cur.cfg.P, *nl, nxt.cfg.N, G, nout, next_positions=npos)
        else:
            acc = g.gdntree_accept_commit(tree, tgt, d["k"], d["v"], d["alpha"], d["beta"], d["state"], cur.cfg.P)
            g.gdntree_build_shared(*nl, nxt.cfg.N, G, npos, out=nout)
        torch.cuda.synchronize()
        runs.append(dict(acc=[a.cpu().numpy() for a in acc], state=d["state"].cpu().numpy(),
                         tree={f: getattr(nout, f).cpu().numpy() for f in
                               ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")}))
    a, b = runs
    for x, y in zip(a["acc"], b["acc"]):
        np.testing.assert_array_equal(x, y)
    assert a["state"].tobytes() == b["state"].tobytes()
    ref = oracle.build_tree_shared(nxt.lat_logp, nxt.lat_tok, nxt.root_tok, nxt.cfg.N, G, pos)
    H.assert_tree_equal(a["tree"], ref)
    H.assert_tree_equal(b["tree"], ref)
    _say(f"fused shared build G={G}: drafts {int(ref['n_nodes'].sum()) - 32}")


# ---------------------------------------------------------------------------------------------
# Markov-head lattices: parent-conditioned edge log-probs and the build over them
# ---------------------------------------------------------------------------------------------
def _markov(name, seed, R, wdtype, B=None):
    """The config's lattice tokens and roots with seeded Markov-head inputs; the embeddings
    cast to the kernel's dtype (bf16 by round-to-nearest-even on the CPU): both sides consume
    the cast values."""
    import workloads
    cfg = CONFIGS[name] if B is None else replace(CONFIGS[name], B=B)
    w = generate(cfg, seed=seed)
    mh = workloads.markov_head(cfg, seed=seed, R=R)
    dt = torch.bfloat16 if wdtype == "bf16" else torch.float32
    W1 = torch.from_numpy(mh.W1).to(dt)
    W2 = torch.from_numpy(mh.W2).to(dt)
    return w, mh.bases, W1, W2


@pytest.mark.parametrize("name,R,wdtype", [("batched", 32, "f32"), ("ragged", 32, "bf16"), ("ragged", 64, "f32"),
                                           ("deep", 16, "bf16")])
def test_markov_edges_against_oracle(name, R, wdtype):
    """Edge log-probs of the Markov head against the oracle's fp64 values.  The kernel works in
    fp32 (an R-term dot product, a max-shifted log-sum-exp over K): the bar is 5e-5 absolute on
    log-probs of magnitude <= ~30, far above fp32 rounding (~1e-6) and far below any real error
    (a wrong previous token or candidate shifts entries by ~1)."""
    import oracle
    import gdn_draft_tree_amd as g
    w, bases, W1, W2 = _markov(name, 4, R, wdtype, B=1 if name == "deep" else 8)
    tok, root = w.lat_tok, w.root_tok
    gpu = g.gdntree_markov_edges(torch.from_numpy(bases).cuda(), torch.from_numpy(tok).cuda(),
                                 torch.from_numpy(root).cuda(), W1.cuda(), W2.cuda())
    torch.cuda.synchronize()
    ref = oracle.markov_edge_logp(bases, tok, root, W1.to(torch.float64).numpy(), W2.to(torch.float64).numpy())
    err = np.abs(gpu.cpu().numpy().astype(np.float64) - ref)
    _say(f"markov edges {name} R={R} {wdtype}: max |err| {err.max():.2e}, |value| <= {np.abs(ref).max():.1f}")
    assert np.all(np.isfinite(gpu.cpu().numpy()))
    assert err.max() <= 5e-5


def test_markov_edges_out_of_range_tokens():
    """A token id outside [0, V) reads an all-zero embedding row (on both the previous-token and
    the candidate side): the oracle over embeddings padded with zero rows at those ids agrees."""
    import oracle
    import gdn_draft_tree_amd as g
    w, bases, W1, W2 = _markov("batched", 1, 16, "f32", B=3)
    tok, root = w.lat_tok.copy(), w.root_tok.copy()
    V = W1.shape[0]
    tok[0, 2, 5] = V + 3     # a candidate, and the previous token of row 5 at position 3
    tok[1, 0, 0] = -7        # negative
    root[2] = V + 1          # the root
    gpu = g.gdntree_markov_edges(torch.from_numpy(bases).cuda(), torch.from_numpy(tok).cuda(),
                                 torch.from_numpy(root).cuda(), W1.cuda(), W2.cuda())
    torch.cuda.synchronize()
    pad = np.zeros((8, W1.shape[1]))
    W1p = np.concatenate([W1.double().numpy(), pad])   # ids V .. V+7 read zeros
    W2p = np.concatenate([W2.double().numpy(), pad])
    tok_o = tok.copy()
    tok_o[1, 0, 0] = V + 7   # the negative id, mapped to a zero row on the oracle side
    ref = oracle.markov_edge_logp(bases, tok_o, root, W1p, W2p)
    assert np.abs(gpu.cpu().numpy() - ref).max() <= 5e-5


def _check_build_cond(edge, tok, root, N):
    import oracle
    import gdn_draft_tree_amd as g
    tree = g.gdntree_build_cond(torch.from_numpy(edge).cuda(), torch.from_numpy(tok).cuda(),
                                torch.from_numpy(root).cuda(), N)
    torch.cuda.synchronize()
    got = {f: getattr(tree, f).cpu().numpy() for f in ("parent", "depth", "rank", "token", "score", "anc", "n_nodes")}
    H.assert_tree_equal(got, oracle.build_tree_cond(edge, tok, root, N))
    return got


@pytest.mark.parametrize("name,N", [("ragged", 64), ("batched", 24), ("deep", 64), ("ragged", 17)])
def test_build_cond_markov_rows(name, N):
    """Trees over Markov-head edge log-probs (the oracle's values, cast to fp32: the input both
    sides build from) bit-exact against the oracle: topology, tokens, scores, masks."""
    import oracle
    w, bases, W1, W2 = _markov(name, 6, 32, "f32", B=1 if name == "deep" else 12)
    edge = oracle.markov_edge_logp(bases, w.lat_tok, w.root_tok, W1.double().numpy(),
                                   W2.double().numpy()).astype(np.float32)
    got = _check_build_cond(edge, w.lat_tok, w.root_tok, N)
    _say(f"build_cond {name} N={N}: nodes {got['n_nodes'].min()}..{got['n_nodes'].max()}, "
         f"max depth {got['depth'].max()}")


def test_build_cond_unsorted_ties_and_minus_inf():
    """Rows in no order (the kernel sorts each (position, parent rank) row), rows of equal
    values (the tie rule alone), -inf entries (candidates like any other) and a trie smaller
    than the budget."""
    rng = np.random.default_rng(11)
    B, P, K, N = 4, 5, 6, 64
    logits = rng.normal(0, 2, size=(B, P, K, K))
    edge = (logits - np.log(np.exp(logits).sum(-1, keepdims=True))).astype(np.float32)
    edge[1] = np.float32(-math.log(K))                 # every edge tied
    edge[2, :, :, 3:] = -np.inf                        # half of every row masked
    edge[3, 2, 1:, :] = -np.inf                        # rows of position 2 masked but for parent rank 0
    tok = rng.integers(0, 5000, size=(B, P, K)).astype(np.int32)
    root = rng.integers(0, 5000, size=B).astype(np.int32)
    _check_build_cond(edge, tok, root, N)
    _check_build_cond(edge[:, :2, :, :].copy(), tok[:, :2].copy(), root, N)  # 6 + 36 = 42 nodes < 64
