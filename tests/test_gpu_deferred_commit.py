"""GPU parity of the deferred commit: gdntree_accept_build (acceptance + next build) followed
by gdntree_accept_commit_verify (the previous step's acceptance and commit inside the next
step's verify), over several decode steps, against the fp64 oracle's step-by-step pipeline.
Trees and acceptance bit-exact; outputs and committed states within 2e-3 of the fp64 state's
Frobenius norm."""
import numpy as np
import pytest
import torch

from workloads import Config, generate, resolve_target

from . import gpu_harness as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _custom(P, K, N, B=2, H_=2, D=128, dtype="bf16", L=1, seed=0, V=1000):
    return generate(Config("custom", B=B, L=L, H=H_, D=D, dtype=dtype, P=P, K=K, V=V, N=N), seed=seed)


def _target(w, tree):
    depth, nn = tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy()
    return resolve_target(depth, nn, w.lat_tok, w.tgt_choice, w.tgt_uniform)


def _oracle_step(w, h_ref):
    import oracle
    return oracle.pipeline(w.lat_logp, w.lat_tok, w.root_tok, w.cfg.N, w.f64("q"), w.f64("k"), w.f64("v"),
                           w.f64("alpha"), w.f64("beta"), h_ref,
                           lambda t: resolve_target(t["depth"], t["n_nodes"], w.lat_tok, w.tgt_choice,
                                                    w.tgt_uniform))


def _tree_np(tree):
    return {f: getattr(tree, f).cpu().numpy() for f in ("parent", "depth", "rank", "token", "score", "anc",
                                                           "n_nodes")}


def run_deferred(steps, label):
    """Step 0: build + verify.  Step i >= 1: acceptance of step i-1 with the build of step i
    (one launch), then step i-1's acceptance + commit + step i's verify (one launch).  After the
    last step: its acceptance + commit.  Every step checked against the oracle, each step
    starting from the oracle's previous committed state."""
    import gdn_draft_tree_amd as g
    w0 = steps[0]
    P, N = w0.cfg.P, w0.cfg.N
    d = [H.device_inputs(w) for w in steps]
    state = d[0]["state"]
    h_ref = w0.h0.double().numpy()
    tree = g.gdntree_build(d[0]["lat_logp"], d[0]["lat_tok"], d[0]["root_tok"], N)
    o = torch.zeros_like(d[0]["q"])
    g.gdntree_verify(tree, d[0]["q"], d[0]["k"], d[0]["v"], d[0]["alpha"], d[0]["beta"], state, o=o)
    prev = pref = None
    worst_o = worst_s = 0.0
    taus = []
    for i, w in enumerate(steps):
        if i > 0:
            pw, pd, ptree, ptarget = prev
            nxt = g.Tree.empty(w.cfg.B, N, "cuda")
            acc = g.gdntree_accept_build(ptree, ptarget, P, d[i]["lat_logp"], d[i]["lat_tok"], d[i]["root_tok"], N,
                                         nxt)
            acc2 = tuple(torch.full_like(a, -7) for a in acc)
            o = torch.zeros_like(d[i]["q"])
            g.gdntree_accept_commit_verify(ptree, ptarget, pd["k"], pd["v"], pd["alpha"], pd["beta"], P, nxt,
                                           d[i]["q"], d[i]["k"], d[i]["v"], d[i]["alpha"], d[i]["beta"], state, o=o,
                                           acc=acc2)
            tree = nxt
            torch.cuda.synchronize()
            for x, x2, y in zip(acc, acc2, (pref["acc_len"], pref["acc_tok"], pref["acc_node"])):
                np.testing.assert_array_equal(x.cpu().numpy(), y)
                np.testing.assert_array_equal(x2.cpu().numpy(), y)
            se = H.state_errors(state.cpu().numpy().astype(np.float64), pref["state"])
            assert se <= H.TOL, f"{label} step {i - 1} committed state error {se:.3e}"
            worst_s = max(worst_s, se)
            taus.append(pref["acc_len"].tolist())
            h_ref = pref["state"]
        torch.cuda.synchronize()
        target = _target(w, tree)
        ref = _oracle_step(w, h_ref)
        H.assert_tree_equal(_tree_np(tree), ref["tree"])
        np.testing.assert_array_equal(target, ref["target"])
        oe = H.output_errors(o.float().cpu().numpy().astype(np.float64), ref["o"], ref["hnorm"],
                             ref["tree"]["n_nodes"])
        assert oe <= H.TOL, f"{label} step {i} output error {oe:.3e}"
        worst_o = max(worst_o, oe)
        prev = (w, d[i], tree, torch.from_numpy(target).cuda())
        pref = ref
    w, dl, tree, target = prev
    acc = g.gdntree_accept_commit(tree, target, dl["k"], dl["v"], dl["alpha"], dl["beta"], state, P)
    torch.cuda.synchronize()
    for x, y in zip(acc, (pref["acc_len"], pref["acc_tok"], pref["acc_node"])):
        np.testing.assert_array_equal(x.cpu().numpy(), y)
    se = H.state_errors(state.cpu().numpy().astype(np.float64), pref["state"])
    assert se <= H.TOL
    _say(f"{label}: {len(steps)} steps, out_err={worst_o:.2e} state_err={max(worst_s, se):.2e} tau={taus}")


@pytest.mark.parametrize("name,heads,reqs,layers", [
    ("ragged", 4, 8, None),      # 65 slots: the 65th-row tile
    ("batched", 8, 8, None),     # 25 slots: two row tiles
    ("one_layer", None, None, None),
    ("deep", 2, None, 6),        # six layers share each tree
    ("tiny", None, None, None),  # fp32 rows and outputs, d = 64
])
def test_deferred_commit_pipeline(name, heads, reqs, layers):
    steps = [H.slice_workload(generate(name, seed=40 + i, B=reqs), H=heads, L=layers) for i in range(4)]
    run_deferred(steps, name)


@pytest.mark.parametrize("D,dtype,N", [(64, "bf16", 64), (128, "f32", 24), (64, "f32", 40), (128, "bf16", 40)])
def test_deferred_commit_dtypes_and_head_dims(D, dtype, N):
    steps = [_custom(P=8, K=16, N=N, B=3, H_=4, D=D, dtype=dtype, seed=60 + i) for i in range(3)]
    run_deferred(steps, f"D={D} {dtype} N={N}")


def test_deferred_commit_of_a_17_row_path():
    """Peaked lattices and targets that always agree with rank 0: every accepted path is 17
    rows long (root + 16 drafts), the longest commit."""
    steps = []
    for i in range(3):
        w = _custom(P=16, K=16, N=64, B=2, H_=4, seed=70 + i)
        logp = w.lat_logp.astype(np.float64)
        logp[..., 0] = -1e-4
        logp[..., 1:] -= 20.0
        w.lat_logp[:] = np.sort(logp, axis=-1)[..., ::-1].astype(np.float32)
        w.tgt_choice[:] = 0
        steps.append(w)
    run_deferred(steps, "tau 17")


def test_deferred_commit_equals_the_two_calls():
    """The fused launch against gdntree_accept_commit followed by gdntree_verify on the same
    inputs: acceptance bitwise; committed state and outputs equal up to fp32 summation order."""
    import gdn_draft_tree_amd as g
    w0, w1 = (H.slice_workload(generate("ragged", seed=50 + i, B=8), H=8) for i in range(2))
    d0, d1 = H.device_inputs(w0), H.device_inputs(w1)
    P, N = w0.cfg.P, w0.cfg.N
    t0 = g.gdntree_build(d0["lat_logp"], d0["lat_tok"], d0["root_tok"], N)
    t1 = g.gdntree_build(d1["lat_logp"], d1["lat_tok"], d1["root_tok"], N)
    torch.cuda.synchronize()
    tgt0 = torch.from_numpy(_target(w0, t0)).cuda()
    s_a, s_b = d0["state"].clone(), d0["state"].clone()
    acc_a = g.gdntree_accept_commit(t0, tgt0, d0["k"], d0["v"], d0["alpha"], d0["beta"], s_a, P)
    o_a = g.gdntree_verify(t1, d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], s_a)
    acc_b = tuple(torch.full_like(x, -7) for x in acc_a)
    o_b = g.gdntree_accept_commit_verify(t0, tgt0, d0["k"], d0["v"], d0["alpha"], d0["beta"], P, t1, d1["q"],
                                         d1["k"], d1["v"], d1["alpha"], d1["beta"], s_b, acc=acc_b)
    torch.cuda.synchronize()
    for x, y in zip(acc_a, acc_b):
        assert torch.equal(x, y)
    norm = torch.linalg.vector_norm(s_a.double(), dim=(-2, -1))
    ds = ((s_a.double() - s_b.double()).abs().amax(dim=(-2, -1)) / norm).max().item()
    nn = t1.n_nodes.cpu()
    do = max(((o_a[:, b, :int(nn[b])].double() - o_b[:, b, :int(nn[b])].double()).abs().max() /
              norm[:, b].min()).item() for b in range(w1.cfg.B))
    _say(f"fused vs two calls: state {ds:.2e}, outputs {do:.2e} (relative to the state norm)")
    assert ds <= 1e-5 and do <= 2e-3


def test_deferred_commit_contains_bad_trees():
    """A previous node count out of range leaves that request's state (and its acceptance
    outputs) untouched; a current node count out of range gives no output but the state is
    still committed; a malformed current tree gives NaN outputs for that request only, with its
    state committed; the other requests are unaffected."""
    import gdn_draft_tree_amd as g
    w0, w1 = (_custom(P=4, K=4, N=8, B=4, H_=2, seed=80 + i) for i in range(2))
    d0, d1 = H.device_inputs(w0), H.device_inputs(w1)
    P, N = 4, 8
    t0 = g.gdntree_build(d0["lat_logp"], d0["lat_tok"], d0["root_tok"], N)
    t1 = g.gdntree_build(d1["lat_logp"], d1["lat_tok"], d1["root_tok"], N)
    torch.cuda.synchronize()
    tgt0 = torch.from_numpy(_target(w0, t0)).cuda()
    s_ref = d0["state"].clone()
    acc_ref = g.gdntree_accept_commit(t0, tgt0, d0["k"], d0["v"], d0["alpha"], d0["beta"], s_ref, P)
    torch.cuda.synchronize()
    t0.n_nodes[0] = 0          # request 0: no acceptance, no commit
    t1.n_nodes[1] = 99         # request 1: no verify output
    t1.parent[2, 5] = 7        # request 2: malformed tree -> NaN outputs
    state = d0["state"].clone()
    acc = tuple(torch.full_like(x, -7) for x in acc_ref)
    o = torch.full_like(d1["q"], 3.0)
    g.gdntree_accept_commit_verify(t0, tgt0, d0["k"], d0["v"], d0["alpha"], d0["beta"], P, t1, d1["q"], d1["k"],
                                   d1["v"], d1["alpha"], d1["beta"], state, o=o, acc=acc)
    torch.cuda.synchronize()
    assert torch.equal(state[:, 0], d0["state"][:, 0])
    assert (acc[0][0] == -7).item() and (acc[1][0] == -7).all() and (acc[2][0] == -7).all()
    for b in (1, 2, 3):
        norm = torch.linalg.vector_norm(s_ref[:, b].double(), dim=(-2, -1))
        err = ((state[:, b].double() - s_ref[:, b].double()).abs().amax(dim=(-2, -1)) / norm).max().item()
        assert err <= 1e-5, (b, err)
        assert torch.equal(acc[0][b], acc_ref[0][b]) and torch.equal(acc[1][b], acc_ref[1][b])
        assert torch.equal(acc[2][b], acc_ref[2][b])
    oc = o.float().cpu()
    assert (oc[:, 1] == 3.0).all()
    assert torch.isnan(oc[:, 2, :int(t1.n_nodes[2])]).all()
    # requests 0 and 3 verify normally: 0 on its unchanged state, 3 on its committed state
    for b, s_use in ((0, d0["state"]), (3, s_ref)):
        o_b = g.gdntree_verify(t1, d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], s_use.clone())
        torch.cuda.synchronize()
        n = int(t1.n_nodes[b])
        diff = (o_b[:, b, :n].float() - o[:, b, :n].float()).abs().max().item()
        assert diff <= 1e-2 * max(1.0, o_b[:, b, :n].float().abs().max().item()), (b, diff)
