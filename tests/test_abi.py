"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments on
the host before touching a device (CPU only: no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdntree.h")


def _lib():
    import gdn_draft_tree_amd as g
    return g


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdntree_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert _declared() == ["gdntree_accept", "gdntree_accept_build", "gdntree_accept_commit",
                           "gdntree_accept_commit_build", "gdntree_accept_commit_build_shared",
                           "gdntree_accept_commit_verify", "gdntree_build", "gdntree_build_cond",
                           "gdntree_build_shared", "gdntree_commit", "gdntree_commit_build",
                           "gdntree_markov_edges", "gdntree_status_str", "gdntree_verify"]


def test_library_exports_every_declared_symbol():
    g = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (gdntree_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(g.LIB, name)
    # nothing else leaks out of the library under the gdntree_ prefix
    assert exported == set(_declared())


def test_status_strings():
    g = _lib()
    seen = set()
    for code in (g.GDNTREE_OK, g.GDNTREE_ERR_ARG, g.GDNTREE_ERR_UNSUPPORTED, g.GDNTREE_ERR_DEVICE):
        s = g.gdntree_status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 4
    assert g.gdntree_status_str(99) == "unknown status"
    assert g.gdntree_status_str(-1) == "unknown status"


FAKE = 0x1000  # never dereferenced: every case below fails validation first


def _tree(g, **null):
    fields = {f: FAKE for f, _ in g.CTree._fields_}
    fields.update({k: None for k in null})
    return g.CTree(**fields)


@pytest.mark.parametrize("case,expect", [
    ("null_logp", 1), ("null_tree_field", 1), ("B0", 1), ("P0", 1), ("K0", 1), ("N0", 1),
    ("P17", 2), ("K65", 2), ("N65", 2),
])
def test_build_rejects(case, expect):
    g = _lib()
    args = dict(logp=FAKE, tok=FAKE, root=FAKE, B=2, P=8, K=16, N=24, tree=_tree(g))
    if case == "null_logp": args["logp"] = None
    if case == "null_tree_field": args["tree"] = _tree(g, anc=1)
    if case == "B0": args["B"] = 0
    if case == "P0": args["P"] = 0
    if case == "K0": args["K"] = 0
    if case == "N0": args["N"] = 0
    if case == "P17": args["P"] = 17
    if case == "K65": args["K"] = 65
    if case == "N65": args["N"] = 65
    st = g.LIB.gdntree_build(args["logp"], args["tok"], args["root"], args["B"], args["P"], args["K"],
                             args["N"], args["tree"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_edge", 1), ("null_tok", 1), ("null_tree_field", 1), ("B0", 1), ("K0", 1), ("N0", 1),
    ("P17", 2), ("K17", 2), ("N65", 2),
])
def test_build_cond_rejects(case, expect):
    """Conditioned rows are staged per request in LDS: K <= 16."""
    g = _lib()
    args = dict(edge=FAKE, tok=FAKE, root=FAKE, B=2, P=8, K=16, N=24, tree=_tree(g))
    if case == "null_edge": args["edge"] = None
    if case == "null_tok": args["tok"] = None
    if case == "null_tree_field": args["tree"] = _tree(g, score=1)
    if case == "B0": args["B"] = 0
    if case == "K0": args["K"] = 0
    if case == "N0": args["N"] = 0
    if case == "P17": args["P"] = 17
    if case == "K17": args["K"] = 17
    if case == "N65": args["N"] = 65
    st = g.LIB.gdntree_build_cond(args["edge"], args["tok"], args["root"], args["B"], args["P"], args["K"],
                                  args["N"], args["tree"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_bases", 1), ("null_w2", 1), ("null_out", 1), ("B0", 1), ("V0", 1), ("R0", 1), ("dtype", 1),
    ("P17", 2), ("K65", 2), ("R65", 2), ("Vbig", 2),
])
def test_markov_edges_rejects(case, expect):
    g = _lib()
    args = dict(bases=FAKE, tok=FAKE, root=FAKE, W1=FAKE, W2=FAKE, dt=g.GDNTREE_F32, B=2, P=8, K=16, V=1000,
                R=32, out=FAKE)
    if case == "null_bases": args["bases"] = None
    if case == "null_w2": args["W2"] = None
    if case == "null_out": args["out"] = None
    if case == "B0": args["B"] = 0
    if case == "V0": args["V"] = 0
    if case == "R0": args["R"] = 0
    if case == "dtype": args["dt"] = 7
    if case == "P17": args["P"] = 17
    if case == "K65": args["K"] = 65
    if case == "R65": args["R"] = 65
    if case == "Vbig": args["V"] = 1 << 25  # V * R * 4 bytes past 2^31
    st = g.LIB.gdntree_markov_edges(args["bases"], args["tok"], args["root"], args["W1"], args["W2"], args["dt"],
                                    args["B"], args["P"], args["K"], args["V"], args["R"], args["out"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_target", 1), ("null_acc", 1), ("null_next_tree_field", 1), ("same_tree", 1), ("B0", 1),
    ("next_K0", 1), ("N65", 2), ("P17", 2), ("next_P17", 2), ("next_K65", 2), ("next_N65", 2),
])
def test_accept_build_rejects(case, expect):
    g = _lib()
    tree, nxt = _tree(g), g.CTree(**{f: 0x2000 for f, _ in g.CTree._fields_})
    a = dict(tree=tree, B=2, N=24, P=8, tgt=FAKE, acc=(FAKE, FAKE, FAKE), lp=FAKE, lt=FAKE, rt=FAKE, nB=2, nP=8,
             nK=16, nN=24, nxt=nxt)
    if case == "null_target": a["tgt"] = None
    if case == "null_acc": a["acc"] = (FAKE, None, FAKE)
    if case == "null_next_tree_field": a["nxt"] = g.CTree(**{**{f: 0x2000 for f, _ in g.CTree._fields_}, "rank": None})
    if case == "same_tree": a["nxt"] = tree
    if case == "B0": a["B"] = 0
    if case == "next_K0": a["nK"] = 0
    if case == "N65": a["N"] = 65
    if case == "P17": a["P"] = 17
    if case == "next_P17": a["nP"] = 17
    if case == "next_K65": a["nK"] = 65
    if case == "next_N65": a["nN"] = 65
    st = g.LIB.gdntree_accept_build(a["tree"], a["B"], a["N"], a["P"], a["tgt"], *a["acc"], a["lp"], a["lt"], a["rt"],
                                    a["nB"], a["nP"], a["nK"], a["nN"], a["nxt"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_prev_token", 1), ("null_prev_target", 1), ("null_prev_k", 1), ("null_q", 1), ("null_state", 1),
    ("acc_mixed", 1), ("prevN0", 1), ("prevP0", 1), ("H0", 1), ("in_dtype", 1), ("out_dtype", 1), ("dk0", 1),
    ("dk96", 2), ("dk_ne_dv", 2), ("N65", 2), ("prevN65", 2), ("prevP17", 2),
])
def test_accept_commit_verify_rejects(case, expect):
    g = _lib()
    a = dict(prev=_tree(g), pN=24, pP=8, ptgt=FAKE, pk=FAKE, pv=FAKE, pa=FAKE, pb=FAKE, acc=(None, None, None),
             tree=_tree(g), B=2, N=24, L=1, H=4, dk=128, dv=128, dt=g.GDNTREE_BF16, q=FAKE, k=FAKE, v=FAKE,
             al=FAKE, be=FAKE, st=FAKE, odt=g.GDNTREE_BF16, o=FAKE)
    if case == "null_prev_token": a["prev"] = _tree(g, token=1)
    if case == "null_prev_target": a["ptgt"] = None
    if case == "null_prev_k": a["pk"] = None
    if case == "null_q": a["q"] = None
    if case == "null_state": a["st"] = None
    if case == "acc_mixed": a["acc"] = (FAKE, FAKE, None)
    if case == "prevN0": a["pN"] = 0
    if case == "prevP0": a["pP"] = 0
    if case == "H0": a["H"] = 0
    if case == "in_dtype": a["dt"] = 5
    if case == "out_dtype": a["odt"] = 5
    if case == "dk0": a["dk"] = 0
    if case == "dk96": a["dk"] = a["dv"] = 96
    if case == "dk_ne_dv": a["dv"] = 64
    if case == "N65": a["N"] = 65
    if case == "prevN65": a["pN"] = 65
    if case == "prevP17": a["pP"] = 17
    st = g.LIB.gdntree_accept_commit_verify(a["prev"], a["pN"], a["pP"], a["ptgt"], a["pk"], a["pv"], a["pa"], a["pb"],
                                            *a["acc"], a["tree"], a["B"], a["N"], a["L"], a["H"], a["dk"], a["dv"],
                                            a["dt"], a["q"], a["k"], a["v"], a["al"], a["be"], a["st"], a["odt"],
                                            a["o"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_logp", 1), ("null_root", 1), ("null_tree_field", 1), ("B0", 1), ("N0", 1), ("Gneg", 1),
    ("P17", 2), ("K65", 2), ("N65", 2), ("B1025", 2), ("BN4097", 2),
])
def test_build_shared_rejects(case, expect):
    """Rejected on the host before any device work (a null positions array is allowed)."""
    g = _lib()
    a = dict(logp=FAKE, tok=FAKE, root=FAKE, B=2, P=8, K=16, N=24, G=30, tree=_tree(g))
    if case == "null_logp": a["logp"] = None
    if case == "null_root": a["root"] = None
    if case == "null_tree_field": a["tree"] = _tree(g, n_nodes=1)
    if case == "B0": a["B"] = 0
    if case == "N0": a["N"] = 0
    if case == "Gneg": a["G"] = -1
    if case == "P17": a["P"] = 17
    if case == "K65": a["K"] = 65
    if case == "N65": a["N"] = 65
    if case == "B1025": a.update(B=1025, N=1)
    if case == "BN4097": a.update(B=65, N=64, G=100)   # 128 lists x 64 keys
    st = g.LIB.gdntree_build_shared(a["logp"], a["tok"], a["root"], None, a["B"], a["P"], a["K"], a["N"],
                                    a["G"], a["tree"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_q", 1), ("null_state", 1), ("null_parent", 1), ("H0", 1), ("L0", 1), ("dtype9", 1),
    ("out_dtype9", 1), ("dk_ne_dv", 2), ("d96", 2), ("d256", 2), ("N65", 2), ("dneg", 1),
])
def test_verify_rejects(case, expect):
    g = _lib()
    a = dict(tree=_tree(g), B=2, N=24, L=1, H=4, dk=128, dv=128, idt=1, q=FAKE, k=FAKE, v=FAKE,
             al=FAKE, be=FAKE, st=FAKE, odt=1, o=FAKE)
    if case == "null_q": a["q"] = None
    if case == "null_state": a["st"] = None
    if case == "null_parent": a["tree"] = _tree(g, parent=1)
    if case == "H0": a["H"] = 0
    if case == "L0": a["L"] = 0
    if case == "dtype9": a["idt"] = 9
    if case == "out_dtype9": a["odt"] = 9
    if case == "dk_ne_dv": a["dv"] = 64
    if case == "d96": a["dk"] = a["dv"] = 96
    if case == "d256": a["dk"] = a["dv"] = 256
    if case == "N65": a["N"] = 65
    if case == "dneg": a["dk"] = -128
    st = g.LIB.gdntree_verify(a["tree"], a["B"], a["N"], a["L"], a["H"], a["dk"], a["dv"], a["idt"], a["q"],
                              a["k"], a["v"], a["al"], a["be"], a["st"], a["odt"], a["o"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_target", 1), ("null_acc", 1), ("null_token", 1), ("P0", 1), ("P17", 2), ("N65", 2),
    ("d32", 2), ("dtype7", 1),
])
def test_accept_commit_rejects(case, expect):
    g = _lib()
    a = dict(tree=_tree(g), B=2, N=24, P=8, tgt=FAKE, L=1, H=4, dk=128, dv=128, idt=1, k=FAKE, v=FAKE,
             al=FAKE, be=FAKE, st=FAKE, al_=FAKE, at=FAKE, an=FAKE)
    if case == "null_target": a["tgt"] = None
    if case == "null_acc": a["an"] = None
    if case == "null_token": a["tree"] = _tree(g, token=1)
    if case == "P0": a["P"] = 0
    if case == "P17": a["P"] = 17
    if case == "N65": a["N"] = 65
    if case == "d32": a["dk"] = a["dv"] = 32
    if case == "dtype7": a["idt"] = 7
    st = g.LIB.gdntree_accept_commit(a["tree"], a["B"], a["N"], a["P"], a["tgt"], a["L"], a["H"], a["dk"],
                                     a["dv"], a["idt"], a["k"], a["v"], a["al"], a["be"], a["st"], a["al_"],
                                     a["at"], a["an"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_target", 1), ("null_acc_tok", 1), ("null_token", 1), ("B0", 1), ("N0", 1), ("P0", 1),
    ("P17", 2), ("N65", 2),
])
def test_accept_rejects(case, expect):
    g = _lib()
    a = dict(tree=_tree(g), B=2, N=24, P=8, tgt=FAKE, al_=FAKE, at=FAKE, an=FAKE)
    if case == "null_target": a["tgt"] = None
    if case == "null_acc_tok": a["at"] = None
    if case == "null_token": a["tree"] = _tree(g, token=1)
    if case == "B0": a["B"] = 0
    if case == "N0": a["N"] = 0
    if case == "P0": a["P"] = 0
    if case == "P17": a["P"] = 17
    if case == "N65": a["N"] = 65
    st = g.LIB.gdntree_accept(a["tree"], a["B"], a["N"], a["P"], a["tgt"], a["al_"], a["at"], a["an"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_acc_len", 1), ("null_acc_node", 1), ("null_state", 1), ("null_parent", 1), ("H0", 1),
    ("P17", 2), ("N65", 2), ("d32", 2), ("dk_ne_dv", 2), ("dtype7", 1),
])
def test_commit_rejects(case, expect):
    g = _lib()
    a = dict(tree=_tree(g), B=2, N=24, P=8, al_=FAKE, an=FAKE, L=1, H=4, dk=128, dv=128, idt=1, k=FAKE,
             v=FAKE, al=FAKE, be=FAKE, st=FAKE)
    if case == "null_acc_len": a["al_"] = None
    if case == "null_acc_node": a["an"] = None
    if case == "null_state": a["st"] = None
    if case == "null_parent": a["tree"] = _tree(g, parent=1)
    if case == "H0": a["H"] = 0
    if case == "P17": a["P"] = 17
    if case == "N65": a["N"] = 65
    if case == "d32": a["dk"] = a["dv"] = 32
    if case == "dk_ne_dv": a["dv"] = 64
    if case == "dtype7": a["idt"] = 7
    st = g.LIB.gdntree_commit(a["tree"], a["B"], a["N"], a["P"], a["al_"], a["an"], a["L"], a["H"], a["dk"],
                              a["dv"], a["idt"], a["k"], a["v"], a["al"], a["be"], a["st"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_acc_node", 1), ("null_state", 1), ("null_next_logp", 1), ("null_next_anc", 1), ("same_tree", 1),
    ("next_B0", 1), ("next_K0", 1), ("H0", 1), ("next_P17", 2), ("next_K65", 2), ("next_N65", 2), ("N65", 2),
    ("d32", 2), ("dtype7", 1),
])
def test_commit_build_rejects(case, expect):
    g = _lib()
    nxt = g.CTree(**{f: 0x2000 for f, _ in g.CTree._fields_})
    a = dict(tree=_tree(g), B=2, N=24, P=8, al_=FAKE, an=FAKE, L=1, H=4, dk=128, dv=128, idt=1, k=FAKE,
             v=FAKE, al=FAKE, be=FAKE, st=FAKE, nlp=FAKE, ntok=FAKE, nroot=FAKE, nB=2, nP=8, nK=16, nN=24,
             nxt=nxt)
    if case == "null_acc_node": a["an"] = None
    if case == "null_state": a["st"] = None
    if case == "null_next_logp": a["nlp"] = None
    if case == "null_next_anc": a["nxt"] = g.CTree(**{f: (None if f == "anc" else 0x2000) for f, _ in g.CTree._fields_})
    if case == "same_tree": a["nxt"] = _tree(g)
    if case == "next_B0": a["nB"] = 0
    if case == "next_K0": a["nK"] = 0
    if case == "H0": a["H"] = 0
    if case == "next_P17": a["nP"] = 17
    if case == "next_K65": a["nK"] = 65
    if case == "next_N65": a["nN"] = 65
    if case == "N65": a["N"] = 65
    if case == "d32": a["dk"] = a["dv"] = 32
    if case == "dtype7": a["idt"] = 7
    st = g.LIB.gdntree_commit_build(a["tree"], a["B"], a["N"], a["P"], a["al_"], a["an"], a["L"], a["H"],
                                    a["dk"], a["dv"], a["idt"], a["k"], a["v"], a["al"], a["be"], a["st"],
                                    a["nlp"], a["ntok"], a["nroot"], a["nB"], a["nP"], a["nK"], a["nN"],
                                    a["nxt"], None)
    assert st == expect


@pytest.mark.parametrize("case,expect", [
    ("null_target", 1), ("null_acc_tok", 1), ("null_token", 1), ("null_next_root", 1), ("same_token", 1),
    ("next_N0", 1), ("L0", 1), ("P17", 2), ("next_K65", 2), ("d96", 2), ("dtype5", 1),
])
def test_accept_commit_build_rejects(case, expect):
    g = _lib()
    nxt = g.CTree(**{f: 0x2000 for f, _ in g.CTree._fields_})
    a = dict(tree=_tree(g), B=2, N=24, P=8, tgt=FAKE, L=1, H=4, dk=128, dv=128, idt=1, k=FAKE, v=FAKE,
             al=FAKE, be=FAKE, st=FAKE, al_=FAKE, at=FAKE, an=FAKE, nlp=FAKE, ntok=FAKE, nroot=FAKE, nB=2, nP=8,
             nK=16, nN=24, nxt=nxt)
    if case == "null_target": a["tgt"] = None
    if case == "null_acc_tok": a["at"] = None
    if case == "null_token": a["tree"] = _tree(g, token=1)
    if case == "null_next_root": a["nroot"] = None
    if case == "same_token": a["nxt"] = g.CTree(**{f: (FAKE if f == "token" else 0x2000) for f, _ in g.CTree._fields_})
    if case == "next_N0": a["nN"] = 0
    if case == "L0": a["L"] = 0
    if case == "P17": a["P"] = 17
    if case == "next_K65": a["nK"] = 65
    if case == "d96": a["dk"] = a["dv"] = 96
    if case == "dtype5": a["idt"] = 5
    st = g.LIB.gdntree_accept_commit_build(a["tree"], a["B"], a["N"], a["P"], a["tgt"], a["L"], a["H"], a["dk"],
                                           a["dv"], a["idt"], a["k"], a["v"], a["al"], a["be"], a["st"],
                                           a["al_"], a["at"], a["an"], a["nlp"], a["ntok"], a["nroot"], a["nB"],
                                           a["nP"], a["nK"], a["nN"], a["nxt"], None)
    assert st == expect


def test_no_device_reports_err_device():
    """Valid arguments on a machine without a GPU stop at the device check (no launch)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case only runs where no device exists")
    g = _lib()
    st = g.LIB.gdntree_verify(_tree(g), 2, 24, 1, 4, 128, 128, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                              FAKE, None)
    assert st == g.GDNTREE_ERR_DEVICE


def test_binding_checks_devices_and_dtypes():
    """The Python binding refuses host tensors before calling the library."""
    import torch
    g = _lib()
    with pytest.raises(ValueError):
        g.gdntree_build(torch.zeros(1, 4, 4), torch.zeros(1, 4, 4, dtype=torch.int32),
                        torch.zeros(1, dtype=torch.int32), 8,
                        out=g.Tree(*[torch.zeros(1, 9)] * 6, torch.zeros(1)))


@pytest.mark.parametrize("case,expect", [("Gneg", 1), ("null_state", 1), ("same_tree", 1), ("nB1025", 2),
                                         ("cut_too_big", 2), ("N65", 2)])
def test_accept_commit_build_shared_rejects(case, expect):
    g = _lib()
    a = dict(tree=_tree(g), nt=g.CTree(**{f: FAKE + 8 for f, _ in g.CTree._fields_}), st=FAKE, nB=2, nN=24, G=30,
             N=24)
    if case == "Gneg": a["G"] = -1
    if case == "null_state": a["st"] = None
    if case == "same_tree": a["nt"] = _tree(g)
    if case == "nB1025": a.update(nB=1025, nN=1, G=10)
    if case == "cut_too_big": a.update(nB=65, nN=64, G=100)
    if case == "N65": a["N"] = 65
    st = g.LIB.gdntree_accept_commit_build_shared(a["tree"], 2, a["N"], 8, FAKE, 1, 4, 128, 128, 1, FAKE, FAKE,
                                                  FAKE, FAKE, a["st"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                  a["nB"], 8, 16, a["nN"], a["G"], a["nt"], None)
    assert st == expect
