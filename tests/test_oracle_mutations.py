"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a flipped sign, a transposed operand, a
wrong index or tie-break, an off-by-one in acceptance) into a copy of the oracle's source
on the CPU, swaps the copy's functions into the ``oracle`` package, and checks that at
least one pin fails.  The real oracle is restored afterwards.
"""
import importlib
import inspect
import types

import pytest

import oracle
from oracle import gdntree_oracle as real

from . import test_oracle_accept as T_acc
from . import test_oracle_build as T_build
from . import test_oracle_markov as T_markov
from . import test_oracle_shared as T_shared
from . import test_oracle_verify as T_ver

MUTATIONS = {
    "drop_alpha": ("return a * (h_prev - b * k[..., :, None] * kT_h[..., None, :]) + b",
                   "return (h_prev - b * k[..., :, None] * kT_h[..., None, :]) + b"),
    "sign_delta": ("(h_prev - b * k[..., :, None]", "(h_prev + b * k[..., :, None]"),
    "drop_beta_write": ("+ b * k[..., :, None] * v[..., None, :]", "+ k[..., :, None] * v[..., None, :]"),
    "transpose_readout": ("return (q[..., None, :] @ h)[..., 0, :]", "return (h @ q[..., :, None])[..., 0]"),
    "transpose_kh": ("kT_h = (k[..., None, :] @ h_prev)[..., 0, :]", "kT_h = (h_prev @ k[..., :, None])[..., 0]"),
    "wrong_parent": ("hp = h0 if i == 0 else states[parent[i]]", "hp = h0 if i == 0 else states[i - 1]"),
    "tie_rank_desc": ("return (-s, p, r)", "return (-s, p, -r)"),
    "tie_parent_desc": ("return (-s, p, r)", "return (-s, -p, r)"),
    "score_wrong_position": ("s = score[p] + float(np.float64(lat_logp[b, depth[p], r]))",
                             "s = score[p] + float(np.float64(lat_logp[b, 0, r]))"),
    "no_bonus": ("+ [int(target[b, u])]", ""),
    "accept_highest_index": ("u = min(nxt)", "u = max(nxt)"),
    "tau_off_by_one": ("acc_len[b] = len(path)", "acc_len[b] = len(path) - 1"),
    "shared_tie_request_desc": ("return (-s, b, p, r)", "return (-s, -b, p, r)"),
    "shared_no_cap": ("if i == N:  # the request is full", "if i == -1:  # the request is full"),
    "shared_budget_off_by_one": ("while total < G and frontier:", "while total <= G and frontier:"),
    "commit_skips_root": ("for i in acc_node[b, :int(acc_len[b])]:",
                          "for i in acc_node[b, 1:int(acc_len[b])]:"),
    "markov_prev_same_position": ("x = int(root_tok[b]) if s == 0 else int(lat_tok[b, s - 1, pr])",
                                  "x = int(root_tok[b]) if s == 0 else int(lat_tok[b, s, pr])"),
    "markov_no_root": ("x = int(root_tok[b]) if s == 0 else int(lat_tok[b, s - 1, pr])",
                       "x = int(lat_tok[b, 0, pr]) if s == 0 else int(lat_tok[b, s - 1, pr])"),
    "markov_sign": ("float(bases[b, s, r]) + float(np.dot(", "float(bases[b, s, r]) - float(np.dot("),
    "markov_no_normalise": ("out[b, s, pr] = logits - (m + np.log(np.sum(np.exp(logits - m))))",
                            "out[b, s, pr] = logits - m"),
    "cond_transposed": ("edge_logp[b, depth[p], rank[p] if depth[p] >= 1 else 0, r]",
                        "edge_logp[b, depth[p], r, rank[p] if depth[p] >= 1 else 0]"),
    "cond_unconditioned": ("edge_logp[b, depth[p], rank[p] if depth[p] >= 1 else 0, r]",
                           "edge_logp[b, depth[p], 0, r]"),
    "cond_tie_rank_desc": ("key=lambda c: (-(score[c[0]] + edge(*c)), c[0], c[1])",
                           "key=lambda c: (-(score[c[0]] + edge(*c)), c[0], -c[1])"),
}

EXPORTS = ["build_tree", "build_tree_shared", "build_tree_cond", "markov_edge_logp", "gdn_update", "gdn_readout", "gdn_step", "verify_request", "verify",
           "accept", "commit", "pipeline"]


def _pins():
    for mod in (T_build, T_shared, T_ver, T_acc, T_markov):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            if not params:
                yield fn, {}
                continue
            argnames, values = params[0].args[0], params[0].args[1]
            names = [a.strip() for a in argnames.split(",")]
            for val in list(values)[:3]:
                val = val if isinstance(val, tuple) else (val,)
                yield fn, dict(zip(names, val))


def _any_pin_fails() -> bool:
    for fn, kwargs in _pins():
        try:
            fn(**kwargs)
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    src = inspect.getsource(real)
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name} not found"
    mutant = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mutant.__dict__)
    for fn in EXPORTS:
        monkeypatch.setattr(oracle, fn, getattr(mutant, fn))
    assert _any_pin_fails(), f"no pin caught mutation {name}"


def test_unmutated_oracle_passes_all_pins():
    importlib.reload(real)
    assert not _any_pin_fails()
