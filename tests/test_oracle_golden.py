"""The oracle still reproduces its stored results on the tiny workload (regression guard;
the fixture is written by tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os

import numpy as np

import oracle
from workloads import generate, resolve_target

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_golden():
    with open(os.path.join(HERE, "golden", "tiny_seed0.json")) as f:
        g = json.load(f)
    w = generate("tiny", seed=0)

    def target_fn(tree):
        return resolve_target(tree["depth"], tree["n_nodes"], w.lat_tok, w.tgt_choice, w.tgt_uniform)

    r = oracle.pipeline(w.lat_logp, w.lat_tok, w.root_tok, w.cfg.N, w.f64("q"), w.f64("k"), w.f64("v"),
                        w.f64("alpha"), w.f64("beta"), w.h0.double().numpy(), target_fn)
    n = g["n_nodes"]
    t = r["tree"]
    assert int(t["n_nodes"][0]) == n
    assert t["parent"][0, :n].tolist() == g["parent"]
    assert t["rank"][0, :n].tolist() == g["rank"]
    assert t["token"][0, :n].tolist() == g["token"]
    assert [float(x).hex() for x in t["score"][0, :n]] == g["score_hex"]
    assert [int(x) for x in t["anc"][0, :n]] == g["anc"]
    assert int(r["acc_len"][0]) == g["acc_len"]
    assert r["acc_tok"][0].tolist() == g["acc_tok"]
    np.testing.assert_allclose(r["o"][0, 0, :n, 0], g["o"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(np.diagonal(r["state"][0, 0, 0]), g["state_diag"], rtol=0, atol=1e-11)
