"""Writes tiny_seed0.json: the oracle's results on the tiny workload (seed 0).

Calls only the oracle and the seeded input generator.  The fixture guards the oracle
against unnoticed changes; regenerate it only with a change whose commit message names
the passage, or the reading of it, that justifies the new values.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import generate, resolve_target  # noqa: E402


def main():
    w = generate("tiny", seed=0)
    cfg = w.cfg

    def target_fn(tree):
        return resolve_target(tree["depth"], tree["n_nodes"], w.lat_tok, w.tgt_choice, w.tgt_uniform)

    r = oracle.pipeline(w.lat_logp, w.lat_tok, w.root_tok, cfg.N, w.f64("q"), w.f64("k"), w.f64("v"),
                        w.f64("alpha"), w.f64("beta"), w.h0.double().numpy(), target_fn)
    n = int(r["tree"]["n_nodes"][0])
    out = {
        "workload": "tiny", "seed": 0,
        "n_nodes": n,
        "parent": r["tree"]["parent"][0, :n].tolist(),
        "depth": r["tree"]["depth"][0, :n].tolist(),
        "rank": r["tree"]["rank"][0, :n].tolist(),
        "token": r["tree"]["token"][0, :n].tolist(),
        "score_hex": [float(x).hex() for x in r["tree"]["score"][0, :n]],
        "anc": [int(x) for x in r["tree"]["anc"][0, :n]],
        "target": r["target"][0, :n].tolist(),
        "acc_len": int(r["acc_len"][0]),
        "acc_tok": r["acc_tok"][0].tolist(),
        "acc_node": r["acc_node"][0].tolist(),
        "o": np.round(r["o"][0, 0, :n, 0], 12).tolist(),
        "hnorm": np.round(r["hnorm"][0, 0, :n, 0], 12).tolist(),
        "state_diag": np.round(np.diagonal(r["state"][0, 0, 0]), 12).tolist(),
        "state_fro": round(float(np.linalg.norm(r["state"][0, 0, 0])), 12),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_seed0.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
