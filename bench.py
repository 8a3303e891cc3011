"""Throughput of the draft-tree verification step on one MI355X.

A step is one pass of the whole path over one batch: tree build, verify, acceptance and
state commit.  Steps are pipelined the way a decode loop can run them: gdntree_verify ->
gdntree_accept_commit_build, where the second call accepts, commits this step's states and
builds the next batch's trees in one launch (each request's next build starts once that
request's acceptance is known: it stands for the next draft, which needs the accepted
tokens); the next verify runs after it.  The same steps strictly in order
(build -> verify -> accept_commit) are reported beside it as `sequential`.  The default workload is the large ragged batch: 32 requests x one
GDN layer (32 heads, d = 128), 16-position x top-16 lattices, N = 64 draft nodes per
request, bf16 rows, fp32 state.  The synthetic target argmax (the stand-in for the target
model's LM head) is resolved once per input set, untimed, from the deterministic tree.

Honest HBM numbers: the timed steps rotate through several independent input sets (more
than the 256 MB last-level cache), so each step reads its rows and states from HBM.

Prints ONE JSON line.  value = verified (node, layer) pairs per second over whole steps.
roofline: the verify kernel (the dominant one), algorithmic bytes per launch / its mean
duration, from HIP events on the launch stream around the same launches run back to back.
cpu_baseline: the fp64 oracle on a bounded sample of the same workload, on the host, in worker
processes (one request per task), with a single-process figure beside it.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload ragged]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE_METRIC = "GDN tree-verify nodes/s per layer + achieved HBM GB/s vs ~8 TB/s peak"
COPY_BYTES = 256 << 20
VERIFY_SRC = os.path.join(ROOT, "gdn_draft_tree_amd", "csrc", "verify_tree.hip")
COUNTERS_MD = os.path.join(ROOT, "profiles", "verify_kernel_ragged_counters.md")


def measured_traffic(workload: str):
    """HBM bytes per verify launch from the committed counter summary, or None when there is
    none for this workload or the kernel source has changed since the counters were taken
    (the summary records the SHA-256 of the kernel source it measured)."""
    import hashlib
    import re
    if workload != "ragged" or not os.path.exists(COUNTERS_MD):
        return None
    text = open(COUNTERS_MD).read()
    src = hashlib.sha256(open(VERIFY_SRC, "rb").read()).hexdigest()
    m_src = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    m_val = re.search(r"HBM bytes per verify launch: ([0-9]+)", text)
    if not m_src or not m_val or m_src.group(1) != src:
        return None
    return int(m_val.group(1))


def verify_bytes(cfg, n_nodes_total: int, out_elem: int) -> int:
    """Algorithmic HBM bytes of one verify launch: the fp32 state of every (layer, request,
    head) once, plus q, k, v, alpha, beta read and o written once per used row."""
    e = 2 if cfg.dtype == "bf16" else 4
    per_row = 3 * cfg.D * e + 2 * e + cfg.D * out_elem
    return cfg.L * cfg.H * (cfg.B * 4 * cfg.D * cfg.D + n_nodes_total * per_row)


def commit_bytes(cfg, tau_total: int) -> int:
    e = 2 if cfg.dtype == "bf16" else 4
    return cfg.L * cfg.H * (cfg.B * 8 * cfg.D * cfg.D + tau_total * (2 * cfg.D * e + 2 * e))


def calibration_kernels(dev) -> None:
    """Kernels of known traffic for scaling hardware byte counters: a plain 256 MiB copy
    (dst = src * 1, torch's elementwise kernel), then the streaming probe reading 256 MiB once
    from a buffer that a 1 GiB write has since pushed out of every cache (no writes)."""
    import ctypes

    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    cal = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush.fill_(0)
    probe = ctypes.CDLL(os.path.join(ROOT, "gdn_draft_tree_amd", "libgdntree_probe.so"))
    probe.gdntree_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_int, ctypes.c_void_p]
    st = probe.gdntree_probe_stream(cal.data_ptr(), COPY_BYTES, None, 0, 4096,
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(f"stream probe failed ({st})")


# The workload the CPU baseline's worker processes share (set before they are forked).
_CPU_WORK: dict = {}


def _oracle_on_requests(job):
    """Worker: the oracle's whole pipeline on requests [b0, b1) and layers [l0, l1) of one
    generated workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import resolve_target
    seed, b0, b1, l0, l1 = job
    w, x = _CPU_WORK[seed]
    sl, ll = slice(b0, b1), slice(l0, l1)
    lat_tok, tch, tun = w.lat_tok[sl], w.tgt_choice[sl], w.tgt_uniform[sl]

    def target_fn(tree):
        return resolve_target(tree["depth"], tree["n_nodes"], lat_tok, tch, tun)

    shared = {}
    if w.cfg.G is not None:  # the batch budget couples the requests: a task is the whole batch
        shared = dict(G=w.cfg.G, positions=w.cfg.positions_for(b1 - b0))
    with threadpool_limits(limits=1):
        r = oracle.pipeline(w.lat_logp[sl], lat_tok, w.root_tok[sl], w.cfg.N, x["q"][ll, sl], x["k"][ll, sl],
                            x["v"][ll, sl], x["alpha"][ll, sl], x["beta"][ll, sl], x["h0"][ll, sl], target_fn,
                            **shared)
    return int(np.asarray(r["tree"]["n_nodes"]).sum()) * (l1 - l0)


def cpu_baseline(name: str, reqs: int, seeds: int, workers: int) -> dict:
    """The fp64 oracle (unchanged) timed on the host: once in one process on `reqs` requests,
    and in up to `workers` forked processes over `seeds` x `reqs` requests split into (request,
    layer) tasks (each runs the oracle's full pipeline on one request and one layer, BLAS
    limited to one thread). Runs before the GPU is touched, so forking is safe."""
    import multiprocessing as mp

    from workloads import generate
    for s in range(seeds):  # inputs widened to fp64 up front, outside the timed region
        w = generate(name, seed=s, B=reqs)
        _CPU_WORK[s] = (w, {f: w.f64(f) for f in ("q", "k", "v", "alpha", "beta", "h0")})
    L = _CPU_WORK[0][0].cfg.L
    t0 = time.perf_counter()
    nodes1 = _oracle_on_requests((0, 0, reqs, 0, L))
    dt1 = time.perf_counter() - t0
    if _CPU_WORK[0][0].cfg.G is None:
        jobs = [(s, b, b + 1, l, l + 1) for s in range(seeds) for b in range(reqs) for l in range(L)]
    else:
        jobs = [(s, 0, reqs, l, l + 1) for s in range(seeds) for l in range(L)]
    workers = min(workers, len(jobs))
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(abs, range(workers))  # workers started before the clock
        t0 = time.perf_counter()
        nodes = sum(pool.map(_oracle_on_requests, jobs, chunksize=1))
        dt = time.perf_counter() - t0
    model = ""
    try:
        model = next(x.split(":", 1)[1].strip() for x in open("/proc/cpuinfo") if x.startswith("model name"))
    except (OSError, StopIteration):
        pass
    unit = "request" if _CPU_WORK[0][0].cfg.G is None else "whole batch"
    _CPU_WORK.clear()
    return {"value": nodes / dt, "unit": "nodes/s", "cores": workers, "kind": "oracle",
            "sample": f"{name} workload, seeds 0..{seeds - 1}, the first {reqs} requests of each "
                      f"({seeds * reqs} requests x {L} layers): the oracle's full build+verify+accept+commit "
                      f"pipeline in fp64 numpy, one ({unit}, "
                      f"layer) per task over {workers} worker "
                      f"processes (BLAS 1 thread each), {dt:.1f} s wall",
            "value_1core": nodes1 / dt1, "sample_1core": f"seed 0, {reqs} requests x {L} layers in one process, {dt1:.1f} s",
            "cpu_model": model}


def stream_ceiling(cfg, units: int, rows_per_unit: float, reps: int = 100) -> dict:
    """What this part streams for the verify launch's traffic with none of its work: the probe
    kernel (gdn_draft_tree_amd/csrc/stream_probe.hip) with one workgroup per (layer, request,
    head) reading that unit's state and rows and writing its output rows; the same reads alone;
    and one plain 1 GiB read.  Buffers rotate over more than 512 MB (so the 256 MB last-level
    cache cannot serve the reads); median over `reps` launches, each timed with HIP events."""
    import ctypes

    import numpy as np
    import torch
    probe = ctypes.CDLL(os.path.join(ROOT, "gdn_draft_tree_amd", "libgdntree_probe.so"))
    probe.gdntree_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_int, ctypes.c_void_p]
    e = 2 if cfg.dtype == "bf16" else 4
    rd = int(units * (4 * cfg.D * cfg.D + rows_per_unit * (3 * cfg.D * e + 2 * e))) // 16 * 16
    wr = int(units * rows_per_unit * cfg.D * e) // 16 * 16
    stream = torch.cuda.current_stream()
    out = {}
    for name, rbytes, wbytes, blocks in (("verify_mix", rd, wr, units), ("verify_reads_only", rd, 0, units),
                                         ("read_1GiB", 1 << 30, 0, 4096)):
        nbuf = max(2, -(-(600 << 20) // rbytes))
        src = torch.empty(nbuf * rbytes, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty(max(16, nbuf * wbytes), dtype=torch.uint8, device="cuda")
        ts = []
        for i in range(reps + 5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = probe.gdntree_probe_stream(src.data_ptr() + (i % nbuf) * rbytes, rbytes,
                                            dst.data_ptr() + (i % nbuf) * wbytes, wbytes, blocks, stream.cuda_stream)
            b.record(stream)
            if st != 0:
                raise RuntimeError(f"stream probe failed: {st}")
            ts.append((a, b))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ts[5:]])) * 1e3
        out[name] = {"read_bytes": rbytes, "write_bytes": wbytes, "blocks": blocks, "median_us": us,
                     "GBps": (rbytes + wbytes) / (us * 1e-6) / 1e9,
                     "frac_of_peak": (rbytes + wbytes) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del src, dst
    return out


def tau_curve(name: str, seeds: int, budgets=(4, 8, 16, 24, 32, 48, 64)) -> None:
    """Exact replay of tau(N): for each node budget N, the library's build and acceptance (one
    launch each, on the GPU) over the workload's seeded lattices and synthetic targets, with the
    mean accepted length tau(N) (accepted drafts + bonus) and each launch's time.  Beside it, the
    lattice-limited tau: the expected tau of a tree holding the whole P x K lattice, where
    acceptance stops only when the target's token is not among a position's K candidates
    (closed form 1 + sum_{d=1..P} (1 - u_b)^d with u_b request b's uniform-token mass), and
    its ratio to tau(N) (the headroom a larger tree could still take).  Prints one JSON line."""
    import numpy as np
    import torch

    import gdn_draft_tree_amd as g
    from workloads import CONFIGS, generate, resolve_target
    from workloads.generate import target_probs

    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    ws = [generate(cfg, seed=s) for s in range(seeds)]
    u = np.concatenate([[target_probs(cfg, float(p))[cfg.K] for p in w.p_top1] for w in ws])
    tau_lat = float(np.mean([1.0 + sum((1.0 - x) ** d for d in range(1, cfg.P + 1)) for x in u]))
    rows = []
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for N in budgets:
        if N > cfg.N:
            continue
        taus, t_build, t_acc = [], [], []
        for w in ws:
            lp, lt, rt = (torch.from_numpy(x).to(dev) for x in (w.lat_logp, w.lat_tok, w.root_tok))
            tree = g.gdntree_build(lp, lt, rt, N)
            torch.cuda.synchronize()
            tgt = resolve_target(tree.depth.cpu().numpy(), tree.n_nodes.cpu().numpy(), w.lat_tok,
                                 w.tgt_choice[:, :N + 1], w.tgt_uniform[:, :N + 1])
            tgt_d = torch.from_numpy(np.ascontiguousarray(tgt)).to(dev)
            acc = g.gdntree_accept(tree, tgt_d, cfg.P)
            p_build = g.gdntree_build(lp, lt, rt, N, out=tree, prepare=True)
            p_acc = g.gdntree_accept(tree, tgt_d, cfg.P, acc=acc, prepare=True)
            for _ in range(3):  # warm
                p_build()
                p_acc()
            e0.record()
            p_build()
            e1.record()
            p_acc()
            e2.record()
            torch.cuda.synchronize()
            t_build.append(e0.elapsed_time(e1) * 1e3)
            t_acc.append(e1.elapsed_time(e2) * 1e3)
            taus.append(acc[0].cpu().numpy())
        tau = np.concatenate(taus)
        rows.append({"N": N, "tau_mean": float(tau.mean()), "tau_hist": np.bincount(tau).tolist(),
                     "lattice_tau_over_tau": tau_lat / float(tau.mean()),
                     "build_us": float(np.median(t_build)), "accept_us": float(np.median(t_acc))})
    print(json.dumps({"metric": "tau(N): mean accepted length per step (accepted drafts + bonus)",
                      "workload": f"{cfg.name}: {cfg.notes}", "requests": cfg.B * seeds,
                      "seeds": seeds, "lattice_tau": tau_lat, "curve": rows,
                      "data": "synthetic lattices and targets (seeded); build and acceptance on the GPU"}))


def markov_timing(name: str, seeds: int, launches: int, R: int = 32) -> None:
    """The Markov-head path alone: parent-conditioned edge log-probs from the head
    (gdntree_markov_edges) and the best-first build over them (gdntree_build_cond), each as
    `launches` launches back to back over `seeds` seeded batches of the workload's shape, timed
    with two events around each batch of launches (medians over five batches).  Prints one JSON
    line."""
    import numpy as np
    import torch

    import gdn_draft_tree_amd as g
    from workloads import CONFIGS, generate, markov_head

    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sets = []
    for s in range(seeds):
        w, mh = generate(cfg, seed=s), markov_head(cfg, seed=s, R=R)
        d = dict(bases=torch.from_numpy(mh.bases).to(dev), lat_tok=torch.from_numpy(w.lat_tok).to(dev),
                 root_tok=torch.from_numpy(w.root_tok).to(dev), W1=torch.from_numpy(mh.W1).to(dev),
                 W2=torch.from_numpy(mh.W2).to(dev))
        d["edge"] = g.gdntree_markov_edges(d["bases"], d["lat_tok"], d["root_tok"], d["W1"], d["W2"])
        d["tree"] = g.gdntree_build_cond(d["edge"], d["lat_tok"], d["root_tok"], cfg.N)
        d["p_edges"] = g.gdntree_markov_edges(d["bases"], d["lat_tok"], d["root_tok"], d["W1"], d["W2"],
                                              out=d["edge"], stream=stream, prepare=True)
        d["p_build"] = g.gdntree_build_cond(d["edge"], d["lat_tok"], d["root_tok"], cfg.N, out=d["tree"],
                                            stream=stream, prepare=True)
        sets.append(d)
    torch.cuda.synchronize()
    n_nodes = torch.cat([d["tree"].n_nodes for d in sets]).cpu().numpy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for what in ("p_edges", "p_build"):
        for i in range(2 * seeds):  # warm
            sets[i % seeds][what]()
        med = []
        for _ in range(5):
            e0.record(stream)
            for i in range(launches):
                sets[i % seeds][what]()
            e1.record(stream)
            torch.cuda.synchronize()
            med.append(e0.elapsed_time(e1) * 1e3 / launches)
        out[what] = float(np.median(med))
    print(json.dumps({"metric": "Markov-head edge log-probs and the conditioned best-first build: us per launch",
                      "workload": f"{cfg.name}: {cfg.notes}", "B": cfg.B, "P": cfg.P, "K": cfg.K, "N": cfg.N,
                      "V": cfg.V, "R": R, "head_dtype": "f32", "seeds": seeds, "launches": launches,
                      "markov_edges_us": out["p_edges"], "build_cond_us": out["p_build"],
                      "mean_nodes": float(n_nodes.mean()),
                      "data": "synthetic head (seeded bases, W1, W2) over the workload's lattice tokens"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ragged")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated through (0: auto)")
    ap.add_argument("--cpu-reqs", type=int, default=32, help="requests per seed the oracle runs on the host")
    ap.add_argument("--cpu-seeds", type=int, default=4, help="input seeds of the multi-process oracle run")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: the CPUs this process may use, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run kernels of known traffic, the reference dispatches for scaling "
                         "hardware byte counters: a plain 256 MiB copy (dst = src * 1) and a 256 MiB "
                         "read of a buffer pushed out of the caches (the streaming probe)")
    ap.add_argument("--tau-curve", action="store_true",
                    help="instead of the step benchmark: replay build + acceptance on the GPU over "
                         "the workload's seeded lattices for a sweep of node budgets N and print tau(N)")
    ap.add_argument("--tau-seeds", type=int, default=8, help="input seeds of the tau(N) replay")
    ap.add_argument("--reps", type=int, default=200,
                    help="verify (and commit) launches timed one by one for the medians (>= 100)")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the streaming probe that measures what this part streams for the verify's bytes")
    ap.add_argument("--deferred-only", type=int, default=0, metavar="K",
                    help="instead of the step benchmark: K launches of the verify with the previous "
                         "step's commit deferred into it (gdntree_accept_commit_verify), back to back over "
                         "the input sets, then exit (a short program for profiler runs)")
    ap.add_argument("--markov-only", type=int, default=0, metavar="K",
                    help="instead of the step benchmark: time the Markov-head edge kernel and the "
                         "conditioned build, K launches back to back each, then exit")
    ap.add_argument("--verify-only", type=int, default=0, metavar="K",
                    help="instead of the step benchmark: K verify launches back to back over the input "
                         "sets, then exit (a short, single-kernel program for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and has no "
              "multi-GPU mode (the verify step shards by request or head with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    if args.tau_curve:
        tau_curve(args.workload, args.tau_seeds)
        return
    if args.markov_only:
        markov_timing(args.workload, 4, args.markov_only)
        return

    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        cfg0 = __import__("workloads").CONFIGS[args.workload]
        cpu = cpu_baseline(args.workload, min(args.cpu_reqs, cfg0.B), args.cpu_seeds, workers)

    import numpy as np
    import torch

    import gdn_draft_tree_amd as g
    from workloads import CONFIGS, generate, resolve_target

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    e = 2 if cfg.dtype == "bf16" else 4
    set_bytes = (5 * cfg.L * cfg.B * cfg.rows * cfg.H * cfg.D * e + cfg.L * cfg.B * cfg.H * cfg.D * cfg.D * 4)
    # enough sets to exceed the 256 MB last-level cache; at most 256 (small workloads are
    # latency-bound, and every set is generated and built up front)
    nsets = args.sets or min(256, max(2, int(np.ceil(600e6 / set_bytes))))

    sets = []
    for s in range(nsets):
        w = generate(cfg, seed=s)
        d = dict(lat_logp=torch.from_numpy(w.lat_logp).to(dev), lat_tok=torch.from_numpy(w.lat_tok).to(dev),
                 root_tok=torch.from_numpy(w.root_tok).to(dev), q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev),
                 alpha=w.alpha.to(dev), beta=w.beta.to(dev), state=w.h0.to(dev))
        if cfg.G is None:
            d["tree"] = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], cfg.N)
        else:
            d["positions"] = None if cfg.positions is None else torch.tensor(cfg.positions_for(), dtype=torch.int32,
                                                                               device=dev)
            d["tree"] = g.gdntree_build_shared(d["lat_logp"], d["lat_tok"], d["root_tok"], cfg.N, cfg.G,
                                               d["positions"])
        torch.cuda.synchronize()
        tgt = resolve_target(d["tree"].depth.cpu().numpy(), d["tree"].n_nodes.cpu().numpy(), w.lat_tok,
                             w.tgt_choice, w.tgt_uniform)
        d["target"] = torch.from_numpy(tgt).to(dev)
        d["o"] = torch.empty(cfg.L, cfg.B, cfg.rows, cfg.H, cfg.D, dtype=w.q.dtype, device=dev)
        d["acc"] = (torch.empty(cfg.B, dtype=torch.int32, device=dev),
                    torch.empty(cfg.B, cfg.P + 1, dtype=torch.int32, device=dev),
                    torch.empty(cfg.B, cfg.P + 1, dtype=torch.int32, device=dev))
        sets.append(d)
        del w
    print(f"# {nsets} input sets of {set_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    # The library calls of every step, validated and marshalled once (binding's prepare=True):
    # the timed loops only enqueue them, so Python's argument checks stay out of the step time.
    for i, d in enumerate(sets):
        dn = sets[(i + 1) % nsets]
        if cfg.G is None:
            d["p_build"] = g.gdntree_build(d["lat_logp"], d["lat_tok"], d["root_tok"], cfg.N, out=d["tree"],
                                           stream=stream, prepare=True)
        else:
            d["p_build"] = g.gdntree_build_shared(d["lat_logp"], d["lat_tok"], d["root_tok"], cfg.N, cfg.G,
                                                  d["positions"], out=d["tree"], stream=stream, prepare=True)
        d["p_verify"] = g.gdntree_verify(d["tree"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"],
                                         o=d["o"], stream=stream, prepare=True)
        d["p_accept_commit"] = g.gdntree_accept_commit(d["tree"], d["target"], d["k"], d["v"], d["alpha"], d["beta"],
                                                       d["state"], cfg.P, acc=d["acc"], stream=stream, prepare=True)
        d["p_accept"] = g.gdntree_accept(d["tree"], d["target"], cfg.P, acc=d["acc"], stream=stream, prepare=True)
        d["p_commit"] = g.gdntree_commit(d["tree"], d["acc"][0], d["acc"][2], d["k"], d["v"], d["alpha"], d["beta"],
                                         d["state"], cfg.P, stream=stream, prepare=True)
        if cfg.G is None:
            # the commit deferred into the next verify: acceptance + next build, then the
            # acceptance + commit of this set's tree inside the verify of the next set's tree
            # (committed into the next set's state: every set carries its own state, so the
            # state buffers rotate with the rows; the work per step is that of a decode loop)
            d["p_accept_build"] = g.gdntree_accept_build(d["tree"], d["target"], cfg.P, dn["lat_logp"], dn["lat_tok"],
                                                         dn["root_tok"], cfg.N, dn["tree"], acc=d["acc"],
                                                         stream=stream, prepare=True)
            d["p_accept_commit_verify"] = g.gdntree_accept_commit_verify(
                d["tree"], d["target"], d["k"], d["v"], d["alpha"], d["beta"], cfg.P, dn["tree"], dn["q"], dn["k"],
                dn["v"], dn["alpha"], dn["beta"], dn["state"], o=dn["o"], stream=stream, prepare=True)
            d["p_accept_commit_build"] = g.gdntree_accept_commit_build(
                d["tree"], d["target"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], cfg.P,
                dn["lat_logp"], dn["lat_tok"], dn["root_tok"], cfg.N, dn["tree"], acc=d["acc"], stream=stream,
                prepare=True)
        else:
            d["p_accept_commit_build"] = g.gdntree_accept_commit_build_shared(
                d["tree"], d["target"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], cfg.P,
                dn["lat_logp"], dn["lat_tok"], dn["root_tok"], cfg.N, cfg.G, dn["tree"],
                next_positions=dn["positions"], acc=d["acc"], stream=stream, prepare=True)

    if args.deferred_only:
        if cfg.G is not None:
            sys.exit("--deferred-only runs without a shared budget")
        for i in range(args.deferred_only):
            sets[i % nsets]["p_accept_commit_verify"]()
        torch.cuda.synchronize()
        if args.copy_calibration:
            calibration_kernels(dev)
        print(json.dumps({"deferred_only": args.deferred_only, "workload": args.workload, "sets": nsets}))
        return

    if args.verify_only:
        for i in range(args.verify_only):
            sets[i % nsets]["p_verify"]()
        torch.cuda.synchronize()
        if args.copy_calibration:
            calibration_kernels(dev)
        print(json.dumps({"verify_only": args.verify_only, "workload": args.workload, "sets": nsets}))
        return

    def step(i, events=None):
        d = sets[i % nsets]
        if events:
            events[0].record(stream)
        d["p_build"]()
        if events:
            events[1].record(stream)
        d["p_verify"]()
        if events:
            events[2].record(stream)
        d["p_accept_commit"]()
        if events:
            events[3].record(stream)

    # Pipelined steps: the end of a step (acceptance and commit) runs in one launch with the
    # next batch's tree build; each request's next build starts in the workgroup that has just
    # walked that request's acceptance (the build stands for the next draft, which needs the
    # accepted tokens); the next verify runs after that launch.  One stream, no events.
    def run_pipelined(i0, k):
        sets[i0 % nsets]["p_build"]()
        for i in range(i0, i0 + k):
            d = sets[i % nsets]
            d["p_verify"]()
            (d["p_accept_commit_build"] if i + 1 < i0 + k else d["p_accept_commit"])()

    # Deferred commit: build(i0) -> verify(i0) -> [accept(i), then per request build(i+1); one
    # launch] -> [accept + commit of step i inside the verify of step i+1; one launch] -> ...;
    # the last step's acceptance and commit on their own.  The same builds, verifies,
    # acceptances and commits as run_pipelined, with the state read once per step.
    def run_deferred(i0, k):
        sets[i0 % nsets]["p_build"]()
        sets[i0 % nsets]["p_verify"]()
        for i in range(i0, i0 + k - 1):
            d = sets[i % nsets]
            d["p_accept_build"]()
            d["p_accept_commit_verify"]()
        sets[(i0 + k - 1) % nsets]["p_accept_commit"]()

    for i in range(args.warmup):
        step(i)
    run_pipelined(0, args.warmup)
    if cfg.G is None:
        run_deferred(0, args.warmup)
    torch.cuda.synchronize()
    if args.copy_calibration:
        calibration_kernels(dev)

    # whole-step throughput (no timing events inside the timed region): pipelined steps (the
    # reported value), then the same steps strictly one after the other
    t0 = time.perf_counter()
    run_pipelined(args.warmup, args.steps)
    t_enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed_seq = time.perf_counter() - t0
    elapsed_def = None
    if cfg.G is None:
        t0 = time.perf_counter()
        run_deferred(args.warmup, args.steps)
        torch.cuda.synchronize()
        elapsed_def = time.perf_counter() - t0

    # per-kernel durations with HIP events on the launch stream
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    t_build = float(np.mean([a.elapsed_time(b) for a, b, _, _ in ev])) * 1e3
    t_verify_step = float(np.mean([b.elapsed_time(c) for _, b, c, _ in ev])) * 1e3
    t_commit = float(np.mean([c.elapsed_time(d_) for _, _, c, d_ in ev])) * 1e3

    # the verify kernel's mean duration for the roofline: the same launches back to back on the
    # launch stream (rotating input sets), two events around each batch of them, so that the
    # per-launch figure carries no event or neighbouring-kernel overhead; the median over five
    # batches, so that one stray delay does not move it
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    batch = max(20, args.steps)
    b2b = []
    for _ in range(5):
        e0.record(stream)
        for i in range(batch):
            sets[(args.warmup + i) % nsets]["p_verify"]()
        e1.record(stream)
        torch.cuda.synchronize()
        b2b.append(e0.elapsed_time(e1) * 1e3 / batch)
    t_verify = float(np.median(b2b))

    # the verify and the commit one launch at a time, each between its own pair of events, over
    # `reps` launches (rotating input sets): medians
    reps = max(100, args.reps)
    vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(vev):
        a.record(stream)
        sets[i % nsets]["p_verify"]()
        b.record(stream)
    torch.cuda.synchronize()
    vus = np.array([a.elapsed_time(b) for a, b in vev]) * 1e3
    vnodes = np.array([int(sets[i % nsets]["tree"].n_nodes.sum()) for i in range(reps)]) * cfg.L
    for i, (a, b) in enumerate(vev):
        d = sets[i % nsets]
        d["p_build"]()   # a fresh tree: the commit below runs on the same (deterministic) tree
        a.record(stream)
        d["p_accept_commit"]()
        b.record(stream)
    torch.cuda.synchronize()
    cus = np.array([a.elapsed_time(b) for a, b in vev]) * 1e3

    # a real model calls verify once per layer: for stacked layers, the same work as L launches
    # of one layer each (back to back, rotating input sets)
    t_verify_layers = None
    if cfg.L > 1:
        nl = max(1, args.steps // 5)
        per_layer = [[g.gdntree_verify(d["tree"], d["q"][l:l + 1], d["k"][l:l + 1], d["v"][l:l + 1],
                                       d["alpha"][l:l + 1], d["beta"][l:l + 1], d["state"][l:l + 1],
                                       o=d["o"][l:l + 1], stream=stream, prepare=True) for l in range(cfg.L)]
                     for d in sets]
        for fn in per_layer[args.warmup % nsets]:  # warm
            fn()
        e0.record(stream)
        for i in range(nl):
            for fn in per_layer[(args.warmup + i) % nsets]:
                fn()
        e1.record(stream)
        torch.cuda.synchronize()
        t_verify_layers = e0.elapsed_time(e1) * 1e3 / nl

    depth = np.concatenate([d["tree"].depth.cpu().numpy()[b, :int(n)] for d in sets
                            for b, n in enumerate(d["tree"].n_nodes.cpu().numpy())])
    # acceptance results exist for the sets the timed and warm-up steps ran on
    used = sets[:min(nsets, args.warmup + args.steps)]
    tau_all = np.concatenate([d["acc"][0].cpu().numpy() for d in used])
    # node counts of the sets the timed steps (and the back-to-back verify launches) ran on
    n_nodes = [int(sets[(args.warmup + i) % nsets]["tree"].n_nodes.sum()) for i in range(args.steps)]
    taus = [int(d["acc"][0].sum()) for d in used]
    nodes_per_step = float(np.mean(n_nodes)) * cfg.L
    ms = elapsed / args.steps * 1e3
    ms_seq = elapsed_seq / args.steps * 1e3
    vbytes = float(np.mean([verify_bytes(cfg, n, e) for n in n_nodes]))
    cbytes = float(np.mean([commit_bytes(cfg, t) for t in taus]))
    achieved = vbytes / (t_verify * 1e-6) / 1e9

    vmed = float(np.median(vus))
    out = {
        "metric": HEADLINE_METRIC, "value": nodes_per_step / (ms * 1e-3),
        "unit": "nodes/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.notes}", "B": cfg.B, "L": cfg.L, "H": cfg.H, "d": cfg.D,
                   "P": cfg.P, "K": cfg.K, "N": cfg.N, "io_dtype": cfg.dtype, "input_sets": nsets,
                   **({} if cfg.G is None else {"G": cfg.G, "positions": list(cfg.positions or ())})},
        "value_is": ("verified (node, layer) pairs per second over whole pipelined steps (build, verify, "
                     "acceptance and commit of every request); the per-layer verify rate by the verify "
                     "kernel's own time is verify_nodes_per_s"),
        "verify_nodes_per_s": float(np.median(vnodes / (vus * 1e-6))),
        "verify_us": {"median": vmed, "p10": float(np.percentile(vus, 10)), "p90": float(np.percentile(vus, 90)),
                      "reps": reps, "mean_back_to_back": t_verify, "back_to_back_batches": [round(x, 2) for x in b2b],
                      "mean_in_step": t_verify_step},
        "commit_us": {"median": float(np.median(cus)), "reps": reps,
                      "what": "acceptance + accepted-path commit (one launch), after a build"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload), "kernel": "verify_kernel",
                     "algorithmic_bytes": vbytes, "mean_us": t_verify,
                     "frac_at_median": vbytes / (vmed * 1e-6) / 1e9 / HBM_PEAK_GBS},
        "kernels_us": {"build": t_build, "verify": t_verify_step, "accept_commit": t_commit,
                       "verify_back_to_back": t_verify},
        "sequential": {"ms_per_step": ms_seq, "value": nodes_per_step / (ms_seq * 1e-3),
                       "order": "build -> verify -> accept_commit, each step after the previous one"},
        "deferred_commit": None if elapsed_def is None else {
            "ms_per_step": elapsed_def / args.steps * 1e3,
            "value": nodes_per_step / (elapsed_def / args.steps),
            "order": ("build -> verify(i0) -> [accept(i), then per request build(i+1); one launch] -> "
                      "[accept(i) + commit(i) + verify(i+1); one launch] -> ...; one stream")},
        "pipelining": ("build -> verify(i) -> [accept(i), then per request build(i+1); commit(i) beside "
                       "them; one launch] -> verify(i+1) ...; one stream") if cfg.G is None else
                      "build_shared -> verify(i) -> [accept(i), then per request build(i+1); commit(i) "
                      "beside them; one launch] -> budget cut of the trees (i+1) -> verify(i+1) ...; one stream",
        "pipelining_leaves_out": ("the drafter: in a decode loop the next lattice comes from a drafter run on "
                                  "the accepted tokens, between acceptance and build; here the lattices are "
                                  "inputs, so the pipelined step hides the build behind the commit as a "
                                  "drafter would hide the commit; the in-order figure is `sequential`"),
        "host_enqueue_us_per_step": t_enqueued / args.steps * 1e6,
        "commit_GBps": cbytes / (t_commit * 1e-6) / 1e9,
        "verify_draft_nodes_per_s": (nodes_per_step - cfg.B * cfg.L) / (vmed * 1e-6),
        "verify_per_layer_launches_us": t_verify_layers,
        "tree": {"depth_max": int(depth.max()), "depth_mean": float(depth.mean()),
                 "depth_hist": np.bincount(depth).tolist(),
                 "tau_hist": np.bincount(tau_all, minlength=2)[1:].tolist()},
        "tau_mean": float(np.mean(taus)) / cfg.B,
        "precision": "state products fp32-exact: every fp32 state entry split into three bf16 parts (its "
                     "24-bit significand exactly) times the bf16 rows on MFMA, fp32 accumulation; Gram "
                     "entries exact products accumulated in fp32; path solves, gates and the per-node "
                     "ancestor sums in fp32; commit in fp32; bf16 rows and outputs; fp64 tree scores",
    }
    if not args.no_stream_ceiling:
        out["stream_ceiling"] = stream_ceiling(cfg, cfg.L * cfg.B * cfg.H,
                                               nodes_per_step / (cfg.L * cfg.B))
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
