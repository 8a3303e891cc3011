"""Thin ctypes binding over libgdntree.so, with the C ABI's names.

Only argument marshalling happens here: shape/dtype/device checks and pointer extraction
from torch tensors (torch provides device memory and the current stream).  Every step of
the verified path runs in the library's HIP kernels; there is no fallback.  If the shared
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdntree.so")

GDNTREE_OK, GDNTREE_ERR_ARG, GDNTREE_ERR_UNSUPPORTED, GDNTREE_ERR_DEVICE = 0, 1, 2, 3
GDNTREE_F32, GDNTREE_BF16 = 0, 1
EXPORTED = ("gdntree_build", "gdntree_build_shared", "gdntree_verify", "gdntree_accept_commit", "gdntree_accept", "gdntree_commit",
            "gdntree_commit_build", "gdntree_accept_commit_build", "gdntree_accept_commit_build_shared",
            "gdntree_build_cond", "gdntree_markov_edges", "gdntree_accept_build", "gdntree_accept_commit_verify",
            "gdntree_status_str")


class GdnTreeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gdntree status {status}: {message}")
        self.status = status


class CTree(ctypes.Structure):
    _fields_ = [("parent", ctypes.c_void_p), ("depth", ctypes.c_void_p), ("rank", ctypes.c_void_p),
                ("token", ctypes.c_void_p), ("score", ctypes.c_void_p), ("anc", ctypes.c_void_p),
                ("n_nodes", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.gdntree_build.argtypes = [vp, vp, vp, i, i, i, i, CTree, vp]
    lib.gdntree_build.restype = i
    lib.gdntree_build_shared.argtypes = [vp, vp, vp, vp, i, i, i, i, i, CTree, vp]
    lib.gdntree_build_shared.restype = i
    lib.gdntree_build_cond.argtypes = [vp, vp, vp, i, i, i, i, CTree, vp]
    lib.gdntree_build_cond.restype = i
    lib.gdntree_markov_edges.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp]
    lib.gdntree_markov_edges.restype = i
    lib.gdntree_verify.argtypes = [CTree, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, i, vp, vp]
    lib.gdntree_verify.restype = i
    lib.gdntree_accept_commit.argtypes = [CTree, i, i, i, vp, i, i, i, i, i, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp]
    lib.gdntree_accept_commit.restype = i
    lib.gdntree_accept.argtypes = [CTree, i, i, i, vp, vp, vp, vp, vp]
    lib.gdntree_accept.restype = i
    lib.gdntree_commit.argtypes = [CTree, i, i, i, vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp]
    lib.gdntree_commit.restype = i
    lib.gdntree_commit_build.argtypes = [CTree, i, i, i, vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp,
                                         vp, vp, vp, i, i, i, i, CTree, vp]
    lib.gdntree_commit_build.restype = i
    lib.gdntree_accept_commit_build.argtypes = [CTree, i, i, i, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, i, i, i, i, CTree, vp]
    lib.gdntree_accept_commit_build.restype = i
    lib.gdntree_accept_commit_build_shared.argtypes = [CTree, i, i, i, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp,
                                                       vp, vp, vp, vp, vp, vp, i, i, i, i, i, CTree, vp]
    lib.gdntree_accept_commit_build_shared.restype = i
    lib.gdntree_accept_build.argtypes = [CTree, i, i, i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, CTree, vp]
    lib.gdntree_accept_build.restype = i
    lib.gdntree_accept_commit_verify.argtypes = [CTree, i, i, vp, vp, vp, vp, vp, vp, vp, vp, CTree, i, i, i, i, i,
                                                 i, i, vp, vp, vp, vp, vp, vp, i, vp, vp]
    lib.gdntree_accept_commit_verify.restype = i
    lib.gdntree_status_str.argtypes = [i]
    lib.gdntree_status_str.restype = ctypes.c_char_p
    return lib


LIB = _load()


def gdntree_status_str(status: int) -> str:
    return LIB.gdntree_status_str(int(status)).decode()


def _check(status: int) -> None:
    if status != GDNTREE_OK:
        raise GdnTreeError(status, gdntree_status_str(status))


@dataclass
class Tree:
    """Device tensors of a batch of best-first trees ([B][N+1] each, n_nodes [B])."""
    parent: torch.Tensor
    depth: torch.Tensor
    rank: torch.Tensor
    token: torch.Tensor
    score: torch.Tensor
    anc: torch.Tensor
    n_nodes: torch.Tensor

    @staticmethod
    def empty(B: int, N: int, device) -> "Tree":
        i32 = dict(dtype=torch.int32, device=device)
        return Tree(parent=torch.empty(B, N + 1, **i32), depth=torch.empty(B, N + 1, **i32),
                    rank=torch.empty(B, N + 1, **i32), token=torch.empty(B, N + 1, **i32),
                    score=torch.empty(B, N + 1, dtype=torch.float64, device=device),
                    anc=torch.empty(B, N + 1, dtype=torch.int64, device=device),
                    n_nodes=torch.empty(B, **i32))

    @property
    def B(self) -> int:
        return self.parent.shape[0]

    @property
    def N(self) -> int:
        return self.parent.shape[1] - 1

    def c(self) -> CTree:
        for name in ("parent", "depth", "rank", "token", "score", "anc", "n_nodes"):
            t = getattr(self, name)
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"tree.{name} must be a contiguous device tensor")
        return CTree(self.parent.data_ptr(), self.depth.data_ptr(), self.rank.data_ptr(),
                     self.token.data_ptr(), self.score.data_ptr(), self.anc.data_ptr(),
                     self.n_nodes.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return GDNTREE_BF16
    if dtype == torch.float32:
        return GDNTREE_F32
    raise ValueError(f"unsupported dtype {dtype}")


class Prepared:
    """One library call with its arguments validated and marshalled once: calling it enqueues
    the same launch again (same tensors, same stream) with no Python-side checks.  It holds
    references to the tensors it points at."""

    def __init__(self, fn, args, result, keep):
        self._fn = fn
        # ctypes objects of the declared argument types, built once
        self._args = tuple(a if isinstance(a, t) else t(a) for a, t in zip(args, fn.argtypes))
        self.result = result
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))
        return self.result


def _run(fn, args, prepare: bool, result, keep=()):
    """Enqueue now, or (prepare=True) return a Prepared call for repeated launches."""
    if prepare:
        return Prepared(fn, args, result, keep)
    _check(fn(*args))
    return result


def gdntree_build(lat_logp: torch.Tensor, lat_tok: torch.Tensor, root_tok: torch.Tensor, N: int,
                  out: Tree | None = None, stream=None, prepare: bool = False) -> Tree:
    """Best-first tree from a [B][P][K] lattice (sorted along K); see gdntree.h."""
    B, P, K = lat_logp.shape
    out = out if out is not None else Tree.empty(B, N, lat_logp.device)
    args = (_dev(lat_logp, "lat_logp", torch.float32, (B, P, K)),
            _dev(lat_tok, "lat_tok", torch.int32, (B, P, K)),
            _dev(root_tok, "root_tok", torch.int32, (B,)))
    if out.B != B or out.N != N:
        raise ValueError("output tree has the wrong shape")
    return _run(LIB.gdntree_build, (*args, B, P, K, N, out.c(), _stream(stream)), prepare, out,
                (lat_logp, lat_tok, root_tok, out))


def gdntree_build_cond(edge_logp: torch.Tensor, lat_tok: torch.Tensor, root_tok: torch.Tensor, N: int,
                       out: Tree | None = None, stream=None, prepare: bool = False) -> Tree:
    """Best-first tree over parent-conditioned edge log-probs [B][P][K][K]; see gdntree.h."""
    B, P, K, K2 = edge_logp.shape
    if K2 != K:
        raise ValueError("edge_logp must be [B][P][K][K]")
    out = out if out is not None else Tree.empty(B, N, edge_logp.device)
    args = (_dev(edge_logp, "edge_logp", torch.float32, (B, P, K, K)),
            _dev(lat_tok, "lat_tok", torch.int32, (B, P, K)),
            _dev(root_tok, "root_tok", torch.int32, (B,)))
    if out.B != B or out.N != N:
        raise ValueError("output tree has the wrong shape")
    return _run(LIB.gdntree_build_cond, (*args, B, P, K, N, out.c(), _stream(stream)), prepare, out,
                (edge_logp, lat_tok, root_tok, out))


def gdntree_markov_edges(bases: torch.Tensor, lat_tok: torch.Tensor, root_tok: torch.Tensor, W1: torch.Tensor,
                         W2: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                         prepare: bool = False) -> torch.Tensor:
    """Markov-head edge log-probs [B][P][K][K] from base logits [B][P][K] and the head's [V][R]
    embeddings (f32 or bf16, the same dtype); see gdntree.h."""
    B, P, K = bases.shape
    V, R = W1.shape
    if W2.dtype != W1.dtype:
        raise ValueError("W1 and W2 must share a dtype")
    out = out if out is not None else torch.empty(B, P, K, K, dtype=torch.float32, device=bases.device)
    args = (_dev(bases, "bases", torch.float32, (B, P, K)), _dev(lat_tok, "lat_tok", torch.int32, (B, P, K)),
            _dev(root_tok, "root_tok", torch.int32, (B,)), _dev(W1, "W1", W1.dtype, (V, R)),
            _dev(W2, "W2", W1.dtype, (V, R)))
    return _run(LIB.gdntree_markov_edges, (*args, _code(W1.dtype), B, P, K, V, R,
                                           _dev(out, "out", torch.float32, (B, P, K, K)), _stream(stream)),
                prepare, out, (bases, lat_tok, root_tok, W1, W2, out))


def gdntree_build_shared(lat_logp: torch.Tensor, lat_tok: torch.Tensor, root_tok: torch.Tensor, N: int,
                         G: int, positions: torch.Tensor | None = None, out: Tree | None = None,
                         stream=None, prepare: bool = False) -> Tree:
    """Best-first trees of a whole batch under one budget of G draft nodes; request b draws
    from its first positions[b] lattice positions (all P when None); see gdntree.h."""
    B, P, K = lat_logp.shape
    out = out if out is not None else Tree.empty(B, N, lat_logp.device)
    args = (_dev(lat_logp, "lat_logp", torch.float32, (B, P, K)),
            _dev(lat_tok, "lat_tok", torch.int32, (B, P, K)),
            _dev(root_tok, "root_tok", torch.int32, (B,)),
            None if positions is None else _dev(positions, "positions", torch.int32, (B,)))
    if out.B != B or out.N != N:
        raise ValueError("output tree has the wrong shape")
    return _run(LIB.gdntree_build_shared, (*args, B, P, K, N, int(G), out.c(), _stream(stream)), prepare,
                out, (lat_logp, lat_tok, root_tok, positions, out))


def gdntree_verify(tree: Tree, q, k, v, alpha, beta, state, o=None, out_dtype=None, stream=None,
                   prepare: bool = False):
    """Per-node GDN outputs o [L][B][N+1][H][d_v] for every tree slot < n_nodes.

    q, k, v: [L][B][N+1][H][d]; alpha, beta: [L][B][N+1][H] (bf16 or fp32, all the same);
    state: fp32 [L][B][H][d_k][d_v] (the d_k x d_v state S of every head), read only.
    """
    L, B, R, H, D = q.shape
    dt = q.dtype
    out_dtype = out_dtype or dt
    if o is None:
        o = torch.empty(L, B, R, H, D, dtype=out_dtype, device=q.device)
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((q, "q"), (k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    op = _dev(o, "o", out_dtype, (L, B, R, H, D))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    return _run(LIB.gdntree_verify, (tree.c(), B, R - 1, L, H, D, D, _code(dt), *ptrs, sp,
                              _code(out_dtype), op, _stream(stream)), prepare, o,
                (tree, q, k, v, alpha, beta, state, o))


def gdntree_accept_commit(tree: Tree, target_argmax, k, v, alpha, beta, state, P: int,
                          acc=None, stream=None, prepare: bool = False):
    """Greedy acceptance + bonus and in-place commit of the accepted-path state.

    Returns (acc_len [B], acc_tok [B][P+1], acc_node [B][P+1]) int32 device tensors.
    """
    L, B, R, H, D = k.shape
    dt = k.dtype
    if acc is None:
        acc = (torch.empty(B, dtype=torch.int32, device=k.device),
               torch.empty(B, P + 1, dtype=torch.int32, device=k.device),
               torch.empty(B, P + 1, dtype=torch.int32, device=k.device))
    acc_len, acc_tok, acc_node = acc
    tp = _dev(target_argmax, "target_argmax", torch.int32, (B, R))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    ap = (_dev(acc_len, "acc_len", torch.int32, (B,)),
          _dev(acc_tok, "acc_tok", torch.int32, (B, P + 1)),
          _dev(acc_node, "acc_node", torch.int32, (B, P + 1)))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    return _run(LIB.gdntree_accept_commit, (tree.c(), B, R - 1, P, tp, L, H, D, D, _code(dt), *ptrs, sp,
                                     *ap, _stream(stream)), prepare, (acc_len, acc_tok, acc_node),
                (tree, target_argmax, k, v, alpha, beta, state, acc_len, acc_tok, acc_node))


def _acc_buffers(B: int, P: int, device, acc=None):
    if acc is None:
        acc = (torch.empty(B, dtype=torch.int32, device=device),
               torch.empty(B, P + 1, dtype=torch.int32, device=device),
               torch.empty(B, P + 1, dtype=torch.int32, device=device))
    return acc


def gdntree_accept(tree: Tree, target_argmax, P: int, acc=None, stream=None, prepare: bool = False):
    """Greedy acceptance + bonus only (no state is touched).

    Returns (acc_len [B], acc_tok [B][P+1], acc_node [B][P+1]) int32 device tensors.
    """
    B, R = target_argmax.shape
    acc_len, acc_tok, acc_node = _acc_buffers(B, P, target_argmax.device, acc)
    tp = _dev(target_argmax, "target_argmax", torch.int32, (B, R))
    ap = (_dev(acc_len, "acc_len", torch.int32, (B,)),
          _dev(acc_tok, "acc_tok", torch.int32, (B, P + 1)),
          _dev(acc_node, "acc_node", torch.int32, (B, P + 1)))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match target_argmax")
    return _run(LIB.gdntree_accept, (tree.c(), B, R - 1, P, tp, *ap, _stream(stream)), prepare,
                (acc_len, acc_tok, acc_node), (tree, target_argmax, acc_len, acc_tok, acc_node))


def gdntree_commit(tree: Tree, acc_len, acc_node, k, v, alpha, beta, state, P: int, stream=None,
                   prepare: bool = False):
    """In-place commit of the state along an accepted path from gdntree_accept."""
    L, B, R, H, D = k.shape
    dt = k.dtype
    lp = _dev(acc_len, "acc_len", torch.int32, (B,))
    np_ = _dev(acc_node, "acc_node", torch.int32, (B, P + 1))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    return _run(LIB.gdntree_commit, (tree.c(), B, R - 1, P, lp, np_, L, H, D, D, _code(dt), *ptrs, sp,
                                     _stream(stream)), prepare, None,
                (tree, acc_len, acc_node, k, v, alpha, beta, state))


def gdntree_commit_build(tree: Tree, acc_len, acc_node, k, v, alpha, beta, state, P: int,
                         next_lat_logp, next_lat_tok, next_root_tok, next_N: int, next_out: Tree,
                         stream=None, prepare: bool = False):
    """gdntree_commit of this step and gdntree_build of the next step's tree into `next_out`,
    in one launch (enqueue after this step's gdntree_accept)."""
    L, B, R, H, D = k.shape
    dt = k.dtype
    lp = _dev(acc_len, "acc_len", torch.int32, (B,))
    np_ = _dev(acc_node, "acc_node", torch.int32, (B, P + 1))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    Bn, Pn, Kn = next_lat_logp.shape
    nl = _dev(next_lat_logp, "next_lat_logp", torch.float32, (Bn, Pn, Kn))
    nt = _dev(next_lat_tok, "next_lat_tok", torch.int32, (Bn, Pn, Kn))
    nr = _dev(next_root_tok, "next_root_tok", torch.int32, (Bn,))
    if next_out.B != Bn or next_out.N != next_N:
        raise ValueError("next_out does not match the next lattice")
    for f in ("parent", "depth", "rank", "token", "score", "anc"):
        _dev(getattr(next_out, f), f, None, (Bn, next_N + 1))
    _dev(next_out.n_nodes, "n_nodes", torch.int32, (Bn,))
    return _run(LIB.gdntree_commit_build, (tree.c(), B, R - 1, P, lp, np_, L, H, D, D, _code(dt), *ptrs, sp,
                                           nl, nt, nr, Bn, Pn, Kn, next_N, next_out.c(), _stream(stream)),
                prepare, next_out, (tree, acc_len, acc_node, k, v, alpha, beta, state, next_lat_logp,
                                    next_lat_tok, next_root_tok, next_out))


def _next_lattice(next_lat_logp, next_lat_tok, next_root_tok, next_N: int, next_out: Tree):
    Bn, Pn, Kn = next_lat_logp.shape
    ptrs = (_dev(next_lat_logp, "next_lat_logp", torch.float32, (Bn, Pn, Kn)),
            _dev(next_lat_tok, "next_lat_tok", torch.int32, (Bn, Pn, Kn)),
            _dev(next_root_tok, "next_root_tok", torch.int32, (Bn,)))
    if next_out.B != Bn or next_out.N != next_N:
        raise ValueError("next_out does not match the next lattice")
    return (*ptrs, Bn, Pn, Kn, next_N, next_out.c())


def gdntree_accept_commit_build(tree: Tree, target_argmax, k, v, alpha, beta, state, P: int,
                                next_lat_logp, next_lat_tok, next_root_tok, next_N: int, next_out: Tree,
                                acc=None, stream=None, prepare: bool = False):
    """gdntree_accept_commit of this step and gdntree_build of the next step's tree into
    `next_out`, in one launch.  Returns (acc_len, acc_tok, acc_node)."""
    L, B, R, H, D = k.shape
    dt = k.dtype
    acc_len, acc_tok, acc_node = _acc_buffers(B, P, k.device, acc)
    tp = _dev(target_argmax, "target_argmax", torch.int32, (B, R))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    ap = (_dev(acc_len, "acc_len", torch.int32, (B,)),
          _dev(acc_tok, "acc_tok", torch.int32, (B, P + 1)),
          _dev(acc_node, "acc_node", torch.int32, (B, P + 1)))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    nxt = _next_lattice(next_lat_logp, next_lat_tok, next_root_tok, next_N, next_out)
    return _run(LIB.gdntree_accept_commit_build, (tree.c(), B, R - 1, P, tp, L, H, D, D, _code(dt), *ptrs, sp,
                                                  *ap, *nxt, _stream(stream)),
                prepare, (acc_len, acc_tok, acc_node),
                (tree, target_argmax, k, v, alpha, beta, state, acc_len, acc_tok, acc_node, next_lat_logp,
                 next_lat_tok, next_root_tok, next_out))


def gdntree_accept_build(tree: Tree, target_argmax, P: int, next_lat_logp, next_lat_tok, next_root_tok,
                         next_N: int, next_out: Tree, acc=None, stream=None, prepare: bool = False):
    """gdntree_accept of this step and gdntree_build of the next step's tree into `next_out`, in
    one launch (no state touched).  Returns (acc_len, acc_tok, acc_node)."""
    B, R = tree.B, tree.N + 1
    acc_len, acc_tok, acc_node = _acc_buffers(B, P, target_argmax.device, acc)
    tp = _dev(target_argmax, "target_argmax", torch.int32, (B, R))
    ap = (_dev(acc_len, "acc_len", torch.int32, (B,)),
          _dev(acc_tok, "acc_tok", torch.int32, (B, P + 1)),
          _dev(acc_node, "acc_node", torch.int32, (B, P + 1)))
    nxt = _next_lattice(next_lat_logp, next_lat_tok, next_root_tok, next_N, next_out)
    return _run(LIB.gdntree_accept_build, (tree.c(), B, R - 1, P, tp, *ap, *nxt, _stream(stream)),
                prepare, (acc_len, acc_tok, acc_node),
                (tree, target_argmax, acc_len, acc_tok, acc_node, next_lat_logp, next_lat_tok, next_root_tok,
                 next_out))


def gdntree_accept_commit_verify(prev_tree: Tree, prev_target_argmax, prev_k, prev_v, prev_alpha, prev_beta,
                                 prev_P: int, tree: Tree, q, k, v, alpha, beta, state, o=None, acc=None,
                                 out_dtype=None, stream=None, prepare: bool = False):
    """The previous step's acceptance and commit deferred into this step's verify, one launch:
    state <- the previous accepted node's state (in place), then o = the verify of `tree` on
    it.  `acc`: optional (acc_len, acc_tok, acc_node) buffers for the previous step's
    acceptance.  Returns o."""
    L, B, R, H, D = q.shape
    dt = q.dtype
    Rp = prev_tree.N + 1
    out_dtype = out_dtype or dt
    if o is None:
        o = torch.empty(L, B, R, H, D, dtype=out_dtype, device=q.device)
    if prev_tree.B != B:
        raise ValueError("previous tree has the wrong batch size")
    pp = [_dev(prev_target_argmax, "prev_target_argmax", torch.int32, (B, Rp))]
    pp += [_dev(x, nm, dt, (L, B, Rp, H, D)) for x, nm in ((prev_k, "prev_k"), (prev_v, "prev_v"))]
    pp += [_dev(x, nm, dt, (L, B, Rp, H)) for x, nm in ((prev_alpha, "prev_alpha"), (prev_beta, "prev_beta"))]
    if acc is None:
        ap = (None, None, None)
    else:
        ap = (_dev(acc[0], "acc_len", torch.int32, (B,)),
              _dev(acc[1], "acc_tok", torch.int32, (B, prev_P + 1)),
              _dev(acc[2], "acc_node", torch.int32, (B, prev_P + 1)))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((q, "q"), (k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    op = _dev(o, "o", out_dtype, (L, B, R, H, D))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    return _run(LIB.gdntree_accept_commit_verify,
                (prev_tree.c(), Rp - 1, prev_P, *pp, *ap, tree.c(), B, R - 1, L, H, D, D, _code(dt), *ptrs, sp,
                 _code(out_dtype), op, _stream(stream)), prepare, o,
                (prev_tree, prev_target_argmax, prev_k, prev_v, prev_alpha, prev_beta, acc, tree, q, k, v, alpha,
                 beta, state, o))


def gdntree_accept_commit_build_shared(tree: Tree, target_argmax, k, v, alpha, beta, state, P: int,
                                       next_lat_logp, next_lat_tok, next_root_tok, next_N: int, next_G: int,
                                       next_out: Tree, next_positions=None, acc=None, stream=None,
                                       prepare: bool = False):
    """gdntree_accept_commit_build with the next trees built under one budget of next_G draft
    nodes (request b over its next_positions[b] positions).  Returns (acc_len, acc_tok, acc_node)."""
    L, B, R, H, D = k.shape
    dt = k.dtype
    acc_len, acc_tok, acc_node = _acc_buffers(B, P, k.device, acc)
    tp = _dev(target_argmax, "target_argmax", torch.int32, (B, R))
    ptrs = [_dev(x, nm, dt, (L, B, R, H, D)) for x, nm in ((k, "k"), (v, "v"))]
    ptrs += [_dev(x, nm, dt, (L, B, R, H)) for x, nm in ((alpha, "alpha"), (beta, "beta"))]
    sp = _dev(state, "state", torch.float32, (L, B, H, D, D))
    ap = (_dev(acc_len, "acc_len", torch.int32, (B,)),
          _dev(acc_tok, "acc_tok", torch.int32, (B, P + 1)),
          _dev(acc_node, "acc_node", torch.int32, (B, P + 1)))
    if tree.B != B or tree.N != R - 1:
        raise ValueError("tree shape does not match the rows")
    lp, lt, rt, Bn, Pn, Kn, Nn, nc = _next_lattice(next_lat_logp, next_lat_tok, next_root_tok, next_N, next_out)
    pp = None if next_positions is None else _dev(next_positions, "next_positions", torch.int32, (Bn,))
    return _run(LIB.gdntree_accept_commit_build_shared,
                (tree.c(), B, R - 1, P, tp, L, H, D, D, _code(dt), *ptrs, sp, *ap, lp, lt, rt, pp, Bn, Pn, Kn, Nn,
                 int(next_G), nc, _stream(stream)),
                prepare, (acc_len, acc_tok, acc_node),
                (tree, target_argmax, k, v, alpha, beta, state, acc_len, acc_tok, acc_node, next_lat_logp,
                 next_lat_tok, next_root_tok, next_positions, next_out))
