"""fp64 CPU oracle for GDN draft-tree verification -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports it and it
imports nothing from the HIP library.

``gdn_oracle.c`` walks every node's root-to-node path with the sequential gated
delta rule in fp64 (page "Trees from Marginals: Autoregressive drafting with
factorized priors", section 3, the state-update equation).  This module builds
it with gcc and wraps it with ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math"]

_lib = None


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle into a shared library (gcc, OpenMP, no FMA contraction)."""
    cmd = ["gcc", *_CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    ci = ctypes.c_int
    lib.oracle_tree.argtypes = [ci, ci, i32p, u32p, i32p, i32p]
    lib.oracle_tree.restype = ci
    lib.oracle_verify.argtypes = [ci] * 6 + [f64p] * 6 + [i32p, i32p, ci, ci] + \
        [f64p] * 4 + [i32p] * 3
    lib.oracle_verify.restype = ci
    lib.oracle_accept.argtypes = [ci, ci] + [i32p] * 7
    lib.oracle_accept.restype = ci
    f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
    lib.oracle_build.argtypes = [ci, ci, ci, ci, f32p, i32p, i32p, i32p, f32p]
    lib.oracle_build.restype = ci
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ci
    return lib


def load(path: str = _LIB):
    """Load the built oracle, building it first if it is missing or stale."""
    global _lib
    if path != _LIB:
        return _bind(path)
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = _bind(_LIB)
    return _lib


def tree(parent: np.ndarray, lib=None):
    """Ancestor bit rows, depths and validity of a batch of trees.

    parent: [B][N] int32.  Returns (mask [B][N][ceil(N/32)] uint32,
    depth [B][N] int32, status [B] int32)."""
    lib = lib or load()
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    if parent.ndim == 1:
        parent = parent[None]
    B, N = parent.shape
    W = (N + 31) // 32
    mask = np.zeros((B, N, W), dtype=np.uint32)
    depth = np.zeros((B, N), dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_tree(B, N, parent, mask, depth, status)
    if rc:
        raise ValueError(f"oracle_tree failed: {rc}")
    return mask, depth, status


def accept(parent, draft, target, target_root, lib=None):
    """Greedy acceptance walk (see gdn_oracle.c): parent, draft, target [B][N]
    int32, target_root [B] int32.  Returns (accepted, accept_len, next_token),
    each [B] int32."""
    lib = lib or load()
    f = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    parent, draft, target, target_root = map(f, (parent, draft, target, target_root))
    B, N = parent.shape
    assert draft.shape == (B, N) == target.shape and target_root.shape == (B,)
    acc = np.empty(B, np.int32)
    alen = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    rc = lib.oracle_accept(B, N, parent, draft, target, target_root, acc, alen, nxt)
    if rc:
        raise ValueError(f"oracle_accept failed: {rc}")
    return acc, alen, nxt


def build_tree(logp, tok, n_nodes, width, lib=None):
    """Draft trees of n_nodes nodes built with `width` expansions per step from
    synthetic drafter scores: logp [B][n_nodes + 1][K] float32 (row 0 the
    prefix's K continuations, row 1 + i node i's), tok the same shape, int32.
    Returns (parent, token, score), [B][n_nodes] each (score float32)."""
    lib = lib or load()
    logp = np.ascontiguousarray(logp, dtype=np.float32)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    B, R, K = logp.shape
    assert R == n_nodes + 1 and tok.shape == logp.shape
    parent = np.empty((B, n_nodes), np.int32)
    token = np.empty((B, n_nodes), np.int32)
    score = np.empty((B, n_nodes), np.float32)
    rc = lib.oracle_build(B, n_nodes, K, width, logp, tok, parent, token, score)
    if rc:
        raise ValueError(f"oracle_build failed: {rc}")
    return parent, token, score


def verify(S0, q, k, v, beta, g, parent, accepted, memo=False, nthreads=0, lib=None):
    """Run the oracle on float64 inputs in the library's layouts.

    S0 [B][Hv][dv][dk], q, k [B][N][Hk][dk], v [B][N][Hv][dv], beta, g
    [B][N][Hv], parent [B][N] int32, accepted [B] int32.
    Returns a dict with o, u, log_gamma, S_commit, path, path_len, status."""
    lib = lib or load()
    f = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    S0, q, k, v, beta, g = map(f, (S0, q, k, v, beta, g))
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    accepted = np.ascontiguousarray(accepted, dtype=np.int32)
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, N)
    assert S0.shape == (B, Hv, dv, dk) and beta.shape == (B, N, Hv) == g.shape
    assert parent.shape == (B, N) and accepted.shape == (B,)
    out = {
        "o": np.empty((B, N, Hv, dv)),
        "u": np.empty((B, Hv, N, dv)),
        "log_gamma": np.empty((B, Hv, N)),
        "S_commit": np.empty((B, Hv, dv, dk)),
        "path": np.empty((B, N), dtype=np.int32),
        "path_len": np.empty(B, dtype=np.int32),
        "status": np.empty(B, dtype=np.int32),
    }
    rc = lib.oracle_verify(B, N, Hk, Hv, dk, dv, S0, q, k, v, beta, g, parent,
                           accepted, int(bool(memo)), int(nthreads), out["o"],
                           out["u"], out["log_gamma"], out["S_commit"], out["path"],
                           out["path_len"], out["status"])
    if rc:
        raise ValueError(f"oracle_verify failed: {rc}")
    return out


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
