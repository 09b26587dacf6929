"""Python binding of libgdntree.so: rollback-free GDN draft-tree verification on
MI355X (gfx950).

The names mirror the C ABI in include/gdn_tree.h.  This module only marshals
arguments: it checks that each torch tensor has the shape, dtype and
contiguity the C ABI documents (so a kernel never reads past a buffer) and
passes device pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no other path.  PyTorch
provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

__all__ = [
    "GDN_F32", "GDN_BF16", "GdnError", "Dims", "Cache", "lib_path", "dims",
    "gdn_tree_cache_bytes", "gdn_tree_verify", "gdn_tree_commit", "gdn_tree_commit_verify",
    "gdn_tree_accept", "gdn_tree_verify_ragged", "gdn_tree_commit_ragged",
    "gdn_tree_commit_verify_ragged", "gdn_tree_accept_ragged", "check_offsets",
    "BuildDims", "build_dims", "gdn_tree_build",
    "gdn_tree_strerror", "TreeCache",
]

GDN_F32, GDN_BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libgdntree.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build the HIP library first "
        "(python tree_masked_gated_amd/build.py)")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_nodes", "h_k", "h_v", "d_k", "d_v", "io_dtype")]


class BuildDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "n_nodes", "topk", "width")]


class Cache(ctypes.Structure):
    _fields_ = [("anc_mask", ctypes.c_void_p), ("depth", ctypes.c_void_p),
                ("u", ctypes.c_void_p), ("log_gamma", ctypes.c_void_p),
                ("tree_status", ctypes.c_void_p)]


# torch first: its bundled HIP runtime (soname libamdhip64.so.7) then also
# serves this library, so tensors and kernels share one runtime.  Loading the
# library first would pull in a second runtime that cannot see torch's memory.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(lib_path)
_vp, _i = ctypes.c_void_p, ctypes.c_int
_sz = ctypes.POINTER(ctypes.c_size_t)
_lib.gdn_tree_cache_bytes.argtypes = [ctypes.POINTER(Dims), _sz, _sz, _sz, _sz, _sz]
_lib.gdn_tree_cache_bytes.restype = _i
_lib.gdn_tree_verify.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 8 + [ctypes.POINTER(Cache), _vp]
_lib.gdn_tree_verify.restype = _i
_lib.gdn_tree_commit.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 3 + \
    [ctypes.POINTER(Cache)] + [_vp] * 3 + [_vp]
_lib.gdn_tree_commit.restype = _i
_lib.gdn_tree_commit_verify.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 3 + [ctypes.POINTER(Cache)] + \
    [_vp] * 10 + [ctypes.POINTER(Cache), _vp]
_lib.gdn_tree_commit_verify.restype = _i
_lib.gdn_tree_accept.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 7 + [_vp]
_lib.gdn_tree_accept.restype = _i
_lib.gdn_tree_verify_ragged.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 9 + [ctypes.POINTER(Cache), _vp]
_lib.gdn_tree_verify_ragged.restype = _i
_lib.gdn_tree_commit_ragged.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 4 + \
    [ctypes.POINTER(Cache)] + [_vp] * 3 + [_vp]
_lib.gdn_tree_commit_ragged.restype = _i
_lib.gdn_tree_commit_verify_ragged.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 4 + \
    [ctypes.POINTER(Cache)] + [_vp] * 11 + [ctypes.POINTER(Cache), _vp]
_lib.gdn_tree_commit_verify_ragged.restype = _i
_lib.gdn_tree_accept_ragged.argtypes = [ctypes.POINTER(Dims)] + [_vp] * 8 + [_vp]
_lib.gdn_tree_accept_ragged.restype = _i
_lib.gdn_tree_build.argtypes = [ctypes.POINTER(BuildDims)] + [_vp] * 5 + [_vp]
_lib.gdn_tree_build.restype = _i
_lib.gdn_tree_strerror.argtypes = [_i]
_lib.gdn_tree_strerror.restype = ctypes.c_char_p


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {gdn_tree_strerror(code)} ({code})")
        self.code = code


def gdn_tree_strerror(code: int) -> str:
    return _lib.gdn_tree_strerror(int(code)).decode()


def dims(batch, n_nodes, h_k, h_v, d_k, d_v, io_dtype) -> Dims:
    if isinstance(io_dtype, str):
        io_dtype = {"f32": GDN_F32, "bf16": GDN_BF16}[io_dtype]
    return Dims(batch, n_nodes, h_k, h_v, d_k, d_v, io_dtype)


def gdn_tree_cache_bytes(d: Dims) -> Dict[str, int]:
    out = [ctypes.c_size_t() for _ in range(5)]
    rc = _lib.gdn_tree_cache_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in out])
    if rc:
        raise GdnError(rc, "gdn_tree_cache_bytes")
    return dict(zip(("anc_mask", "depth", "u", "log_gamma", "tree_status"),
                    (x.value for x in out)))


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _io_dtype(d: Dims):
    torch = _torch()
    return torch.float32 if d.io_dtype == GDN_F32 else torch.bfloat16


def _ptr(x, shape, dtype, name):
    """Device pointer of x after checking it covers the documented layout.
    Raw integers are taken as device pointers as they are; None gives NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or a device pointer")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class TreeCache:
    """Device buffers of a gdn_tree_cache for one Dims, allocated with torch
    (allocation is plumbing; the library itself allocates nothing)."""

    def __init__(self, d: Dims, device="cuda"):
        torch = _torch()
        B, N, Hv, dv = d.batch, d.n_nodes, d.h_v, d.d_v
        W = (N + 31) // 32
        self.dims = d
        self.anc_mask = torch.zeros((B, N, W), dtype=torch.int32, device=device)
        self.depth = torch.zeros((B, N), dtype=torch.int32, device=device)
        self.u = torch.zeros((B, Hv, N, dv), dtype=torch.float32, device=device)
        self.log_gamma = torch.zeros((B, Hv, N), dtype=torch.float32, device=device)
        self.tree_status = torch.zeros((B,), dtype=torch.int32, device=device)
        sizes = gdn_tree_cache_bytes(d)
        for key, size in sizes.items():
            t = getattr(self, key)
            assert t.numel() * t.element_size() == size, key
        self.struct = Cache(*(getattr(self, key).data_ptr() for key in
                              ("anc_mask", "depth", "u", "log_gamma", "tree_status")))


def _cache_struct(cache):
    if isinstance(cache, TreeCache):
        return cache.struct
    if isinstance(cache, Cache):
        return cache
    raise TypeError("cache: expected TreeCache or Cache")


def gdn_tree_verify(d: Dims, S0, q, k, v, beta, g, parent, o, cache, stream=None) -> None:
    """Enqueue verification of every node of every tree (see gdn_tree.h)."""
    torch = _torch()
    B, N, Hk, Hv, dk, dv = d.batch, d.n_nodes, d.h_k, d.h_v, d.d_k, d.d_v
    io = _io_dtype(d)
    if isinstance(cache, TreeCache):
        _check_cache(cache, d)
    args = [
        _ptr(S0, (B, Hv, dv, dk), torch.float32, "S0"),
        _ptr(q, (B, N, Hk, dk), io, "q"),
        _ptr(k, (B, N, Hk, dk), io, "k"),
        _ptr(v, (B, N, Hv, dv), io, "v"),
        _ptr(beta, (B, N, Hv), torch.float32, "beta"),
        _ptr(g, (B, N, Hv), torch.float32, "g"),
        _ptr(parent, (B, N), torch.int32, "parent"),
        _ptr(o, (B, N, Hv, dv), io, "o"),
    ]
    rc = _lib.gdn_tree_verify(ctypes.byref(d), *args, ctypes.byref(_cache_struct(cache)),
                              _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_verify")


def gdn_tree_commit(d: Dims, S_in, S_out, k, cache, accepted, path, path_len,
                    stream=None) -> None:
    """Enqueue the commit of each sequence's accepted node (see gdn_tree.h)."""
    torch = _torch()
    B, N, Hk, Hv, dk, dv = d.batch, d.n_nodes, d.h_k, d.h_v, d.d_k, d.d_v
    if isinstance(cache, TreeCache):
        _check_cache(cache, d)
    args = [
        _ptr(S_in, (B, Hv, dv, dk), torch.float32, "S_in"),
        _ptr(S_out, (B, Hv, dv, dk), torch.float32, "S_out"),
        _ptr(k, (B, N, Hk, dk), _io_dtype(d), "k"),
    ]
    tail = [
        _ptr(accepted, (B,), torch.int32, "accepted"),
        _ptr(path, (B, N), torch.int32, "path"),
        _ptr(path_len, (B,), torch.int32, "path_len"),
    ]
    rc = _lib.gdn_tree_commit(ctypes.byref(d), *args, ctypes.byref(_cache_struct(cache)),
                              *tail, _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_commit")


def gdn_tree_commit_verify(d: Dims, S_prev, S_new, k_prev, cache_prev, accepted_prev, path_prev,
                           path_len_prev, q, k, v, beta, g, parent, o, cache, stream=None) -> None:
    """Enqueue the previous tree's commit and the new tree's verification as one
    step, the committed state used directly as the new prefix state (see
    gdn_tree.h)."""
    torch = _torch()
    B, N, Hk, Hv, dk, dv = d.batch, d.n_nodes, d.h_k, d.h_v, d.d_k, d.d_v
    io = _io_dtype(d)
    for c in (cache_prev, cache):
        if isinstance(c, TreeCache):
            _check_cache(c, d)
    head = [
        _ptr(S_prev, (B, Hv, dv, dk), torch.float32, "S_prev"),
        _ptr(S_new, (B, Hv, dv, dk), torch.float32, "S_new"),
        _ptr(k_prev, (B, N, Hk, dk), io, "k_prev"),
    ]
    mid = [
        _ptr(accepted_prev, (B,), torch.int32, "accepted_prev"),
        _ptr(path_prev, (B, N), torch.int32, "path_prev"),
        _ptr(path_len_prev, (B,), torch.int32, "path_len_prev"),
        _ptr(q, (B, N, Hk, dk), io, "q"),
        _ptr(k, (B, N, Hk, dk), io, "k"),
        _ptr(v, (B, N, Hv, dv), io, "v"),
        _ptr(beta, (B, N, Hv), torch.float32, "beta"),
        _ptr(g, (B, N, Hv), torch.float32, "g"),
        _ptr(parent, (B, N), torch.int32, "parent"),
        _ptr(o, (B, N, Hv, dv), io, "o"),
    ]
    rc = _lib.gdn_tree_commit_verify(ctypes.byref(d), *head, ctypes.byref(_cache_struct(cache_prev)),
                                     *mid, ctypes.byref(_cache_struct(cache)), _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_commit_verify")


def gdn_tree_accept(d: Dims, parent, draft, target, target_root, accepted, accept_len, next_token,
                    stream=None) -> None:
    """Enqueue the greedy acceptance walk (see gdn_tree.h)."""
    torch = _torch()
    B, N = d.batch, d.n_nodes
    ptrs = [
        _ptr(parent, (B, N), torch.int32, "parent"),
        _ptr(draft, (B, N), torch.int32, "draft"),
        _ptr(target, (B, N), torch.int32, "target"),
        _ptr(target_root, (B,), torch.int32, "target_root"),
        _ptr(accepted, (B,), torch.int32, "accepted"),
        _ptr(accept_len, (B,), torch.int32, "accept_len"),
        _ptr(next_token, (B,), torch.int32, "next_token"),
    ]
    rc = _lib.gdn_tree_accept(ctypes.byref(d), *ptrs, _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_accept")


# ---------------------------------------------------------------- ragged batches
# Per-node arrays packed sequence after sequence: T rows in all (the leading
# extent of every per-node tensor, taken from the first one), sequence b owning
# rows offsets[b] .. offsets[b+1] - 1 (offsets: int32 [B + 1] on the device).


def check_offsets(offsets, d: Dims, T: int) -> None:
    """Host-side check (copies offsets to the host and so synchronises) that
    the offsets describe B trees of at most N nodes inside T rows.  The library
    itself only checks each sequence's own count on the device; an offsets
    array that points past T rows is the caller's error."""
    o = offsets.cpu().tolist() if hasattr(offsets, "cpu") else list(offsets)
    if len(o) != d.batch + 1 or o[0] != 0:
        raise ValueError("offsets: expected B + 1 entries starting at 0")
    if any(b < a or b - a > d.n_nodes for a, b in zip(o, o[1:])):
        raise ValueError("offsets: non-decreasing, at most n_nodes rows per sequence")
    if o[-1] > T:
        raise ValueError(f"offsets: {o[-1]} rows, arrays hold {T}")


def _rows(x, name):
    if isinstance(x, int) or x is None:
        raise TypeError(f"{name}: ragged calls take tensors (their leading extent is T)")
    return int(x.shape[0])


def gdn_tree_verify_ragged(d: Dims, offsets, S0, q, k, v, beta, g, parent, o, cache,
                           stream=None) -> None:
    """Enqueue verification of a batch of trees of different sizes (see
    gdn_tree.h, ragged batches)."""
    torch = _torch()
    B, Hk, Hv, dk, dv = d.batch, d.h_k, d.h_v, d.d_k, d.d_v
    T = _rows(q, "q")
    io = _io_dtype(d)
    if isinstance(cache, TreeCache):
        _check_cache(cache, d)
    args = [
        _ptr(offsets, (B + 1,), torch.int32, "offsets"),
        _ptr(S0, (B, Hv, dv, dk), torch.float32, "S0"),
        _ptr(q, (T, Hk, dk), io, "q"),
        _ptr(k, (T, Hk, dk), io, "k"),
        _ptr(v, (T, Hv, dv), io, "v"),
        _ptr(beta, (T, Hv), torch.float32, "beta"),
        _ptr(g, (T, Hv), torch.float32, "g"),
        _ptr(parent, (T,), torch.int32, "parent"),
        _ptr(o, (T, Hv, dv), io, "o"),
    ]
    rc = _lib.gdn_tree_verify_ragged(ctypes.byref(d), *args, ctypes.byref(_cache_struct(cache)),
                                     _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_verify_ragged")


def gdn_tree_commit_ragged(d: Dims, offsets, S_in, S_out, k, cache, accepted, path, path_len,
                           stream=None) -> None:
    """Enqueue the commit of each sequence's accepted node, ragged layout."""
    torch = _torch()
    B, Hk, Hv, dk, dv = d.batch, d.h_k, d.h_v, d.d_k, d.d_v
    T = _rows(k, "k")
    if isinstance(cache, TreeCache):
        _check_cache(cache, d)
    args = [
        _ptr(offsets, (B + 1,), torch.int32, "offsets"),
        _ptr(S_in, (B, Hv, dv, dk), torch.float32, "S_in"),
        _ptr(S_out, (B, Hv, dv, dk), torch.float32, "S_out"),
        _ptr(k, (T, Hk, dk), _io_dtype(d), "k"),
    ]
    tail = [
        _ptr(accepted, (B,), torch.int32, "accepted"),
        _ptr(path, (T,), torch.int32, "path"),
        _ptr(path_len, (B,), torch.int32, "path_len"),
    ]
    rc = _lib.gdn_tree_commit_ragged(ctypes.byref(d), *args, ctypes.byref(_cache_struct(cache)),
                                     *tail, _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_commit_ragged")


def gdn_tree_commit_verify_ragged(d: Dims, offsets_prev, S_prev, S_new, k_prev, cache_prev,
                                  accepted_prev, path_prev, path_len_prev, offsets, q, k, v, beta,
                                  g, parent, o, cache, stream=None) -> None:
    """Enqueue the previous tree's commit and the new tree's verification as one
    step, ragged layout (each tree its own offsets)."""
    torch = _torch()
    B, Hk, Hv, dk, dv = d.batch, d.h_k, d.h_v, d.d_k, d.d_v
    Tp, T = _rows(k_prev, "k_prev"), _rows(q, "q")
    io = _io_dtype(d)
    for c in (cache_prev, cache):
        if isinstance(c, TreeCache):
            _check_cache(c, d)
    head = [
        _ptr(offsets_prev, (B + 1,), torch.int32, "offsets_prev"),
        _ptr(S_prev, (B, Hv, dv, dk), torch.float32, "S_prev"),
        _ptr(S_new, (B, Hv, dv, dk), torch.float32, "S_new"),
        _ptr(k_prev, (Tp, Hk, dk), io, "k_prev"),
    ]
    mid = [
        _ptr(accepted_prev, (B,), torch.int32, "accepted_prev"),
        _ptr(path_prev, (Tp,), torch.int32, "path_prev"),
        _ptr(path_len_prev, (B,), torch.int32, "path_len_prev"),
        _ptr(offsets, (B + 1,), torch.int32, "offsets"),
        _ptr(q, (T, Hk, dk), io, "q"),
        _ptr(k, (T, Hk, dk), io, "k"),
        _ptr(v, (T, Hv, dv), io, "v"),
        _ptr(beta, (T, Hv), torch.float32, "beta"),
        _ptr(g, (T, Hv), torch.float32, "g"),
        _ptr(parent, (T,), torch.int32, "parent"),
        _ptr(o, (T, Hv, dv), io, "o"),
    ]
    rc = _lib.gdn_tree_commit_verify_ragged(ctypes.byref(d), *head,
                                            ctypes.byref(_cache_struct(cache_prev)), *mid,
                                            ctypes.byref(_cache_struct(cache)), _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_commit_verify_ragged")


def gdn_tree_accept_ragged(d: Dims, offsets, parent, draft, target, target_root, accepted,
                           accept_len, next_token, stream=None) -> None:
    """Enqueue the greedy acceptance walk, ragged layout."""
    torch = _torch()
    B = d.batch
    T = _rows(parent, "parent")
    ptrs = [
        _ptr(offsets, (B + 1,), torch.int32, "offsets"),
        _ptr(parent, (T,), torch.int32, "parent"),
        _ptr(draft, (T,), torch.int32, "draft"),
        _ptr(target, (T,), torch.int32, "target"),
        _ptr(target_root, (B,), torch.int32, "target_root"),
        _ptr(accepted, (B,), torch.int32, "accepted"),
        _ptr(accept_len, (B,), torch.int32, "accept_len"),
        _ptr(next_token, (B,), torch.int32, "next_token"),
    ]
    rc = _lib.gdn_tree_accept_ragged(ctypes.byref(d), *ptrs, _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_accept_ragged")


# ---------------------------------------------------------------- tree construction

def build_dims(batch, n_nodes, topk, width) -> BuildDims:
    return BuildDims(batch, n_nodes, topk, width)


def gdn_tree_build(bd: BuildDims, logp, tok, parent, token, score, stream=None) -> None:
    """Enqueue draft-tree construction with `width` expansions per step from the
    drafter's top-k continuations (see gdn_tree.h)."""
    torch = _torch()
    B, N, K = bd.batch, bd.n_nodes, bd.topk
    ptrs = [
        _ptr(logp, (B, N + 1, K), torch.float32, "logp"),
        _ptr(tok, (B, N + 1, K), torch.int32, "tok"),
        _ptr(parent, (B, N), torch.int32, "parent"),
        _ptr(token, (B, N), torch.int32, "token"),
        _ptr(score, (B, N), torch.float32, "score"),
    ]
    rc = _lib.gdn_tree_build(ctypes.byref(bd), *ptrs, _stream(stream))
    if rc:
        raise GdnError(rc, "gdn_tree_build")


def _check_cache(c: TreeCache, d: Dims):
    cd = c.dims
    if (cd.batch, cd.n_nodes, cd.h_v, cd.d_v) != (d.batch, d.n_nodes, d.h_v, d.d_v):
        raise ValueError("cache was allocated for different dims")
