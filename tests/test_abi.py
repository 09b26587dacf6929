"""The C-ABI library loads and exports every declared symbol, and its host-side
argument checks return the documented codes before anything is launched.
CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")

T = pytest.importorskip("tree_masked_gated_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_tree_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["gdn_tree_accept", "gdn_tree_accept_ragged", "gdn_tree_build",
                     "gdn_tree_cache_bytes",
                     "gdn_tree_commit", "gdn_tree_commit_ragged", "gdn_tree_commit_verify",
                     "gdn_tree_commit_verify_ragged", "gdn_tree_strerror", "gdn_tree_verify",
                     "gdn_tree_verify_ragged"]
    out = subprocess.run(["nm", "-D", "--defined-only", T.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(T._lib, n)


def test_header_compiles_as_c():
    """The header is plain C: a C compiler accepts it on its own."""
    src = '#include "gdn_tree.h"\nint main(void){gdn_tree_dims d={0};(void)d;return 0;}\n'
    p = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", "-"], input=src, text=True,
                       capture_output=True)
    assert p.returncode == 0, p.stderr


def V(d, ptrs, cache=None):
    return T._lib.gdn_tree_verify(ctypes.byref(d) if d is not None else None, *ptrs,
                                  ctypes.byref(cache) if cache is not None else None, None)


def C(d, ptrs, cache=None, tail=(None, None, None)):
    return T._lib.gdn_tree_commit(ctypes.byref(d) if d is not None else None, *ptrs,
                                  ctypes.byref(cache) if cache is not None else None,
                                  *tail, None)


def CV(d, head, cache_prev, mid, cache):
    r = lambda c: ctypes.byref(c) if c is not None else None
    return T._lib.gdn_tree_commit_verify(r(d), *head, r(cache_prev), *mid, r(cache), None)


FAKE = 0x10000          # a 16-byte-aligned pointer value, never dereferenced here
ODD = 0x10004


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="fake device pointers are only passed where no GPU exists")
def test_error_codes():
    good = T.dims(2, 7, 1, 2, 16, 16, "f32")
    ok8 = [FAKE] * 8
    cache = T.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert V(None, ok8, cache) == -1
    assert V(good, [None] + ok8[1:], cache) == -1
    assert V(good, ok8, None) == -1
    assert V(good, ok8, T.Cache(FAKE, None, FAKE, FAKE, FAKE)) == -1
    assert V(good, ok8, T.Cache(FAKE, FAKE, ODD, FAKE, FAKE)) == -5
    assert V(good, ok8[:3] + [ODD] + ok8[4:], cache) == -5
    assert V(T.dims(2, 7, 1, 2, 16, 16, 5), ok8, cache) == -3
    for bad in [T.dims(-1, 7, 1, 2, 16, 16, 0), T.dims(2, 0, 1, 2, 16, 16, 0),
                T.dims(2, 1025, 1, 2, 16, 16, 0), T.dims(2, 7, 0, 2, 16, 16, 0),
                T.dims(2, 7, 2, 3, 16, 16, 0), T.dims(2, 7, 1, 2, 0, 16, 0),
                T.dims(2, 7, 1, 2, 16, 257, 0)]:
        assert V(bad, ok8, cache) == -2
    # batch 0 launches nothing and succeeds, whatever the pointers
    assert V(T.dims(0, 7, 1, 2, 16, 16, 0), [None] * 8, None) == 0
    ok3 = [FAKE] * 3
    assert C(None, ok3, cache, (FAKE,) * 3) == -1
    assert C(good, ok3, cache, (FAKE, None, FAKE)) == -1
    assert C(good, ok3, cache, (FAKE, FAKE, ODD)) == -5
    assert C(good, [FAKE, ODD, FAKE], cache, (FAKE,) * 3) == -5
    assert C(T.dims(0, 7, 1, 2, 16, 16, 0), [None] * 3, None) == 0
    assert C(T.dims(2, 7, 1, 2, 16, 16, 9), ok3, cache, (FAKE,) * 3) == -3
    # fused commit + verify: the same checks, and the two caches must not share a buffer
    other = T.Cache(FAKE + 256, FAKE + 512, FAKE + 768, FAKE + 1024, FAKE + 1280)
    ok10 = [FAKE] * 10
    assert CV(None, ok3, cache, ok10, other) == -1
    assert CV(good, ok3, None, ok10, other) == -1
    assert CV(good, ok3, cache, ok10[:4] + [None] + ok10[5:], other) == -1
    assert CV(good, ok3, cache, ok10, T.Cache(FAKE, FAKE, ODD, FAKE, FAKE)) == -5
    assert CV(good, [FAKE, ODD, FAKE], cache, ok10, other) == -5
    assert CV(T.dims(2, 7, 1, 2, 16, 16, 5), ok3, cache, ok10, other) == -3
    assert CV(T.dims(2, 0, 1, 2, 16, 16, 0), ok3, cache, ok10, other) == -2
    assert CV(good, ok3, cache, ok10, cache) == -6
    assert CV(good, ok3, other, ok10,
              T.Cache(FAKE, FAKE, FAKE, FAKE + 1280, FAKE)) == -6
    assert CV(T.dims(0, 7, 1, 2, 16, 16, 0), [None] * 3, None, [None] * 10, None) == 0
    # acceptance walk
    AC = lambda d, p: T._lib.gdn_tree_accept(ctypes.byref(d) if d is not None else None, *p, None)
    ok7 = [FAKE] * 7
    assert AC(None, ok7) == -1
    assert AC(good, ok7[:2] + [None] + ok7[3:]) == -1
    assert AC(good, ok7[:6] + [ODD]) == -5
    assert AC(T.dims(2, 2000, 1, 2, 16, 16, 0), ok7) == -2
    assert AC(T.dims(0, 7, 1, 2, 16, 16, 0), [None] * 7) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="fake device pointers are only passed where no GPU exists")
def test_ragged_error_codes():
    """The ragged calls check their offsets pointer (NULL -1, not 4-byte aligned
    -5) after the dims and before everything else, and otherwise run the dense
    calls' checks."""
    r = lambda c: ctypes.byref(c) if c is not None else None
    good = T.dims(2, 7, 1, 2, 16, 16, "f32")
    cache = T.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    other = T.Cache(FAKE + 256, FAKE + 512, FAKE + 768, FAKE + 1024, FAKE + 1280)
    OFF, OFF_ODD = FAKE + 4, FAKE + 2       # int32 alignment suffices for offsets
    VR = lambda d, off, p, c: T._lib.gdn_tree_verify_ragged(r(d), off, *p, r(c), None)
    ok8 = [FAKE] * 8
    assert VR(None, OFF, ok8, cache) == -1
    assert VR(good, None, ok8, cache) == -1
    assert VR(good, OFF_ODD, ok8, cache) == -5
    assert VR(good, OFF, ok8[:7] + [None], cache) == -1
    assert VR(good, OFF, ok8[:3] + [ODD] + ok8[4:], cache) == -5
    assert VR(T.dims(2, 1025, 1, 2, 16, 16, 0), OFF, ok8, cache) == -2
    assert VR(T.dims(0, 7, 1, 2, 16, 16, 0), None, [None] * 8, None) == 0
    CR = lambda d, off, p, c, t: T._lib.gdn_tree_commit_ragged(r(d), off, *p, r(c), *t, None)
    assert CR(good, None, [FAKE] * 3, cache, (FAKE,) * 3) == -1
    assert CR(good, OFF_ODD, [FAKE] * 3, cache, (FAKE,) * 3) == -5
    assert CR(good, OFF, [FAKE] * 3, cache, (FAKE, None, FAKE)) == -1
    assert CR(T.dims(2, 7, 1, 2, 16, 16, 9), OFF, [FAKE] * 3, cache, (FAKE,) * 3) == -3
    CVR = lambda d, op, head, cp, mid, c: T._lib.gdn_tree_commit_verify_ragged(
        r(d), op, *head, r(cp), *mid, r(c), None)
    mid = lambda off: [FAKE] * 3 + [off] + [FAKE] * 7
    assert CVR(good, None, [FAKE] * 3, cache, mid(OFF), other) == -1
    assert CVR(good, OFF, [FAKE] * 3, cache, mid(None), other) == -1
    assert CVR(good, OFF, [FAKE] * 3, cache, mid(OFF_ODD), other) == -5
    assert CVR(good, OFF, [FAKE] * 3, cache, mid(OFF), cache) == -6
    assert CVR(T.dims(0, 7, 1, 2, 16, 16, 0), None, [None] * 3, None, [None] * 11, None) == 0
    ACR = lambda d, off, p: T._lib.gdn_tree_accept_ragged(r(d), off, *p, None)
    ok7 = [FAKE] * 7
    assert ACR(good, None, ok7) == -1
    assert ACR(good, OFF_ODD, ok7) == -5
    assert ACR(good, OFF, ok7[:6] + [ODD]) == -5
    assert ACR(T.dims(0, 7, 1, 2, 16, 16, 0), None, [None] * 7) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="fake device pointers are only passed where no GPU exists")
def test_build_error_codes():
    """Tree construction: sizes (N in [1, 1024], K in [1, 64], w >= 1, the
    working set within LDS), NULL and alignment, batch 0."""
    r = lambda d: ctypes.byref(d) if d is not None else None
    BD = lambda d, p: T._lib.gdn_tree_build(r(d), *p, None)
    ok5 = [FAKE] * 5
    assert BD(None, ok5) == -1
    for bad in [(2, 0, 8, 8), (2, 1025, 8, 8), (2, 128, 0, 8), (2, 128, 65, 8), (2, 128, 8, 0),
                (-1, 128, 8, 8), (2, 1024, 64, 8)]:
        assert BD(T.build_dims(*bad), ok5) == -2, bad
    good = T.build_dims(2, 128, 8, 8)
    assert BD(good, ok5[:2] + [None] + ok5[3:]) == -1
    assert BD(good, ok5[:4] + [ODD]) == -5
    assert BD(T.build_dims(0, 128, 8, 8), [None] * 5) == 0


def test_strerror_and_cache_bytes():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert T.gdn_tree_strerror(code) and T.gdn_tree_strerror(code) != "unknown gdn_status"
    assert T.gdn_tree_strerror(-99) == "unknown gdn_status"
    d = T.dims(3, 70, 2, 4, 32, 64, "bf16")
    b = T.gdn_tree_cache_bytes(d)
    assert b == {"anc_mask": 3 * 70 * 3 * 4, "depth": 3 * 70 * 4, "u": 3 * 4 * 70 * 64 * 4,
                 "log_gamma": 3 * 4 * 70 * 4, "tree_status": 3 * 4}
    with pytest.raises(T.GdnError):
        T.gdn_tree_cache_bytes(T.dims(1, 2000, 1, 1, 16, 16, 0))
