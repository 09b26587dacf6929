"""GPU parity of the ragged calls: one batch whose trees differ in size, the
per-node arrays packed sequence after sequence and located by offsets.

Each tree is checked against the oracle run on that tree alone, at its own
size: floating point within relative L2 1e-2 per (sequence, value head) unit
(o, u, path log-gates, committed state); the tree's ancestor rows, depths,
status, path and path length bit for bit.  Cache rows past a tree's size must
hold depth -1 and zero ancestor words; o rows outside every tree, and those of
a sequence with unusable offsets, must be left as they were.  A ragged call
whose trees all have N nodes must reproduce the dense call bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-2
SENTINEL = 0x7bcd        # bf16 / int16 pattern written to o before a call


def _announce(what):
    print(f"[gpu-ragged] {what}", flush=True)


def build_case(seed, trees, N, Hk, Hv, d, io="bf16", accepted=None, extra_rows=3,
               bad=None):
    """trees: per-sequence parent arrays (any size <= N, or 0).  bad: index of a
    sequence given unusable offsets (a count of N + 1 rows)."""
    rng = np.random.default_rng(seed)
    B = len(trees)
    lens = [len(p) for p in trees]
    if bad is not None:
        lens[bad] = N + 1
    lay = W.draw_layer(rng, B, N + 1, Hk, Hv, d, io)
    par = np.full((B, N + 1), -1, np.int32)
    for b, p in enumerate(trees):
        par[b, :len(p)] = p
    if accepted is None:
        accepted = [W.pick_leaf(rng, p) if len(p) else -1 for p in trees]
    off = W.ragged_offsets(lens)
    packed = {key: W.pack_rows(lay[key], lens) for key in ("q", "k", "v", "beta", "g")}
    packed["parent"] = W.pack_rows(par, lens)
    T = int(off[-1]) + extra_rows                   # rows past the last tree: untouched
    for key in packed:
        a = packed[key]
        pad = np.zeros((extra_rows,) + a.shape[1:], a.dtype)
        packed[key] = np.ascontiguousarray(np.concatenate([a, pad]))
    assert packed["q"].shape[0] == T
    return {"lay": lay, "par": par, "trees": trees, "lens": lens, "off": off,
            "packed": packed, "accepted": np.asarray(accepted, np.int32), "B": B, "N": N,
            "Hk": Hk, "Hv": Hv, "d": d, "io": io, "bad": bad}


def gpu_ragged(c, in_place=False):
    import torch
    import tree_masked_gated_amd as T
    io, B, N, Hv, d = c["io"], c["B"], c["N"], c["Hv"], c["d"]
    dims = T.dims(B, N, c["Hk"], Hv, d, d, io)
    dev = lambda a, x="": W.to_device(a, x)
    p = c["packed"]
    Tn = p["q"].shape[0]
    off = dev(c["off"])
    if c["bad"] is None:
        T.check_offsets(off, dims, Tn)
    S0 = dev(c["lay"]["S0"])
    S0_before = S0.clone()
    q, k, v = dev(p["q"], io), dev(p["k"], io), dev(p["v"], io)
    o = torch.full((Tn, Hv, d), 0, dtype=q.dtype, device="cuda")
    o.view(torch.int16 if io == "bf16" else torch.int32).fill_(SENTINEL)
    cache = T.TreeCache(dims)
    T.gdn_tree_verify_ragged(dims, off, S0, q, k, v, dev(p["beta"]), dev(p["g"]),
                             dev(p["parent"]), o, cache)
    torch.cuda.synchronize()
    s0_unchanged = bool(torch.equal(S0.view(torch.int32), S0_before.view(torch.int32)))
    S_out = S0 if in_place else torch.empty_like(S0)
    path = torch.full((Tn,), -7, dtype=torch.int32, device="cuda")
    plen = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    T.gdn_tree_commit_ragged(dims, off, S0, S_out, k, cache, dev(c["accepted"]), path, plen)
    torch.cuda.synchronize()
    raw = o.view(torch.int16 if io == "bf16" else torch.int32).cpu().numpy()
    return {"o": W.from_device_f64(o), "o_raw": raw, "u": cache.u.cpu().numpy(),
            "log_gamma": cache.log_gamma.cpu().numpy(),
            "anc_mask": cache.anc_mask.cpu().numpy().view(np.uint32),
            "depth": cache.depth.cpu().numpy(), "status": cache.tree_status.cpu().numpy(),
            "S_commit": S_out.cpu().numpy().astype(np.float64),
            "S0": c["lay"]["S0"].astype(np.float64),
            "path": path.cpu().numpy(), "path_len": plen.cpu().numpy(),
            "s0_unchanged": s0_unchanged}


def oracle_tree_ref(c, b):
    """The oracle on sequence b's tree alone (n_b >= 1 nodes)."""
    import oracle
    n, io = c["lens"][b], c["io"]
    lay = c["lay"]
    f = lambda a: W.io_to_f64(a[b:b + 1, :n], io)
    parent = c["par"][b:b + 1, :n]
    r = oracle.verify(lay["S0"][b:b + 1].astype(np.float64), f(lay["q"]), f(lay["k"]), f(lay["v"]),
                      lay["beta"][b:b + 1, :n].astype(np.float64),
                      lay["g"][b:b + 1, :n].astype(np.float64), parent,
                      c["accepted"][b:b + 1], memo=True)
    mask, depth, status = oracle.tree(parent)
    r.update(anc_mask=mask, depth=depth, tree_status=status)
    return r


def compare(c, x, tol=TOL):
    B, N, Hv = c["B"], c["N"], c["Hv"]
    off, lens = c["off"], c["lens"]
    assert x["s0_unchanged"], "verify wrote S0"
    covered = np.zeros(x["o_raw"].shape[0], bool)
    worst = {"o": 0.0, "u": 0.0, "log_gamma": 0.0, "S_commit": 0.0}
    for b in range(B):
        n, r0 = lens[b], int(off[b])
        if b == c["bad"]:
            assert x["status"][b] == -1 and x["path_len"][b] == -1, b
            assert np.array_equal(x["S_commit"][b], x["S0"][b]), b
            assert (x["depth"][b] == -1).all() and not x["anc_mask"][b].any(), b
            continue
        covered[r0:r0 + n] = True
        assert (x["depth"][b, n:] == -1).all(), ("depth past n", b)
        assert not x["anc_mask"][b, n:].any(), ("anc_mask past n", b)
        if n == 0:
            assert x["status"][b] == 0, b
            assert x["path_len"][b] == (0 if c["accepted"][b] == -1 else -1), b
            assert np.array_equal(x["S_commit"][b], x["S0"][b]), b
            continue
        ref = oracle_tree_ref(c, b)
        Wb = ref["anc_mask"].shape[-1]
        assert x["status"][b] == ref["tree_status"][0], ("status", b)
        assert np.array_equal(x["anc_mask"][b, :n, :Wb], ref["anc_mask"][0]), ("anc_mask", b)
        assert not x["anc_mask"][b, :n, Wb:].any(), ("anc_mask words", b)
        assert np.array_equal(x["depth"][b, :n], ref["depth"][0]), ("depth", b)
        assert x["path_len"][b] == ref["path_len"][0], ("path_len", b)
        assert np.array_equal(x["path"][r0:r0 + n], ref["path"][0]), ("path", b)
        for h in range(Hv):
            worst["S_commit"] = max(worst["S_commit"], rel_l2(x["S_commit"][b, h], ref["S_commit"][0, h]))
        if ref["tree_status"][0]:
            assert np.isnan(x["o"][r0:r0 + n]).all(), ("o not NaN", b)
            continue
        assert np.isfinite(x["o"][r0:r0 + n]).all(), ("o not finite", b)
        for h in range(Hv):
            worst["o"] = max(worst["o"], rel_l2(x["o"][r0:r0 + n, h], ref["o"][0, :, h]))
            worst["u"] = max(worst["u"], rel_l2(x["u"][b, h, :n], ref["u"][0, h]))
            worst["log_gamma"] = max(worst["log_gamma"],
                                     rel_l2(x["log_gamma"][b, h, :n], ref["log_gamma"][0, h]))
    untouched = x["o_raw"][~covered]
    assert (untouched == SENTINEL).all(), "o rows outside the trees were written"
    _announce(f"  max unit rel-L2 {worst}")
    for key, e in worst.items():
        assert e <= tol, (key, e)


def run(name, c, in_place=False):
    _announce(f"{name} B={c['B']} N={c['N']} lens={c['lens']} Hk={c['Hk']} Hv={c['Hv']} "
              f"d={c['d']} io={c['io']}")
    x = gpu_ragged(c, in_place)
    compare(c, x)
    return x


def mixed_trees(rng, N, sizes):
    out = []
    for i, n in enumerate(sizes):
        if n == 0:
            out.append(np.zeros(0, np.int32))
        elif i % 3 == 0:
            out.append(W.tree_random_recursive(rng, n))
        elif i % 3 == 1:
            out.append(W.tree_chain(n))
        else:
            out.append(W.tree_mary(rng, 4, -(-n // 4))[:n].copy())
    return out


@pytest.mark.parametrize("N,Hk,Hv,sizes", [
    (128, 1, 2, [128, 64, 17, 1, 0, 100, 33, 128]),       # 16-block rows, two heads per wave
    (64, 2, 4, [64, 5, 0, 48, 63, 16, 1]),                 # 4-block rows
    (64, 2, 6, [1, 64, 0, 31]),                            # 4-block rows, one head per wave
    (96, 1, 3, [96, 40, 0, 7]),                            # one head per wave
])
def test_ragged_tiled(N, Hk, Hv, sizes):
    rng = np.random.default_rng(300 + N)
    c = build_case(301 + N, mixed_trees(rng, N, sizes), N, Hk, Hv, 128)
    run("tiled", c)


@pytest.mark.parametrize("N,sizes", [
    (256, [256, 129, 0, 30, 200, 1, 5, 16]),         # chains of 129, 200, 16 and 1 nodes
    (512, [512, 300, 17, 0, 511, 40, 3, 9]),         # chains of 300, 511 and 9 nodes
    (1024, [1024, 600, 0, 1023, 513, 130, 7, 1]),    # chains of 600, 513 and 1 nodes
])
def test_ragged_large(N, sizes):
    rng = np.random.default_rng(310 + N)
    c = build_case(311 + N, mixed_trees(rng, N, sizes), N, 1, 2, 128)
    run("large", c)


@pytest.mark.parametrize("N,d,io,sizes", [
    (40, 64, "bf16", [40, 3, 0, 27]),
    (33, 16, "f32", [1, 33, 0, 20, 9]),
    (200, 128, "f32", [200, 7, 0, 150]),
])
def test_ragged_generic(N, d, io, sizes):
    rng = np.random.default_rng(320 + N + d)
    c = build_case(321 + N + d, mixed_trees(rng, N, sizes), N, 1, 2, d, io)
    run("generic", c)


@pytest.mark.parametrize("N,d,io", [(128, 128, "bf16"), (300, 128, "bf16"), (50, 32, "f32")])
def test_ragged_bad_offsets_and_invalid_tree(N, d, io):
    """A sequence whose offsets give more than N rows is skipped with status -1;
    an invalid parent row gives NaN o rows for that tree only; accepted = -1
    and an accepted node past the tree's size commit nothing."""
    rng = np.random.default_rng(330 + N)
    trees = mixed_trees(rng, N, [N, N // 2, 9, N - 1, 5])
    trees[2] = trees[2].copy()
    trees[2][4] = 6                                   # forward parent: invalid tree
    acc = [W.pick_leaf(rng, trees[0]), -1, 3, W.pick_leaf(rng, trees[3]), 5]   # 5 is past tree 4
    c = build_case(331 + N, trees, N, 1, 2, d, io, accepted=acc, bad=1)
    x = run("bad offsets", c)
    assert x["path_len"][4] == -1 and x["path_len"][2] == -1


def test_ragged_full_equals_dense():
    """Every tree at N nodes: the ragged call gives the dense call's bytes."""
    import torch
    import tree_masked_gated_amd as T
    from gpu_harness import gpu_run
    rng = np.random.default_rng(340)
    N, B = 128, 4
    trees = [W.tree_mary(rng, 8, 16) for _ in range(B)]
    c = build_case(341, trees, N, 2, 4, 128, extra_rows=0)
    _announce("full == dense")
    x = gpu_ragged(c)
    lay = {key: c["lay"][key][:, :N] for key in ("q", "k", "v", "beta", "g")}
    lay["S0"] = c["lay"]["S0"]
    y = gpu_run(c["par"][:, :N], c["accepted"], lay, "bf16", 2, 4)
    for key in ("u", "log_gamma", "anc_mask", "depth", "status", "path_len"):
        assert np.array_equal(x[key], y[key]), key
    assert np.array_equal(x["path"], y["path"].reshape(-1))
    assert np.array_equal(x["S_commit"], y["S_commit"])
    assert np.array_equal(x["o"].reshape(y["o"].shape), y["o"])
    torch.cuda.synchronize()


def test_ragged_accept():
    """The acceptance walk per packed tree against the oracle's walk on that
    tree alone; a sequence with unusable offsets gets accepted = -1, length -1."""
    import torch
    import oracle
    import tree_masked_gated_amd as T
    rng = np.random.default_rng(350)
    N = 300
    trees = mixed_trees(rng, N, [300, 1, 0, 77, 150, 2])
    lens = [len(p) for p in trees]
    lens_dev = list(lens)
    lens_dev[5] = N + 1                                # unusable: skipped
    off = W.ragged_offsets(lens_dev)
    Tn = int(off[-1])
    par = np.full(Tn, -1, np.int32)
    draft = rng.integers(0, 5, Tn).astype(np.int32)   # small vocabulary: long walks
    target = rng.integers(0, 5, Tn).astype(np.int32)
    root = rng.integers(0, 5, len(trees)).astype(np.int32)
    for b, p in enumerate(trees):
        par[off[b]:off[b] + len(p)] = p
    dims = T.dims(len(trees), N, 1, 1, 16, 16, "f32")
    dev = lambda a: W.to_device(a)
    outs = [torch.full((len(trees),), -7, dtype=torch.int32, device="cuda") for _ in range(3)]
    _announce(f"accept ragged lens={lens_dev}")
    T.gdn_tree_accept_ragged(dims, dev(off), dev(par), dev(draft), dev(target), dev(root), *outs)
    acc, alen, nxt = (t.cpu().numpy() for t in outs)
    for b, n in enumerate(lens):
        if b == 5:
            assert (acc[b], alen[b], nxt[b]) == (-1, -1, root[b])
            continue
        if n == 0:
            assert (acc[b], alen[b], nxt[b]) == (-1, 0, root[b])
            continue
        sl = slice(int(off[b]), int(off[b]) + n)
        ra, rl, rn = oracle.accept(par[None, sl], draft[None, sl], target[None, sl], root[b:b + 1])
        assert (acc[b], alen[b], nxt[b]) == (ra[0], rl[0], rn[0]), b


def test_ragged_fused_decode_loop():
    """Three decode steps whose trees change size from step to step, each step
    one fused commit (previous tree) + verify (new tree) call, against the
    oracle chained per sequence; and against the same loop as two calls."""
    fused_loop_case(360, 128, 1, 2, 128,
                    [[128, 64, 0, 33, 100], [16, 128, 77, 0, 1], [64, 64, 64, 64, 64]])


@pytest.mark.parametrize("N,B,lo", [(128, 64, 16), (64, 32, 0)])
def test_ragged_fused_full_batch(N, B, lo):
    """The same loop in the ragged benchmark's launch configuration: 64
    sequences with trees of 16 .. 128 nodes, 16 key / 32 value heads, so the
    persistent fused launch takes several items per workgroup, largest tree
    first; and 32 sequences of 0 .. 64 nodes on the split-column form."""
    rng = np.random.default_rng(365 + N)
    sizes = [[int(x) for x in rng.integers(lo, N + 1, B)] for _ in range(3)]
    fused_loop_case(366 + N, N, 16, 32, 128, sizes)


def fused_loop_case(seed, N, Hk, Hv, d, sizes):
    import torch
    import oracle
    import tree_masked_gated_amd as T
    rng = np.random.default_rng(seed)
    B = len(sizes[0])
    steps = []
    for st, sz in enumerate(sizes):
        trees = mixed_trees(rng, N, sz)
        acc = [W.pick_leaf(rng, p) if len(p) else -1 for p in trees]
        steps.append(build_case(seed + 10 + st, trees, N, Hk, Hv, d, accepted=acc, extra_rows=1))
    # every step starts from the first step's S0, carried forward
    dims = T.dims(B, N, Hk, Hv, d, d, "bf16")
    dev = lambda a, x="": W.to_device(a, x)

    def loop(fused):
        caches = [T.TreeCache(dims), T.TreeCache(dims)]
        S = dev(steps[0]["lay"]["S0"])
        bufs = []
        for c in steps:
            p = c["packed"]
            Tn = p["q"].shape[0]
            bufs.append({"off": dev(c["off"]), "q": dev(p["q"], "bf16"), "k": dev(p["k"], "bf16"),
                         "v": dev(p["v"], "bf16"), "beta": dev(p["beta"]), "g": dev(p["g"]),
                         "parent": dev(p["parent"]), "acc": dev(c["accepted"]),
                         "o": torch.empty((Tn, Hv, d), dtype=torch.bfloat16, device="cuda"),
                         "path": torch.full((Tn,), -7, dtype=torch.int32, device="cuda"),
                         "plen": torch.full((B,), -7, dtype=torch.int32, device="cuda")})
            T.check_offsets(bufs[-1]["off"], dims, Tn)
        x = bufs[0]
        T.gdn_tree_verify_ragged(dims, x["off"], S, x["q"], x["k"], x["v"], x["beta"], x["g"],
                                 x["parent"], x["o"], caches[0])
        states, us = [], []
        for t, x in enumerate(bufs):
            prev = caches[t % 2]
            S_new = torch.empty_like(S)
            if t + 1 < len(bufs):
                y = bufs[t + 1]
                if fused:
                    T.gdn_tree_commit_verify_ragged(dims, x["off"], S, S_new, x["k"], prev, x["acc"],
                                                    x["path"], x["plen"], y["off"], y["q"], y["k"],
                                                    y["v"], y["beta"], y["g"], y["parent"], y["o"],
                                                    caches[(t + 1) % 2])
                else:
                    T.gdn_tree_commit_ragged(dims, x["off"], S, S_new, x["k"], prev, x["acc"],
                                             x["path"], x["plen"])
                    T.gdn_tree_verify_ragged(dims, y["off"], S_new, y["q"], y["k"], y["v"], y["beta"],
                                             y["g"], y["parent"], y["o"], caches[(t + 1) % 2])
            else:
                T.gdn_tree_commit_ragged(dims, x["off"], S, S_new, x["k"], prev, x["acc"],
                                         x["path"], x["plen"])
            torch.cuda.synchronize()
            us.append(prev.u.cpu().numpy())
            states.append(S_new.cpu().numpy().astype(np.float64))
            S = S_new
        return [{"o": W.from_device_f64(x["o"]), "path": x["path"].cpu().numpy(),
                 "path_len": x["plen"].cpu().numpy(), "S": s, "u": u}
                for x, s, u in zip(bufs, states, us)]

    _announce(f"fused ragged loop sizes={sizes}")
    fz = loop(True)
    sp = loop(False)
    S = steps[0]["lay"]["S0"].astype(np.float64)
    for t, c in enumerate(steps):
        for b in range(B):
            n, r0 = c["lens"][b], int(c["off"][b])
            if n == 0:
                assert fz[t]["path_len"][b] == 0
                assert np.array_equal(fz[t]["S"][b], fz[t - 1]["S"][b] if t else S[b].astype(np.float32))
                continue
            f = lambda a: W.io_to_f64(a[b:b + 1, :n], "bf16")
            lay = c["lay"]
            ref = oracle.verify(S[b:b + 1], f(lay["q"]), f(lay["k"]), f(lay["v"]),
                                lay["beta"][b:b + 1, :n].astype(np.float64),
                                lay["g"][b:b + 1, :n].astype(np.float64), c["par"][b:b + 1, :n],
                                c["accepted"][b:b + 1], memo=True)
            assert fz[t]["path_len"][b] == ref["path_len"][0], (t, b)
            assert np.array_equal(fz[t]["path"][r0:r0 + n], ref["path"][0]), (t, b)
            for h in range(Hv):
                assert rel_l2(fz[t]["o"][r0:r0 + n, h], ref["o"][0, :, h]) <= TOL, (t, b, h)
                assert rel_l2(fz[t]["S"][b, h], ref["S_commit"][0, h]) <= TOL, (t, b, h)
            S[b] = ref["S_commit"][0]
        assert np.array_equal(fz[t]["path"], sp[t]["path"]), t
        assert np.array_equal(fz[t]["path_len"], sp[t]["path_len"]), t
        assert rel_l2(fz[t]["S"], sp[t]["S"]) <= 1e-5, t
