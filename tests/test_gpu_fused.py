"""GPU parity of the fused step gdn_tree_commit_verify: a decode loop of several
trees, each step committing the previous tree's accepted node and verifying the
next tree in one call, against the oracle run tree by tree (each tree's prefix
state is the oracle's commit of the one before).

Floating point: relative L2 error <= 1e-2 per (sequence, value head) unit on o,
u, the path log-gates and every committed state.  Integer results (the new
tree's ancestor rows, depths and status; the previous tree's path and its
length) must match bit for bit.  The same loop run as separate commit and
verify calls must agree with the fused one to fp32 rounding.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _announce(what):
    print(f"[gpu-fused] {what}", flush=True)


def gpu_chain(steps, io, Hk, Hv, fused=True, in_place=False, device="cuda"):
    """steps: list of (parent, accepted, layer dict); the first layer's S0 is the
    loop's initial state.  Returns per step the outputs of its verify and of its
    commit, read back once the loop is done."""
    import torch
    import tree_masked_gated_amd as T
    B, N = steps[0][0].shape
    d = steps[0][2]["S0"].shape[-1]
    dims = T.dims(B, N, Hk, Hv, d, d, io)
    caches = [T.TreeCache(dims, device), T.TreeCache(dims, device)]
    S = W.to_device(steps[0][2]["S0"], device=device)
    dev = []
    for parent, accepted, lay in steps:
        dev.append({
            "q": W.to_device(lay["q"], io, device), "k": W.to_device(lay["k"], io, device),
            "v": W.to_device(lay["v"], io, device), "beta": W.to_device(lay["beta"], device=device),
            "g": W.to_device(lay["g"], device=device),
            "parent": W.to_device(parent.astype(np.int32), device=device),
            "acc": W.to_device(np.asarray(accepted, np.int32), device=device),
            "path": torch.full((B, N), -7, dtype=torch.int32, device=device),
            "plen": torch.full((B,), -7, dtype=torch.int32, device=device),
        })
        dev[-1]["o"] = torch.empty((B, N, Hv, d), dtype=dev[-1]["q"].dtype, device=device)
    out = []
    states = []
    x = dev[0]
    T.gdn_tree_verify(dims, S, x["q"], x["k"], x["v"], x["beta"], x["g"], x["parent"], x["o"],
                      caches[0])
    for t in range(len(steps)):
        x = dev[t]
        prev_cache = caches[t % 2]
        S_new = S if in_place else torch.empty_like(S)
        if t + 1 < len(steps):
            y = dev[t + 1]
            if fused:
                T.gdn_tree_commit_verify(dims, S, S_new, x["k"], prev_cache, x["acc"], x["path"],
                                         x["plen"], y["q"], y["k"], y["v"], y["beta"], y["g"],
                                         y["parent"], y["o"], caches[(t + 1) % 2])
            else:
                T.gdn_tree_commit(dims, S, S_new, x["k"], prev_cache, x["acc"], x["path"],
                                  x["plen"])
                T.gdn_tree_verify(dims, S_new, y["q"], y["k"], y["v"], y["beta"], y["g"],
                                  y["parent"], y["o"], caches[(t + 1) % 2])
        else:
            T.gdn_tree_commit(dims, S, S_new, x["k"], prev_cache, x["acc"], x["path"], x["plen"])
        torch.cuda.synchronize()
        # this tree's cache is overwritten two steps on: read it now
        out.append({
            "u": prev_cache.u.cpu().numpy(), "log_gamma": prev_cache.log_gamma.cpu().numpy(),
            "anc_mask": prev_cache.anc_mask.cpu().numpy().view(np.uint32),
            "depth": prev_cache.depth.cpu().numpy(), "status": prev_cache.tree_status.cpu().numpy(),
        })
        states.append(S_new.cpu().numpy().astype(np.float64))
        S = S_new
    torch.cuda.synchronize()
    for t, x in enumerate(dev):
        out[t].update(o=W.from_device_f64(x["o"]), path=x["path"].cpu().numpy(),
                      path_len=x["plen"].cpu().numpy(), S_commit=states[t])
    return out


def oracle_chain(steps, io):
    import oracle
    f = lambda a: W.io_to_f64(a, io)
    S = steps[0][2]["S0"].astype(np.float64)
    refs = []
    for parent, accepted, lay in steps:
        r = oracle.verify(S, f(lay["q"]), f(lay["k"]), f(lay["v"]), lay["beta"].astype(np.float64),
                          lay["g"].astype(np.float64), parent, np.asarray(accepted, np.int32),
                          memo=True)
        mask, depth, status = oracle.tree(parent)
        r.update(anc_mask=mask, depth=depth, tree_status=status)
        refs.append(r)
        S = r["S_commit"]
    return refs


def compare(gpu, ref, Hv, tol=TOL):
    worst = {"o": 0.0, "u": 0.0, "log_gamma": 0.0, "S_commit": 0.0}
    for t, (x, r) in enumerate(zip(gpu, ref)):
        assert np.array_equal(x["status"], r["tree_status"]), ("status", t)
        assert np.array_equal(x["anc_mask"], r["anc_mask"]), ("anc_mask", t)
        assert np.array_equal(x["depth"], r["depth"]), ("depth", t)
        assert np.array_equal(x["path_len"], r["path_len"]), ("path_len", t)
        assert np.array_equal(x["path"], r["path"]), ("path", t)
        B = x["o"].shape[0]
        for b in range(B):
            worst["S_commit"] = max(worst["S_commit"],
                                    max(rel_l2(x["S_commit"][b, h], r["S_commit"][b, h])
                                        for h in range(Hv)))
            if r["tree_status"][b]:
                assert np.isnan(x["o"][b]).all(), ("o not NaN", t, b)
                continue
            assert np.isfinite(x["o"][b]).all(), ("o not finite", t, b)
            for h in range(Hv):
                worst["o"] = max(worst["o"], rel_l2(x["o"][b, :, h], r["o"][b, :, h]))
                worst["u"] = max(worst["u"], rel_l2(x["u"][b, h], r["u"][b, h]))
                worst["log_gamma"] = max(worst["log_gamma"],
                                         rel_l2(x["log_gamma"][b, h], r["log_gamma"][b, h]))
    _announce(f"  max unit rel-L2 {worst}")
    for key, e in worst.items():
        assert e <= tol, (key, e)


def run_case(name, steps, io, Hk, Hv, in_place=False):
    B, N = steps[0][0].shape
    _announce(f"{name} steps={len(steps)} B={B} N={N} Hk={Hk} Hv={Hv} "
              f"d={steps[0][2]['S0'].shape[-1]} io={io} in_place={in_place}")
    fused = gpu_chain(steps, io, Hk, Hv, fused=True, in_place=in_place)
    ref = oracle_chain(steps, io)
    compare(fused, ref, Hv)
    sep = gpu_chain(steps, io, Hk, Hv, fused=False, in_place=in_place)
    for t, (x, y) in enumerate(zip(fused, sep)):
        for key in ("path", "path_len", "anc_mask", "depth", "status"):
            assert np.array_equal(x[key], y[key]), (key, t)
        ok = ref[t]["tree_status"] == 0
        assert rel_l2(x["S_commit"], y["S_commit"]) <= 1e-5, ("S_commit", t)
        # S enters the Gram products in bf16: an fp32 rounding difference in the
        # committed state can move a bf16 rounding, so u is compared looser
        assert rel_l2(x["log_gamma"][ok], y["log_gamma"][ok]) <= 1e-6, ("log_gamma", t)
        assert rel_l2(x["u"][ok], y["u"][ok]) <= 1e-4, ("u", t)
        assert rel_l2(x["o"][ok], y["o"][ok]) <= 1e-3, ("o", t)
    return fused, ref


def chain_steps(seed, parents_per_step, accepted_per_step, Hk, Hv, d, io="bf16"):
    rng = np.random.default_rng(seed)
    steps = []
    for parents, acc in zip(parents_per_step, accepted_per_step):
        parent = np.stack([np.asarray(p, np.int32) for p in parents])
        lay = W.draw_layer(rng, parent.shape[0], parent.shape[1], Hk, Hv, d, io)
        steps.append((parent, np.asarray(acc, np.int32), lay))
    return steps


def test_fused_decode_loop_mixed():
    """Three steps over 64-node trees of every shape, with nothing accepted,
    the root only, a leaf, an invalid previous tree and an invalid new tree."""
    rng = np.random.default_rng(80)
    N = 64
    trees = lambda: [W.tree_random_recursive(rng, N), W.tree_chain(N), W.tree_star(N),
                     W.tree_random_recursive(rng, N), W.tree_chain(N),
                     W.tree_random_recursive(rng, N)]
    p0, p1, p2 = trees(), trees(), trees()
    p1[4] = p1[4].copy(); p1[4][10] = 40          # forward parent: step 1, sequence 4 invalid
    acc = lambda ps: [W.pick_leaf(rng, ps[0]), N - 1, -1, 0, N - 1, W.pick_leaf(rng, ps[5])]
    steps = chain_steps(81, [p0, p1, p2], [acc(p0), acc(p1), acc(p2)], 2, 4, 128)
    fused, ref = run_case("mixed", steps, "bf16", 2, 4)
    assert ref[1]["tree_status"][4] != 0 and fused[1]["path_len"][4] == -1
    # the invalid tree commits nothing: the next state is its prefix state
    assert np.array_equal(fused[1]["S_commit"][4], fused[0]["S_commit"][4])


@pytest.mark.parametrize("N,Hk,Hv", [(128, 1, 2), (128, 2, 2), (33, 1, 2), (100, 2, 8), (7, 1, 1)])
def test_fused_long_paths(N, Hk, Hv):
    """Chains accept every node, so the commit stages its path in several rounds."""
    rng = np.random.default_rng(90 + N)
    ps = [[W.tree_chain(N), W.tree_random_recursive(rng, N)] for _ in range(3)]
    accs = [[N - 1, W.pick_leaf(rng, p[1])] for p in ps]
    steps = chain_steps(91 + N, ps, accs, Hk, Hv, 128)
    run_case(f"long N={N}", steps, "bf16", Hk, Hv)


def test_fused_in_place():
    rng = np.random.default_rng(95)
    N = 96
    ps = [[W.tree_random_recursive(rng, N) for _ in range(4)] for _ in range(3)]
    accs = [[W.pick_leaf(rng, p) for p in pp] for pp in ps]
    steps = chain_steps(96, ps, accs, 2, 4, 128)
    run_case("in-place", steps, "bf16", 2, 4, in_place=True)


@pytest.mark.parametrize("N,d,io", [(40, 16, "f32"), (70, 64, "bf16")])
def test_fused_other_sizes(N, d, io):
    """Sizes outside the MFMA forms run commit and verify as two launches."""
    rng = np.random.default_rng(97 + N)
    ps = [[W.tree_random_recursive(rng, N), W.tree_chain(N)] for _ in range(2)]
    accs = [[W.pick_leaf(rng, p[0]), N - 1] for p in ps]
    steps = chain_steps(98 + N, ps, accs, 1, 2, d, io)
    run_case(f"other N={N} d={d}", steps, io, 1, 2)


@pytest.mark.parametrize("N", [200, 256, 300, 512, 1000, 1024])
def test_fused_large_trees(N):
    """Trees of 129 .. 1024 nodes: the commit runs inside the larger-tree
    launch.  Chains whose every node is accepted (paths of N nodes, several
    rounds of 256 path nodes from N = 300), random recursive trees with
    a leaf accepted, a sequence with nothing accepted and one whose previous
    tree is invalid; then the same loop in place."""
    rng = np.random.default_rng(110 + N)
    trees = lambda: [W.tree_chain(N), W.tree_random_recursive(rng, N), W.tree_chain(N),
                     W.tree_random_recursive(rng, N)]
    ps = [trees() for _ in range(3)]
    ps[1][3] = ps[1][3].copy(); ps[1][3][N // 2] = N - 1     # forward parent: invalid tree
    accs = [[N - 1, W.pick_leaf(rng, p[1]), -1, W.pick_leaf(rng, p[3])] for p in ps]
    steps = chain_steps(111 + N, ps, accs, 2, 4, 128)
    fused, ref = run_case(f"large N={N}", steps, "bf16", 2, 4)
    assert ref[1]["tree_status"][3] != 0 and fused[1]["path_len"][3] == -1
    assert fused[0]["path_len"][0] == N
    run_case(f"large in-place N={N}", steps, "bf16", 2, 4, in_place=True)


@pytest.mark.parametrize("B,M", [(64, 8), (32, 4)])
def test_fused_full_batch_shape(B, M):
    """The benchmark's launch configurations: 64 sequences of 8-ary, 16-deep
    trees (128 nodes), and 32 sequences of 4-ary ones (64 nodes, each item's
    value columns split over two workgroups), 16 key / 32 value heads,
    d = 128, so that the persistent fused launch takes several items per
    workgroup and every item hand-off (the next item's S rows, k / q rows and
    previous-tree path read ahead) runs.  Three decode steps, every
    (sequence, value head) unit compared."""
    rng = np.random.default_rng(97 + M)
    depth = 16
    ps = [[W.tree_mary(rng, M, depth) for _ in range(B)] for _ in range(3)]
    accs = [[W.pick_leaf(rng, p) for p in pp] for pp in ps]
    steps = chain_steps(98, ps, accs, 16, 32, 128)
    run_case("full batch", steps, "bf16", 16, 32)
