"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Floating point: relative L2 error <= 1e-2 per (sequence, value head) unit on
the outputs o, the committed state, the cached writes u and the path
log-gates.  Integer results (ancestor rows, depths, tree status, committed
path and its length) must match bit for bit.  Verification must leave S0
untouched bit for bit.
"""
import concurrent.futures

import numpy as np
import pytest

import workloads as W
from gpu_harness import (check_exact, gpu_fused_layer, gpu_run, oracle_commit, oracle_run,
                         record, rel_l2, unit_errors)

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _announce(what):
    print(f"[gpu-parity] {what}", flush=True)


def check_case(parent, accepted, lay, io, Hk, Hv, tol=TOL, in_place=False, name=""):
    _announce(f"{name} B={parent.shape[0]} N={parent.shape[1]} Hk={Hk} Hv={Hv} "
              f"d={lay['S0'].shape[-1]} io={io}")
    gpu = gpu_run(parent, accepted, lay, io, Hk, Hv, in_place=in_place)
    ref = oracle_run(parent, accepted, lay, io)
    check_exact(gpu, ref)
    err = unit_errors(gpu, ref, Hk, Hv)
    _announce(f"  max unit rel-L2 {err}")
    record(name, err)
    for key, e in err.items():
        assert e <= tol, (key, e)
    bad = ref["status"] != 0
    if bad.any():
        assert np.isnan(gpu["o"][bad]).all()
    assert np.isfinite(gpu["o"][~bad]).all()
    return gpu, ref, err


@pytest.mark.parametrize("name", ["tiny7", "mary64_b1", "mary64_b32", "chain256_b8",
                                  "rrt512_b8"])
def test_workload_full(name):
    s = W.spec(name)
    parent, accepted = W.make_trees(s)
    lay = W.make_layer(s, 0)
    gpu, ref, err = check_case(parent, accepted, lay, s.io, s.h_k, s.h_v, name=name)
    if s.io == "f32":
        assert max(err.values()) < 1e-4
    if s.tree == "chain":
        # the error of a chain grows with depth; over all 256 nodes the shallow
        # ones would dilute it, so the deepest 16 nodes are held to the bar alone
        deep = {"o_deepest16": 0.0, "u_deepest16": 0.0}
        for b in range(s.batch):
            for h in range(s.h_v):
                deep["o_deepest16"] = max(deep["o_deepest16"], rel_l2(
                    gpu["o"][b, -16:, h], ref["o"][b, -16:, h]))
                deep["u_deepest16"] = max(deep["u_deepest16"], rel_l2(
                    gpu["u"][b, h, -16:], ref["u"][b, h, -16:]))
        _announce(f"  deepest 16 nodes: {deep}")
        record(name, deep)
        for key, e in deep.items():
            assert e <= TOL, (key, e)


@pytest.mark.parametrize("chunk", range(6))
def test_layer_stack_all_layers(chunk):
    """The 36-layer, 64-sequence, 128-node workload, six layers per case, each
    through the benchmark's launches: the tree verified on the layer's S0, then
    one gdn_tree_commit_verify launch that commits its accepted node and
    verifies the tree again on the committed state.  Every layer's committed
    state is compared for all 64 x 32 units (the oracle's state of the
    accepted node, reached along its path); the outputs of both verifications
    and the cache of the second for four sequences per layer, rotated so the
    36 layers cover every sequence; ancestor rows, depths, status, the path and
    its length bit for bit everywhere."""
    import oracle
    s = W.spec("mary128_b64_l36")
    parent, accepted = W.make_trees(s)
    mask, depth, status = oracle.tree(parent)
    layers = list(range(6 * chunk, 6 * chunk + 6))
    worst = {"o1": 0.0, "o2": 0.0, "u": 0.0, "log_gamma": 0.0, "S_commit": 0.0}
    with concurrent.futures.ThreadPoolExecutor(2) as ex:
        futs = [ex.submit(W.make_layer, s, l) for l in layers]
        for l, fut in zip(layers, futs):
            lay = fut.result()
            _announce(f"{s.name} layer {l}: fused step B={s.batch} N={s.n_nodes}")
            gpu = gpu_fused_layer(parent, accepted, lay, s.io, s.h_k, s.h_v)
            for c in ("A", "B"):
                assert np.array_equal(gpu[c]["status"], status), (l, c, "status")
                assert np.array_equal(gpu[c]["anc_mask"], mask), (l, c, "anc_mask")
                assert np.array_equal(gpu[c]["depth"], depth), (l, c, "depth")
            S1, paths, plen = oracle_commit(parent, accepted, lay, s.io, lay["S0"])
            assert np.array_equal(gpu["path"], paths), (l, "path")
            assert np.array_equal(gpu["path_len"], plen), (l, "path_len")
            for b in range(s.batch):
                for h in range(s.h_v):
                    worst["S_commit"] = max(worst["S_commit"],
                                            rel_l2(gpu["S1"][b, h], S1[b, h]))
            sub = [(4 * l + j) % s.batch for j in range(4)]
            pick = lambda a: {key: val[sub] for key, val in a.items()}
            r1 = oracle.verify(lay["S0"][sub].astype(np.float64),
                               *(W.io_to_f64(lay[key][sub], s.io) for key in ("q", "k", "v")),
                               lay["beta"][sub].astype(np.float64),
                               lay["g"][sub].astype(np.float64), parent[sub],
                               accepted[sub], memo=True)
            assert np.allclose(r1["S_commit"], S1[sub], rtol=1e-12, atol=1e-14)
            r2 = oracle.verify(S1[sub], *(W.io_to_f64(lay[key][sub], s.io)
                                          for key in ("q", "k", "v")),
                               lay["beta"][sub].astype(np.float64),
                               lay["g"][sub].astype(np.float64), parent[sub],
                               accepted[sub], memo=True)
            gb = pick(gpu["B"])
            for j in range(len(sub)):
                b = sub[j]
                for h in range(s.h_v):
                    worst["o1"] = max(worst["o1"], rel_l2(gpu["o1"][b, :, h], r1["o"][j, :, h]))
                    worst["o2"] = max(worst["o2"], rel_l2(gpu["o2"][b, :, h], r2["o"][j, :, h]))
                    worst["u"] = max(worst["u"], rel_l2(gb["u"][j, h], r2["u"][j, h]),
                                     rel_l2(gpu["A"]["u"][b, h], r1["u"][j, h]))
                    worst["log_gamma"] = max(worst["log_gamma"],
                                             rel_l2(gb["log_gamma"][j, h], r2["log_gamma"][j, h]))
            assert np.isfinite(gpu["o2"]).all() and np.isfinite(gpu["S1"]).all()
            _announce(f"  worst so far {worst}")
            del lay, gpu
    record(f"{s.name} (all 36 layers, fused)", worst)
    for key, e in worst.items():
        assert e <= TOL, (key, e)


def custom(seed, parents, Hk, Hv, d, io="bf16", beta_mu=0.0):
    rng = np.random.default_rng(seed)
    N = len(parents[0])
    parent = np.stack([np.asarray(p, np.int32) for p in parents])
    lay = W.draw_layer(rng, len(parents), N, Hk, Hv, d, io, beta_mu)
    return parent, lay


RAGGED = [1, 2, 33, 37, 64, 100, 127, 129, 200, 255, 256, 257, 300, 512, 513, 1000, 1024]


@pytest.mark.parametrize("N", RAGGED)
def test_ragged_sizes(N):
    rng = np.random.default_rng(100 + N)
    parents = [W.tree_random_recursive(rng, N), W.tree_chain(N)]
    parent, lay = custom(N, parents, 2, 4, 128)
    accepted = np.array([W.pick_leaf(rng, p) for p in parents], np.int32)
    check_case(parent, accepted, lay, "bf16", 2, 4, name=f"ragged N={N}")


def tree_of_depth(rng, n, depth):
    """n nodes whose deepest node has exactly `depth` strict ancestors: a chain
    of depth + 1 nodes, then each further node under a uniformly drawn
    earlier node of depth < `depth` (depth 0: every node under the prefix)."""
    parent = np.full(n, -1, np.int32)
    dep = np.zeros(n, np.int64)
    for i in range(1, n):
        if i <= depth:
            parent[i] = i - 1
        else:
            cand = np.flatnonzero(dep[:i] < depth)
            parent[i] = rng.choice(cand) if depth > 0 else -1
        dep[i] = dep[parent[i]] + 1 if parent[i] >= 0 else 0
    assert dep.max() == min(depth, n - 1)
    return parent


@pytest.mark.parametrize("N", [200, 300, 1000])
def test_large_tree_depths(N):
    """The larger-tree path (one launch that checks the tree, builds its
    preorder and path log-gates by pointer doubling, whose round count follows
    the deepest path, then walks its block rows) at depths on either side of
    powers of two, up to a chain."""
    rng = np.random.default_rng(900 + N)
    depths = [0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 63, 64, 65, 128, N - 1]
    if N > 512:                                  # past the last rows of U kept in LDS
        depths = [0, 1, 9, 16, 65, 128, 129, 255, 256, 300, 511, 512, 513, 700, N - 2, N - 1]
    parents = [tree_of_depth(rng, N, dd) for dd in depths]
    parent, lay = custom(901 + N, parents, 1, 2, 128)
    # accept node `depth`, the end of the chain: the longest committed path
    accepted = np.array(depths, np.int32)
    check_case(parent, accepted, lay, "bf16", 1, 2, name=f"depths N={N}")


@pytest.mark.parametrize("d,io", [(16, "f32"), (16, "bf16"), (128, "f32"), (64, "bf16"),
                                  (32, "f32")])
def test_head_sizes(d, io):
    rng = np.random.default_rng(7 + d)
    parents = [W.tree_mary(rng, 4, 6), W.tree_random_recursive(rng, 24)]
    parent, lay = custom(d, parents, 1, 2, d, io)
    accepted = np.array([W.pick_leaf(rng, p) for p in parents], np.int32)
    _, _, err = check_case(parent, accepted, lay, io, 1, 2, name=f"d={d} {io}")
    if io == "f32":
        assert max(err.values()) < 1e-4


def test_edge_cases():
    rng = np.random.default_rng(55)
    N = 40
    parents = [
        W.tree_star(N),                                   # every node a child of 0
        np.full(N, -1, np.int32),                         # all nodes under S0
        W.tree_chain(N),
        np.array([-1 if i % 10 == 0 else i - 1 for i in range(N)], np.int32),  # forest
        W.tree_mary(rng, 4, 10),
        W.tree_random_recursive(rng, N),
    ]
    parent, lay = custom(56, parents, 3, 6, 128)
    accepted = np.array([-1, 0, N - 1, 5, 200, -7], np.int32)   # incl. out-of-range
    gpu, ref, _ = check_case(parent, accepted, lay, "bf16", 3, 6, name="edge")
    assert gpu["path_len"].tolist() == [0, 1, N, 6, -1, -1]


def test_gate_and_beta_extremes():
    rng = np.random.default_rng(57)
    parents = [W.tree_mary(rng, 4, 8), W.tree_chain(32)]
    parent, lay = custom(58, parents, 1, 1, 128)
    lay["beta"][:] = 0.0                     # pure decay
    lay["g"][1] = 1.0                        # no decay on the chain
    accepted = np.array([30, 31], np.int32)
    check_case(parent, accepted, lay, "bf16", 1, 1, name="beta=0, g=1")
    lay["beta"][:] = 1.0
    check_case(parent, accepted, lay, "bf16", 1, 1, name="beta=1")


@pytest.mark.parametrize("N", [200, 300, 1024])
def test_chain_path_extremes(N):
    """Chains in the larger-tree kernel take the chunked recurrence (each
    16-node block row starts from the state at the node before it); a chain
    with one extra branch, in the same launch, takes the tile path.  Gates and
    write strengths at their extremes: pure decay (beta = 0), no decay with
    full writes (g = 1, beta = 1), and gates so small that the factors of
    distant nodes underflow to zero in fp32."""
    rng = np.random.default_rng(60 + N)
    near = W.tree_chain(N)
    near[N - 1] = N - 3                                   # a sibling of node N - 2
    parents = [W.tree_chain(N), near]
    parent, lay = custom(61 + N, parents, 2, 4, 128)
    accepted = np.array([N - 1, N - 2], np.int32)
    check_case(parent, accepted, lay, "bf16", 2, 4, name=f"chain path N={N}")
    lay0 = {k: v.copy() for k, v in lay.items()}
    lay["beta"][:] = 0.0
    check_case(parent, accepted, lay, "bf16", 2, 4, name=f"chain path N={N}, beta=0")
    lay = {k: v.copy() for k, v in lay0.items()}
    lay["beta"][:] = 1.0
    lay["g"][:] = 1.0
    check_case(parent, accepted, lay, "bf16", 2, 4, name=f"chain path N={N}, beta=1, g=1")
    lay = {k: v.copy() for k, v in lay0.items()}
    lay["g"][:] = 1e-3
    check_case(parent, accepted, lay, "bf16", 2, 4, name=f"chain path N={N}, g=1e-3")


def test_invalid_trees():
    rng = np.random.default_rng(59)
    N = 20
    good = W.tree_random_recursive(rng, N)
    bad1 = good.copy(); bad1[7] = 7             # self parent
    bad2 = good.copy(); bad2[3] = 15            # forward parent
    bad3 = good.copy(); bad3[11] = -2           # below -1
    parent, lay = custom(60, [good, bad1, bad2, bad3], 1, 2, 128)
    accepted = np.array([N - 1, 2, 2, 2], np.int32)
    gpu, ref, _ = check_case(parent, accepted, lay, "bf16", 1, 2, name="invalid")
    assert gpu["status"].tolist() == [0, 8, 4, 12]
    assert gpu["path_len"].tolist()[1:] == [-1, -1, -1]
    for b in (1, 2, 3):
        assert np.array_equal(gpu["S_commit"][b], lay["S0"][b].astype(np.float64))


def test_in_place_commit():
    s = W.spec("mary64_b1")
    parent, accepted = W.make_trees(s)
    lay = W.make_layer(s, 0)
    check_case(parent, accepted, lay, s.io, s.h_k, s.h_v, in_place=True, name="in-place")


def test_grouped_heads_g4():
    rng = np.random.default_rng(61)
    parents = [W.tree_mary(rng, 8, 8) for _ in range(3)]
    parent, lay = custom(62, parents, 2, 8, 128)
    accepted = np.array([W.pick_leaf(rng, p) for p in parents], np.int32)
    check_case(parent, accepted, lay, "bf16", 2, 8, name="G=4")


def test_deterministic_and_non_ancestor_independent():
    """Two runs give identical bits; perturbing every non-ancestor of a node
    leaves that node's output bit-identical."""
    rng = np.random.default_rng(63)
    N = 96
    par = W.tree_random_recursive(rng, N)
    parent, lay = custom(64, [par], 1, 2, 128)
    acc = np.array([N - 1], np.int32)
    r1 = gpu_run(parent, acc, lay, "bf16", 1, 2)
    r2 = gpu_run(parent, acc, lay, "bf16", 1, 2)
    for key in ("o", "u", "log_gamma", "S_commit"):
        assert np.array_equal(r1[key], r2[key]), key
    node = N - 1
    anc = set()
    j = par[node]
    while j >= 0:
        anc.add(int(j)); j = par[j]
    others = [j for j in range(N) if j != node and j not in anc]
    lay2 = {key: val.copy() for key, val in lay.items()}
    pert = W.draw_layer(np.random.default_rng(65), 1, N, 1, 2, 128)
    for key in ("q", "k", "v", "beta", "g"):
        lay2[key][:, others] = pert[key][:, others]
    r3 = gpu_run(parent, acc, lay2, "bf16", 1, 2)
    assert np.array_equal(r3["o"][0, node], r1["o"][0, node])
    assert np.array_equal(r3["S_commit"], r1["S_commit"])


@pytest.mark.parametrize("N", [200, 700])
def test_invalid_trees_large(N):
    """Tree errors on the path for 129 .. 1024 nodes (found by the setup of
    the single larger-tree launch, before it builds the preorder)."""
    rng = np.random.default_rng(66)
    good = W.tree_random_recursive(rng, N)
    bad1 = good.copy(); bad1[150] = 150         # self parent
    bad2 = good.copy(); bad2[130] = 199         # forward parent
    bad3 = good.copy(); bad3[3] = -5            # below -1
    parent, lay = custom(67, [good, bad1, bad2, bad3], 1, 2, 128)
    accepted = np.array([N - 1, 2, 2, 2], np.int32)
    gpu, ref, _ = check_case(parent, accepted, lay, "bf16", 1, 2, name="invalid large")
    assert gpu["status"].tolist() == [0, 151, 131, 4]
    assert gpu["path_len"].tolist()[1:] == [-1, -1, -1]
    for b in (1, 2, 3):
        assert np.array_equal(gpu["S_commit"][b], lay["S0"][b].astype(np.float64))


def test_deterministic_large():
    """The larger-tree path gives identical bits on two runs, and a node's
    output does not move when every non-ancestor's inputs change."""
    rng = np.random.default_rng(68)
    N = 300
    par = W.tree_random_recursive(rng, N)
    parent, lay = custom(69, [par], 1, 2, 128)
    acc = np.array([N - 1], np.int32)
    r1 = gpu_run(parent, acc, lay, "bf16", 1, 2)
    r2 = gpu_run(parent, acc, lay, "bf16", 1, 2)
    for key in ("o", "u", "log_gamma", "S_commit"):
        assert np.array_equal(r1[key], r2[key]), key
    node = N - 1
    anc = set()
    j = par[node]
    while j >= 0:
        anc.add(int(j)); j = par[j]
    others = [j for j in range(N) if j != node and j not in anc]
    lay2 = {key: val.copy() for key, val in lay.items()}
    pert = W.draw_layer(np.random.default_rng(70), 1, N, 1, 2, 128)
    for key in ("q", "k", "v", "beta", "g"):
        lay2[key][:, others] = pert[key][:, others]
    r3 = gpu_run(parent, acc, lay2, "bf16", 1, 2)
    assert np.array_equal(r3["o"][0, node], r1["o"][0, node])
    assert np.array_equal(r3["S_commit"], r1["S_commit"])


def random_topological_order(rng, parent):
    """A uniformly drawn sequence of the nodes in which every node comes after
    its parent: at each step one of the nodes whose parent is already placed."""
    N = len(parent)
    kids = [[] for _ in range(N)]
    ready = []
    for i, p in enumerate(parent):
        (ready if p < 0 else kids[p]).append(i)
    order = []
    while ready:
        i = ready.pop(int(rng.integers(0, len(ready))))
        order.append(i)
        ready.extend(kids[i])
    return np.array(order, np.int64)


@pytest.mark.parametrize("N", [64, 300, 512, 1000])
def test_topological_relabel(N):
    """Re-ordering the caller's nodes into another topological order permutes
    o, u, the path log-gates, depths and ancestor rows, and leaves the
    committed state and the committed path's nodes unchanged.  Both orders are
    also compared with the oracle."""
    rng = np.random.default_rng(1000 + N)
    trees = [W.tree_random_recursive(rng, N),
             W.tree_mary(rng, 4, N // 4) if N % 4 == 0 else tree_of_depth(rng, N, 40),
             tree_of_depth(rng, N, min(N - 1, 100))]
    parent, lay = custom(1001 + N, trees, 1, 2, 128)
    accepted = np.array([W.pick_leaf(rng, p) for p in trees], np.int32)
    B = len(trees)
    orders = [random_topological_order(rng, p) for p in trees]     # new -> old
    invs = []
    for o in orders:
        inv = np.empty(N, np.int64); inv[o] = np.arange(N); invs.append(inv)
    parent2 = np.stack([np.array([-1 if trees[b][o] < 0 else invs[b][trees[b][o]]
                                  for o in orders[b]], np.int32) for b in range(B)])
    assert all((parent2[b] < np.arange(N)).all() for b in range(B))
    lay2 = dict(lay)
    for key in ("q", "k", "v", "beta", "g"):
        lay2[key] = np.ascontiguousarray(np.stack([lay[key][b, orders[b]] for b in range(B)]))
    accepted2 = np.array([invs[b][accepted[b]] for b in range(B)], np.int32)
    g1, _, _ = check_case(parent, accepted, lay, "bf16", 1, 2, name=f"relabel N={N} original")
    g2, _, _ = check_case(parent2, accepted2, lay2, "bf16", 1, 2, name=f"relabel N={N} relabelled")
    worst = {"o": 0.0, "u": 0.0, "log_gamma": 0.0, "S_commit": 0.0}
    for b in range(B):
        o = orders[b]
        assert np.array_equal(g2["depth"][b], g1["depth"][b, o]), b
        bits = lambda m: np.unpackbits(m.view(np.uint8), axis=1, bitorder="little")[:, :N]
        assert np.array_equal(bits(g2["anc_mask"][b]), bits(g1["anc_mask"][b])[o][:, o]), b
        n = g1["path_len"][b]
        assert g2["path_len"][b] == n
        assert np.array_equal(o[g2["path"][b, :n]], g1["path"][b, :n]), b
        for h in range(2):
            worst["o"] = max(worst["o"], rel_l2(g2["o"][b, :, h], g1["o"][b, o, h]))
            worst["u"] = max(worst["u"], rel_l2(g2["u"][b, h], g1["u"][b, h, o]))
            worst["log_gamma"] = max(worst["log_gamma"],
                                     rel_l2(g2["log_gamma"][b, h], g1["log_gamma"][b, h, o]))
            worst["S_commit"] = max(worst["S_commit"],
                                    rel_l2(g2["S_commit"][b, h], g1["S_commit"][b, h]))
    _announce(f"  relabelled vs original {worst}")
    record(f"relabel N={N} (relabelled vs original)", worst)
    for key, e in worst.items():
        assert e <= TOL, (key, e)
