"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Floating point: relative L2 error <= 1e-2 per (sequence, value head) unit on
the outputs o, the committed state, the cached writes u and the path
log-gates.  Integer results (ancestor rows, depths, tree status, committed
path and its length) must match bit for bit.  Verification must leave S0
untouched bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from gpu_harness import check_exact, gpu_run, oracle_run, unit_errors

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
    _, _, err = check_case(parent, accepted, lay, s.io, s.h_k, s.h_v, name=name)
    if s.io == "f32":
        assert max(err.values()) < 1e-4


def test_layer_stack_sampled_layers():
    """The 36-layer, 64-sequence, 128-node workload: two full layers through
    the same launch configuration the benchmark uses, all units compared."""
    s = W.spec("mary128_b64_l36")
    parent, accepted = W.make_trees(s)
    for layer in (0, 35):
        lay = W.make_layer(s, layer)
        check_case(parent, accepted, lay, s.io, s.h_k, s.h_v, name=f"{s.name}[{layer}]")


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


@pytest.mark.parametrize("N", [200, 300])
def test_large_tree_depths(N):
    """The larger-tree path (a separate tree launch and a solve launch, both
    building by pointer doubling whose round count follows the deepest
    path) at depths on either side of powers of two, up to a chain."""
    rng = np.random.default_rng(900 + N)
    depths = [0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 63, 64, 65, 128, N - 1]
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


def test_invalid_trees_large():
    """Tree errors on the path for 129 .. 512 nodes (a separate tree launch)."""
    rng = np.random.default_rng(66)
    N = 200
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
