"""Seeded generators: determinism, shapes, value ranges, bf16 rounding (CPU)."""
import hashlib

import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0e-39, 65504.0, 0.0], np.float32)])
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def digest(lay):
    h = hashlib.sha256()
    for key in sorted(lay):
        h.update(np.ascontiguousarray(lay[key]).tobytes())
    return h.hexdigest()


def test_determinism_and_shapes():
    for name in ("tiny7", "mary64_b1", "chain256_b8"):
        s = W.spec(name)
        p1, a1 = W.make_trees(s)
        p2, a2 = W.make_trees(s)
        assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
        l1, l2 = W.make_layer(s), W.make_layer(s)
        assert digest(l1) == digest(l2)
        assert l1["q"].shape == (s.batch, s.n_nodes, s.h_k, s.d)
        assert l1["v"].shape == (s.batch, s.n_nodes, s.h_v, s.d)
        assert l1["S0"].shape == (s.batch, s.h_v, s.d, s.d)
        assert ((l1["g"] > 0) & (l1["g"] < 1)).all()
        assert ((l1["beta"] > 0) & (l1["beta"] < 1)).all()
        qn = np.linalg.norm(W.io_to_f64(l1["q"], s.io), axis=-1)
        assert np.allclose(qn, 1, atol=1e-2)


def test_tree_shapes():
    s = W.spec("mary128_b64_l36")
    par, acc = W.make_trees(s)
    assert par.shape == (64, 128)
    for b in range(64):
        p = par[b]
        assert (p[:8] == -1).all()
        for j in range(2, 17):
            blk = p[(j - 1) * 8: j * 8]
            assert ((blk >= (j - 2) * 8) & (blk < (j - 1) * 8)).all()
        assert acc[b] in W.leaves(p)
    s = W.spec("rrt512_b8")
    par, acc = W.make_trees(s)
    assert all((par[b][1:] < np.arange(1, 512)).all() and par[b][0] == -1 for b in range(8))
    s = W.spec("chain256_b8")
    par, acc = W.make_trees(s)
    assert (acc == 255).all() and (par[:, 1:] == np.arange(255)).all()
    par, acc = W.make_trees(W.spec("tiny7"))
    assert par[0].tolist() == [-1, 0, 0, 1, 1, 2, 2] and acc[0] == 5


@pytest.mark.parametrize("name", ["tiny7", "mary64_b32", "mary128_b64_l36", "chain256_b8", "rrt512_b8"])
def test_tokens_accept_the_chosen_leaf(name):
    """The benchmark's synthetic tokens make the oracle's acceptance walk stop
    at the workload's chosen node, with the path length of that node."""
    import oracle
    s = W.spec(name)
    parent, accepted = W.make_trees(s)
    draft, target, root = W.make_tokens(s, parent, accepted)
    acc, alen, _ = oracle.accept(parent, draft, target, root)
    assert np.array_equal(acc, accepted)
    _, depth, _ = oracle.tree(parent)
    assert np.array_equal(alen, depth[np.arange(len(accepted)), accepted] + 1)


def test_ragged_workload_packing():
    """The ragged workload's tree sizes match the trees make_trees draws (entries
    past a tree's size are -1), the offsets are their prefix sums, and packing
    keeps each sequence's rows in order."""
    import workloads as W
    s = W.spec("maryragged_b64_l36")
    parent, accepted = W.make_trees(s)
    sizes = W.tree_sizes(s)
    assert set(sizes.tolist()) <= {16, 32, 64, 128} and len(set(sizes.tolist())) > 1
    for b, n in enumerate(sizes):
        assert (parent[b, :n] < np.arange(n)).all() and (parent[b, n:] == -1).all()
        assert 0 <= accepted[b] < n
    off = W.ragged_offsets(sizes)
    assert off[0] == 0 and off[-1] == sizes.sum() and (np.diff(off) == sizes).all()
    x = np.arange(s.batch * s.n_nodes * 3).reshape(s.batch, s.n_nodes, 3)
    p = W.pack_rows(x, sizes)
    for b, n in enumerate(sizes):
        assert np.array_equal(p[off[b]:off[b + 1]], x[b, :n])
