"""Pins that tie the fp64 oracle to facts outside itself.

Each pin is a function of the loaded oracle library and raises AssertionError
when the oracle disagrees with:
  * a gradient step of the online regression loss computed by autograd
    (the delta rule is that step, applied to the decayed state);
  * closed forms (beta = 0 is pure decay; beta = 1 with q = k of unit norm
    writes v exactly, for any gate);
  * a worked example derived by hand (tests/golden/hand_d2_tree3.json);
  * the product form of the affine recurrence on a chain;
  * a boolean transitive closure of the parent relation (masks, depth, paths);
  * a dense numpy linear solve of the unrolled tree system (tests/wy_dense.py);
  * tree invariants: siblings, non-ancestors, topological relabelling, and the
    conventions for invalid trees and accepted indices;
  * for the acceptance walk, a per-node restatement of greedy acceptance
    checked node by node (tests/oracle_pins.py, accept_brute_force);
  * for the tree construction, a worked example derived by hand
    (tests/golden/hand_build_k2_n5.json), the best path scores of an infinite
    tree counted by convolution (width 1 is best-first expansion), and each
    step of the output checked against the candidates open at that step.
The same battery runs against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake trips a pin.
"""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers

def unit_inputs(rng, parent, dk, dv, beta=None, g=None):
    N = len(parent)
    K = rng.standard_normal((N, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((N, dk))
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    V = rng.standard_normal((N, dv))
    be = 1 / (1 + np.exp(-rng.standard_normal(N))) if beta is None else np.broadcast_to(beta, (N,)).astype(float)
    ga = 1 / (1 + np.exp(rng.standard_normal(N))) if g is None else np.broadcast_to(g, (N,)).astype(float)
    S0 = rng.standard_normal((dv, dk)) / np.sqrt(dk)
    return dict(S0=S0, K=K, Q=Q, V=V, beta=np.array(be), g=np.array(ga),
                parent=np.asarray(parent, np.int32))


def run1(lib, u, accepted=-1, memo=False):
    """Oracle on one unit (B = H_k = H_v = 1)."""
    N = len(u["parent"])
    return oracle.verify(u["S0"][None, None], u["Q"][None, :, None], u["K"][None, :, None],
                         u["V"][None, :, None], u["beta"][None, :, None],
                         u["g"][None, :, None], u["parent"][None],
                         np.array([accepted], np.int32), memo=memo, lib=lib)


def closure(parent):
    """Strict-ancestor relation as a boolean matrix, by repeated squaring of
    the parent adjacency (reach[i][j] = j is a strict ancestor of i)."""
    N = len(parent)
    A = np.zeros((N, N), dtype=np.int64)
    for i, p in enumerate(parent):
        if p >= 0:
            A[i, p] = 1
    reach = A.copy()
    while True:
        nxt = ((reach + reach @ reach) > 0).astype(np.int64)
        if np.array_equal(nxt, reach):
            return reach.astype(bool)
        reach = nxt


def mask_bits(mask_rows, N):
    return np.array([[(mask_rows[i, j // 32] >> (j % 32)) & 1 for j in range(N)]
                     for i in range(N)], dtype=bool)


def some_trees(rng):
    return {
        "binary7": W.tree_binary7(),
        "chain9": W.tree_chain(9),
        "star8": W.tree_star(8),
        "mary4x4": W.tree_mary(rng, 4, 4),
        "rrt40": W.tree_random_recursive(rng, 40),
        "forest": np.array([-1, -1, 0, 1, 2, -1, 5, 3, 0, -1], np.int32),
    }


# ------------------------------------------------------------------ pins

def pin_autograd_step(lib):
    """One node: S_1 = S~ - beta * grad_S~ 0.5 |S~ k - v|^2 at S~ = g S0."""
    import torch
    rng = np.random.default_rng(11)
    dk, dv = 5, 3          # non-square: a transposed operand cannot hide
    for trial in range(4):
        u = unit_inputs(rng, [-1], dk, dv)
        r = run1(lib, u, accepted=0)
        St = torch.tensor(u["g"][0] * u["S0"], dtype=torch.float64, requires_grad=True)
        k = torch.tensor(u["K"][0]); v = torch.tensor(u["V"][0])
        loss = 0.5 * ((St @ k - v) ** 2).sum()
        (grad,) = torch.autograd.grad(loss, St)
        S1 = (St - u["beta"][0] * grad).detach().numpy()
        assert np.allclose(r["S_commit"][0, 0], S1, rtol=1e-13, atol=1e-14), "state"
        assert np.allclose(r["o"][0, 0, 0], S1 @ u["Q"][0], rtol=1e-13, atol=1e-14), "output"
        # the write vector: S_1 = g S0 + u k^T
        assert np.allclose(np.outer(r["u"][0, 0, 0], u["K"][0]),
                           S1 - u["g"][0] * u["S0"], rtol=1e-12, atol=1e-14), "u"


def pin_hand_example(lib):
    with open(os.path.join(GOLDEN, "hand_d2_tree3.json")) as f:
        ex = json.load(f)
    u = dict(S0=np.array(ex["S0"], float), K=np.array(ex["k"], float),
             Q=np.array(ex["q"], float), V=np.array(ex["v"], float),
             beta=np.array(ex["beta"], float), g=np.array(ex["g"], float),
             parent=np.array(ex["parent"], np.int32))
    for a in range(3):
        r = run1(lib, u, accepted=a)
        assert np.allclose(r["o"][0, :, 0], ex["o"], rtol=0, atol=1e-14), "o"
        assert np.allclose(r["u"][0, 0], ex["u"], rtol=0, atol=1e-14), "u"
        assert np.allclose(r["S_commit"][0, 0], ex["S"][a], rtol=0, atol=1e-14), "S"


def pin_beta_zero_pure_decay(lib):
    rng = np.random.default_rng(12)
    for name, par in some_trees(rng).items():
        u = unit_inputs(rng, par, 6, 4, beta=0.0)
        clo = closure(par)
        for a in (-1, len(par) - 1):
            r = run1(lib, u, accepted=a)
            for i in range(len(par)):
                gp = u["g"][i] * np.prod(u["g"][clo[i]])
                assert np.allclose(r["o"][0, i, 0], gp * (u["S0"] @ u["Q"][i]),
                                   rtol=1e-13, atol=1e-15), (name, i)
                assert np.isclose(np.exp(r["log_gamma"][0, 0, i]), gp, rtol=1e-13), (name, i)
            if a >= 0:
                ga = u["g"][a] * np.prod(u["g"][clo[a]])
                assert np.allclose(r["S_commit"][0, 0], ga * u["S0"], rtol=1e-13, atol=1e-15)


def pin_projector_writes_v(lib):
    """beta = 1, q_i = k_i, |k_i| = 1: S_i k_i = v_i whatever the gate or S."""
    rng = np.random.default_rng(13)
    for name, par in some_trees(rng).items():
        u = unit_inputs(rng, par, 8, 5, beta=1.0)
        u["Q"] = u["K"].copy()
        r = run1(lib, u)
        assert np.allclose(r["o"][0, :, 0], u["V"], rtol=1e-12, atol=1e-13), name


def pin_chain_product_form(lib):
    """Chain: S_t = S_{t-1} A_t + beta_t v_t k_t^T with A_t = g_t (I - beta_t k_t k_t^T),
    so S_t = S0 A_1..A_t + sum_s beta_s v_s k_s^T A_{s+1}..A_t (numpy matmuls)."""
    rng = np.random.default_rng(14)
    N, dk, dv = 7, 4, 3
    par = W.tree_chain(N)
    u = unit_inputs(rng, par, dk, dv)
    r = run1(lib, u, accepted=N - 1)
    A = [u["g"][t] * (np.eye(dk) - u["beta"][t] * np.outer(u["K"][t], u["K"][t]))
         for t in range(N)]
    for t in range(N):
        S = u["S0"] @ np.linalg.multi_dot([np.eye(dk)] + A[:t + 1])
        for s in range(t + 1):
            tail = np.linalg.multi_dot([np.eye(dk), np.eye(dk)] + A[s + 1:t + 1])
            S = S + u["beta"][s] * np.outer(u["V"][s], u["K"][s]) @ tail
        assert np.allclose(r["o"][0, t, 0], S @ u["Q"][t], rtol=1e-12, atol=1e-14), t
        if t == N - 1:
            assert np.allclose(r["S_commit"][0, 0], S, rtol=1e-12, atol=1e-14)


def pin_chain_is_linear_scan(lib):
    """A chain tree reproduces the plain sequential scan over its tokens,
    written here in the error-correcting form S <- gS + beta (v - g S k) k^T."""
    rng = np.random.default_rng(15)
    N, d = 40, 16
    u = unit_inputs(rng, W.tree_chain(N), d, d)
    r = run1(lib, u, accepted=N - 1)
    S = u["S0"].copy()
    for t in range(N):
        S = u["g"][t] * S + u["beta"][t] * np.outer(u["V"][t] - u["g"][t] * S @ u["K"][t], u["K"][t])
        assert np.allclose(r["o"][0, t, 0], S @ u["Q"][t], rtol=1e-11, atol=1e-13), t
    assert np.allclose(r["S_commit"][0, 0], S, rtol=1e-11, atol=1e-13)


def pin_chain256_is_linear_scan(lib):
    """The 256-node chain workload at its full size (8 sequences x 16 heads,
    d = 128, bf16 q/k/v widened exactly, beta pushed toward 1): every node's
    output and the committed state of the last node equal a plain sequential
    scan over the chain, all 128 (sequence, value head) units stepped together
    with numpy matrix products."""
    s = W.spec("chain256_b8")
    parent, accepted = W.make_trees(s)
    lay = W.make_layer(s, 0)
    f = lambda a: W.io_to_f64(a, s.io)
    q, k, v = f(lay["q"]), f(lay["k"]), f(lay["v"])
    beta, g = lay["beta"].astype(np.float64), lay["g"].astype(np.float64)
    S0 = lay["S0"].astype(np.float64)
    assert (accepted == s.n_nodes - 1).all()
    r = oracle.verify(S0, q, k, v, beta, g, parent, accepted, memo=True, lib=lib)
    hk = np.arange(s.h_v) // s.group                  # value head -> key head
    S = S0.copy()                                     # [B][Hv][dv][dk]
    for t in range(s.n_nodes):
        kt, qt = k[:, t][:, hk, :, None], q[:, t][:, hk, :, None]
        gt, bt = g[:, t, :, None, None], beta[:, t, :, None, None]
        S = gt * S + bt * (v[:, t, :, :, None] - gt * (S @ kt)) @ kt.transpose(0, 1, 3, 2)
        o = (S @ qt)[..., 0]
        assert np.allclose(r["o"][:, t], o, rtol=1e-10, atol=1e-12), t
    assert np.allclose(r["S_commit"], S, rtol=1e-10, atol=1e-12)


def pin_masks_paths(lib):
    rng = np.random.default_rng(16)
    trees = some_trees(rng)
    trees["rrt100"] = W.tree_random_recursive(rng, 100)
    trees["chain70"] = W.tree_chain(70)
    for name, par in trees.items():
        N = len(par)
        mask, depth, status = oracle.tree(par, lib=lib)
        clo = closure(par)
        assert status[0] == 0, name
        assert np.array_equal(mask_bits(mask[0], N), clo), name
        assert np.array_equal(depth[0], clo.sum(1)), name
        bits = np.unpackbits(mask[0].view(np.uint8), axis=1, bitorder="little")
        assert not bits[:, N:].any(), name          # padding bits stay zero
        for a in (0, N - 1, N // 2):
            u = unit_inputs(rng, par, 2, 2)
            r = run1(lib, u, accepted=a)
            want = sorted(np.nonzero(clo[a])[0].tolist() + [a])
            assert r["path_len"][0] == len(want), name
            assert r["path"][0, :len(want)].tolist() == want, name
            assert (r["path"][0, len(want):] == -1).all(), name


def pin_dense_solve(lib):
    rng = np.random.default_rng(17)
    import wy_dense
    for name, par in some_trees(rng).items():
        u = unit_inputs(rng, par, 12, 10)
        for a in (-1, len(par) - 1):
            r = run1(lib, u, accepted=a)
            O, U, G, Sa = wy_dense.solve_unit(u["S0"], u["K"], u["Q"], u["V"], u["beta"],
                                              u["g"], par, a)
            assert np.allclose(r["o"][0, :, 0], O, rtol=1e-11, atol=1e-13), name
            assert np.allclose(r["u"][0, 0], U, rtol=1e-11, atol=1e-13), name
            assert np.allclose(r["log_gamma"][0, 0], G, rtol=1e-13, atol=1e-14), name
            assert np.allclose(r["S_commit"][0, 0], Sa, rtol=1e-11, atol=1e-13), name


def pin_grouped_heads(lib):
    """Two value heads per key head: value head h must read key head h // 2."""
    import wy_dense
    rng = np.random.default_rng(18)
    B, N, Hk, Hv, d = 2, 9, 2, 4, 6
    par = np.stack([W.tree_mary(rng, 3, 3), W.tree_random_recursive(rng, 9)])
    acc = np.array([8, 4], np.int32)
    q = rng.standard_normal((B, N, Hk, d)); k = rng.standard_normal((B, N, Hk, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, Hv, d))
    beta = rng.uniform(0.1, 0.9, (B, N, Hv)); g = rng.uniform(0.3, 0.99, (B, N, Hv))
    S0 = rng.standard_normal((B, Hv, d, d)) / np.sqrt(d)
    r = oracle.verify(S0, q, k, v, beta, g, par, acc, lib=lib)
    for b in range(B):
        for h in range(Hv):
            O, U, G, Sa = wy_dense.solve_unit(S0[b, h], k[b, :, h // 2], q[b, :, h // 2],
                                              v[b, :, h], beta[b, :, h], g[b, :, h],
                                              par[b], acc[b])
            assert np.allclose(r["o"][b, :, h], O, rtol=1e-11, atol=1e-13), (b, h)
            assert np.allclose(r["S_commit"][b, h], Sa, rtol=1e-11, atol=1e-13), (b, h)


def pin_siblings_share_parent(lib):
    """Siblings with identical inputs get identical outputs and states; the
    pre-update state of siblings is the parent's state (u_i differ only via v)."""
    rng = np.random.default_rng(19)
    par = np.array([-1, 0, 1, 1, 1, 2], np.int32)   # nodes 2, 3, 4 are siblings
    u = unit_inputs(rng, par, 7, 7)
    for key in ("K", "Q", "V"):
        u[key][3] = u[key][2]
    u["beta"][3] = u["beta"][2]; u["g"][3] = u["g"][2]
    r2 = run1(lib, u, accepted=2)
    r3 = run1(lib, u, accepted=3)
    assert np.array_equal(r2["o"][0, 2], r2["o"][0, 3])
    assert np.array_equal(r2["u"][0, 0, 2], r2["u"][0, 0, 3])
    assert np.array_equal(r2["S_commit"], r3["S_commit"])
    # sibling 4 shares the parent state: its write uses S_1 k_4
    S1 = run1(lib, u, accepted=1)["S_commit"][0, 0]
    want = u["beta"][4] * (u["V"][4] - u["g"][4] * S1 @ u["K"][4])
    assert np.allclose(r2["u"][0, 0, 4], want, rtol=1e-13, atol=1e-15)


def pin_non_ancestors_do_not_matter(lib):
    rng = np.random.default_rng(20)
    par = W.tree_random_recursive(rng, 30)
    clo = closure(par)
    base = unit_inputs(rng, par, 6, 5)
    r0 = run1(lib, base)
    for i in (5, 17, 29):
        u = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in base.items()}
        others = [j for j in range(30) if j != i and not clo[i, j]]
        for j in others:
            u["K"][j] = rng.standard_normal(6); u["V"][j] = rng.standard_normal(5)
            u["Q"][j] = rng.standard_normal(6)
            u["beta"][j] = rng.uniform(); u["g"][j] = rng.uniform(0.1, 1)
        r = run1(lib, u)
        assert np.array_equal(r["o"][0, i], r0["o"][0, i]), i
        assert np.array_equal(r["u"][0, 0, i], r0["u"][0, 0, i]), i


def pin_topological_relabel(lib):
    rng = np.random.default_rng(21)
    par = W.tree_random_recursive(rng, 25)
    N = len(par)
    u = unit_inputs(rng, par, 5, 4)
    r = run1(lib, u, accepted=N - 1)
    # a different topological order: sort by (depth, random key)
    depth = closure(par).sum(1)
    order = np.lexsort((rng.random(N), depth))          # new position -> old node
    inv = np.empty(N, int); inv[order] = np.arange(N)    # old node -> new position
    par2 = np.array([-1 if par[o] < 0 else inv[par[o]] for o in order], np.int32)
    assert all(par2[i] < i for i in range(N))
    u2 = {key: (u[key][order] if key in ("K", "Q", "V", "beta", "g") else u[key])
          for key in u}
    u2["parent"] = par2
    r2 = run1(lib, u2, accepted=int(inv[N - 1]))
    assert np.allclose(r2["o"][0, :, 0], r["o"][0, order, 0], rtol=1e-12, atol=1e-14)
    assert np.allclose(r2["S_commit"], r["S_commit"], rtol=1e-12, atol=1e-14)
    assert r2["path_len"][0] == r["path_len"][0]
    assert np.array_equal(np.sort(order[r2["path"][0, :r2["path_len"][0]]]),
                          r["path"][0, :r["path_len"][0]])


def pin_memo_equals_walk(lib):
    rng = np.random.default_rng(22)
    for name, par in some_trees(rng).items():
        u = unit_inputs(rng, par, 9, 7)
        a = int(W.leaves(par)[-1])
        r0 = run1(lib, u, accepted=a, memo=False)
        r1 = run1(lib, u, accepted=a, memo=True)
        for key in r0:
            assert np.array_equal(r0[key], r1[key], equal_nan=True), (name, key)


def pin_conventions(lib):
    rng = np.random.default_rng(23)
    par = W.tree_binary7()
    u = unit_inputs(rng, par, 4, 4)
    r = run1(lib, u, accepted=-1)
    assert r["path_len"][0] == 0 and (r["path"][0] == -1).all()
    assert np.array_equal(r["S_commit"][0, 0], u["S0"])
    for bad in (7, -2, 100):
        r = run1(lib, u, accepted=bad)
        assert r["path_len"][0] == -1 and (r["path"][0] == -1).all()
        assert np.array_equal(r["S_commit"][0, 0], u["S0"])
        assert np.isfinite(r["o"]).all()
    for badpar, first in (([-1, 0, 2, 1], 3), ([0, -1], 1), ([-1, -2, 0], 2), ([-1, 0, 1, 3], 4)):
        p = np.array(badpar, np.int32)
        ub = unit_inputs(rng, p, 3, 3)
        r = run1(lib, ub, accepted=0)
        assert r["status"][0] == first, badpar
        assert r["path_len"][0] == -1
        assert np.isnan(r["o"]).all()
        assert np.array_equal(r["S_commit"][0, 0], ub["S0"])
        _, depth, st = oracle.tree(p, lib=lib)
        assert st[0] == first


def accept_brute_force(parent, draft, target, target_root):
    """Greedy acceptance restated per node: node i is reached iff every node j
    on its root-to-node path carries the prediction of j's predecessor (the
    prefix's for a root) and is the lowest-index sibling carrying it; the
    accepted node is the deepest node reached (at most one per depth)."""
    N = len(parent)
    if any(not (-1 <= parent[i] < i) for i in range(N)):
        return -1, -1, int(target_root)
    pred = lambda j: int(target_root) if j < 0 else int(target[j])
    best, best_len = -1, 0
    for i in range(N):
        path, j = [], i
        while j >= 0:
            path.append(j)
            j = parent[j]
        ok = True
        for j in path:
            want = pred(parent[j])
            first = min(x for x in range(N) if parent[x] == parent[j] and draft[x] == want) \
                if any(parent[x] == parent[j] and draft[x] == want for x in range(N)) else None
            if draft[j] != want or first != j:
                ok = False
                break
        if ok and len(path) > best_len:
            best, best_len = i, len(path)
    return best, best_len, pred(best)


def pin_accept_brute_force(lib):
    """The acceptance walk against the per-node restatement on random trees
    with a three-token vocabulary (so siblings often tie and paths run deep)."""
    rng = np.random.default_rng(31)
    trees = []
    for n in (1, 2, 7, 20, 45):
        for _ in range(6):
            trees.append(W.tree_random_recursive(rng, n))
    trees += [W.tree_chain(30), W.tree_star(12), W.tree_mary(rng, 3, 5)]
    for parent in trees:
        N = len(parent)
        draft = rng.integers(0, 3, size=N).astype(np.int32)
        target = rng.integers(0, 3, size=N).astype(np.int32)
        root = np.array([rng.integers(0, 3)], np.int32)
        acc, alen, nxt = oracle.accept(parent[None], draft[None], target[None], root, lib=lib)
        assert (acc[0], alen[0], nxt[0]) == accept_brute_force(parent, draft, target, root[0]), parent


def pin_accept_conventions(lib):
    """Whole chain accepted; nothing accepted; the lowest-index tie wins; an
    invalid parent row."""
    N = 9
    chain = W.tree_chain(N)
    target = np.arange(100, 100 + N, dtype=np.int32)
    draft = np.concatenate([[7], target[:-1]]).astype(np.int32)
    acc, alen, nxt = oracle.accept(chain[None], draft[None], target[None], np.array([7], np.int32), lib=lib)
    assert (acc[0], alen[0], nxt[0]) == (N - 1, N, target[N - 1])
    acc, alen, nxt = oracle.accept(chain[None], draft[None], target[None], np.array([8], np.int32), lib=lib)
    assert (acc[0], alen[0], nxt[0]) == (-1, 0, 8)
    # two roots with the predicted token, each with a matching child
    par = np.array([-1, -1, 0, 1], np.int32)
    dr = np.array([5, 5, 6, 6], np.int32)
    tg = np.array([6, 6, 1, 2], np.int32)
    acc, alen, nxt = oracle.accept(par[None], dr[None], tg[None], np.array([5], np.int32), lib=lib)
    assert (acc[0], alen[0], nxt[0]) == (2, 2, 1)
    bad = chain.copy()
    bad[4] = 4
    acc, alen, nxt = oracle.accept(bad[None], draft[None], target[None], np.array([7], np.int32), lib=lib)
    assert (acc[0], alen[0], nxt[0]) == (-1, -1, 7)


def pin_build_hand_example(lib):
    """Tree construction against the hand-worked example (widths 2, 1, 8)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_build_k2_n5.json")))
    lp = np.array(g["logp"], np.float32)[None]
    tk = np.array(g["tok"], np.int32)[None]
    for case in g["cases"]:
        par, tok, sc = oracle.build_tree(lp, tk, g["n_nodes"], case["width"], lib=lib)
        assert par[0].tolist() == case["parent"], case["width"]
        assert tok[0].tolist() == case["token"], case["width"]
        assert sc[0].tolist() == case["score"], case["width"]


def top_path_scores(logp_row, n):
    """The n highest path scores of the infinite tree in which every node has
    the same K continuations (log-probabilities logp_row, all negative
    multiples of 1/4): counts of paths by depth and score by convolution, then
    the best n scores, each as often as it occurs."""
    steps = [int(round(-4 * x)) for x in logp_row]           # score = -steps / 4
    counts = {0: 1}                                          # depth 0: the prefix
    best = {}
    for _ in range(n):
        nxt = {}
        for s0, c0 in counts.items():
            for st in steps:
                nxt[s0 + st] = nxt.get(s0 + st, 0) + c0
        counts = nxt
        for s0, c0 in counts.items():
            best[s0] = best.get(s0, 0) + c0
    out = []
    for s0 in sorted(best):
        out += [-s0 / 4] * best[s0]
        if len(out) >= n:
            break
    return out[:n]


def pin_build_best_first_top_scores(lib):
    """Width 1 is best-first expansion: when every node offers the same
    continuations with negative log-probabilities, the tree holds the n best
    paths of the infinite tree, so its scores are the n highest path scores
    (counted independently, by convolution)."""
    rng = np.random.default_rng(41)
    for K, n in ((2, 9), (3, 20), (4, 33), (1, 6)):
        row = -(rng.integers(1, 12, size=K) / 4.0)
        lp = np.broadcast_to(row.astype(np.float32), (1, n + 1, K)).copy()
        tk = np.arange((n + 1) * K, dtype=np.int32).reshape(1, n + 1, K)
        par, tok, sc = oracle.build_tree(lp, tk, n, 1, lib=lib)
        assert sorted(sc[0].tolist(), reverse=True) == top_path_scores(row, n), (K, n)


def pin_build_steps_valid(lib):
    """Each step's nodes, checked against the definition from the output alone:
    the step sizes (min(w, nodes left, candidates)); every node's parent placed
    in an earlier step; its token and score from its parent's row (score in
    fp32); and the step's nodes are the best of the candidates open at that
    step (score, then parent, then rank), in that order.  Scores are
    quantised so that ties across parents and ranks occur."""
    rng = np.random.default_rng(43)
    for B, K, n, w in ((3, 4, 30, 4), (2, 2, 17, 3), (2, 5, 40, 8), (2, 3, 12, 1), (1, 1, 7, 3),
                       (1, 8, 20, 64)):
        lp = (-rng.integers(0, 6, size=(B, n + 1, K)) / 2.0).astype(np.float32)
        tk = rng.permutation(B * (n + 1) * K).astype(np.int32).reshape(B, n + 1, K)
        par, tok, sc = oracle.build_tree(lp, tk, n, w, lib=lib)
        for b in range(B):
            rank = {}
            for i in range(n):
                p = int(par[b, i])
                row = p + 1
                c = [x for x in range(K) if tk[b, row, x] == tok[b, i]]
                assert len(c) == 1, (b, i)
                rank[i] = c[0]
                base = np.float32(0.0) if p < 0 else sc[b, p]
                assert sc[b, i] == np.float32(base + lp[b, row, c[0]]), (b, i)
            placed, open_ = 0, [(-1, x) for x in range(K)]
            score_of = lambda pc: (np.float32(0.0) if pc[0] < 0 else sc[b, pc[0]]) + lp[b, pc[0] + 1, pc[1]]
            while placed < n:
                m = min(w, n - placed, len(open_))
                ranked = sorted(open_, key=lambda pc: (-np.float32(score_of(pc)), pc[0], pc[1]))
                step = [(int(par[b, i]), rank[i]) for i in range(placed, placed + m)]
                assert step == ranked[:m], (b, placed)
                for i in range(placed, placed + m):
                    assert par[b, i] < placed, (b, i)
                open_ = ranked[m:] + [(i, x) for i in range(placed, placed + m) for x in range(K)]
                placed += m


ALL_PINS = [
    pin_autograd_step, pin_hand_example, pin_beta_zero_pure_decay,
    pin_projector_writes_v, pin_chain_product_form, pin_chain_is_linear_scan,
    pin_masks_paths, pin_dense_solve, pin_grouped_heads, pin_siblings_share_parent,
    pin_non_ancestors_do_not_matter, pin_topological_relabel, pin_memo_equals_walk,
    pin_conventions, pin_accept_brute_force, pin_accept_conventions,
    pin_build_hand_example, pin_build_best_first_top_scores, pin_build_steps_valid,
    pin_chain256_is_linear_scan,
]
