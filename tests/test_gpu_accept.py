"""GPU parity of the acceptance walk gdn_tree_accept against the oracle's walk,
bit for bit (accepted node, accepted length, next token), and of the on-device
decode step built from it: verify, accept on the device, commit the accepted
node, all without the host."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import rel_l2

pytestmark = pytest.mark.gpu


def _announce(what):
    print(f"[gpu-accept] {what}", flush=True)


def gpu_accept(parent, draft, target, root, device="cuda"):
    import torch
    import tree_masked_gated_amd as T
    B, N = parent.shape
    d = T.dims(B, N, 1, 1, 16, 16, "f32")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)
    acc = torch.full((B,), -9, dtype=torch.int32, device=device)
    alen = torch.full((B,), -9, dtype=torch.int32, device=device)
    nxt = torch.full((B,), -9, dtype=torch.int32, device=device)
    T.gdn_tree_accept(d, t(parent), t(draft), t(target), t(root), acc, alen, nxt)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), alen.cpu().numpy(), nxt.cpu().numpy()


def tokens(rng, parent, vocab, follow=0.0):
    """Draft / target tokens; with probability `follow` a node's draft token
    is its parent's target token (so paths are accepted deep)."""
    B, N = parent.shape
    target = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
    root = rng.integers(0, vocab, size=B).astype(np.int32)
    draft = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
    for b in range(B):
        for i in range(N):
            if rng.random() < follow:
                p = parent[b, i]
                draft[b, i] = root[b] if p < 0 else target[b, p]
    return draft, target, root


def check(name, parent, draft, target, root):
    import oracle
    _announce(f"{name} B={parent.shape[0]} N={parent.shape[1]}")
    g = gpu_accept(parent, draft, target, root)
    r = oracle.accept(parent, draft, target, root)
    for key, x, y in zip(("accepted", "accept_len", "next_token"), g, r):
        assert np.array_equal(x, y), (key, x, y)
    return g


@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 128, 300, 512, 1024])
def test_accept_random(N):
    rng = np.random.default_rng(200 + N)
    B = 16
    parent = np.stack([W.tree_random_recursive(rng, N) for _ in range(B // 2)] +
                      [W.tree_mary(rng, 4, (N + 3) // 4)[:N] for _ in range(B // 2)])
    for vocab, follow in ((2, 0.0), (5, 0.6), (1000, 0.9)):
        draft, target, root = tokens(rng, parent, vocab, follow)
        g = check(f"random vocab={vocab} follow={follow}", parent, draft, target, root)
    assert (g[1] >= 0).all()


def test_accept_long_chains_and_edges():
    rng = np.random.default_rng(210)
    N = 1024
    chain = np.stack([W.tree_chain(N)] * 4)
    target = rng.integers(0, 50, size=(4, N)).astype(np.int32)
    root = np.array([3, 3, 3, 3], np.int32)
    draft = np.empty_like(target)
    draft[:, 0] = root
    draft[:, 1:] = target[:, :-1]
    draft[1, 700] = (target[1, 699] + 1) % 50           # stops at node 699
    draft[2, 0] = 4                                      # nothing accepted
    bad = chain.copy()
    bad[3, 10] = 10                                      # invalid tree
    g = check("chains", bad, draft, target, root)
    assert g[0].tolist() == [N - 1, 699, -1, -1]
    assert g[1].tolist() == [N, 700, 0, -1]
    # siblings tied on the predicted token: the lowest index wins
    par = np.array([[-1, -1, -1, 0, 1, 2, 2]], np.int32)
    dr = np.array([[9, 5, 5, 1, 1, 1, 1]], np.int32)
    tg = np.array([[0, 1, 1, 0, 0, 7, 8]], np.int32)
    g = check("ties", par, dr, tg, np.array([5], np.int32))
    assert (g[0][0], g[1][0], g[2][0]) == (4, 2, 0)


def test_decode_step_on_device():
    """Verify a tree, accept on the device, commit the device's accepted node:
    the committed state matches the oracle's commit of the oracle's accepted
    node."""
    import torch
    import oracle
    import tree_masked_gated_amd as T
    s = W.spec("mary64_b32")
    parent, _ = W.make_trees(s)
    lay = W.make_layer(s, 0)
    rng = np.random.default_rng(220)
    draft, target, root = tokens(rng, parent, 4, 0.7)
    B, N = parent.shape
    dims = T.dims(B, N, s.h_k, s.h_v, s.d, s.d, s.io)
    dev = "cuda"
    S0 = W.to_device(lay["S0"], device=dev)
    q, k, v = (W.to_device(lay[x], s.io, dev) for x in ("q", "k", "v"))
    beta, g = W.to_device(lay["beta"], device=dev), W.to_device(lay["g"], device=dev)
    par = W.to_device(parent.astype(np.int32), device=dev)
    o = torch.empty((B, N, s.h_v, s.d), dtype=q.dtype, device=dev)
    cache = T.TreeCache(dims, dev)
    T.gdn_tree_verify(dims, S0, q, k, v, beta, g, par, o, cache)
    ti = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    T.gdn_tree_accept(dims, par, ti(draft), ti(target), ti(root), acc, alen, nxt)
    S1 = torch.empty_like(S0)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    plen = torch.empty((B,), dtype=torch.int32, device=dev)
    T.gdn_tree_commit(dims, S0, S1, k, cache, acc, path, plen)
    torch.cuda.synchronize()
    racc, ralen, _ = oracle.accept(parent, draft, target, root)
    assert np.array_equal(acc.cpu().numpy(), racc)
    f = lambda a: W.io_to_f64(a, s.io)
    ref = oracle.verify(lay["S0"].astype(np.float64), f(lay["q"]), f(lay["k"]), f(lay["v"]),
                        lay["beta"].astype(np.float64), lay["g"].astype(np.float64), parent, racc,
                        memo=True)
    assert np.array_equal(plen.cpu().numpy(), ralen)
    got = S1.cpu().numpy().astype(np.float64)
    worst = max(rel_l2(got[b, h], ref["S_commit"][b, h]) for b in range(B) for h in range(s.h_v))
    _announce(f"decode step: accepted lengths {sorted(set(ralen.tolist()))}, max unit rel-L2 {worst:.2e}")
    assert worst <= 1e-2
