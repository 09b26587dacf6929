"""GPU parity of draft-tree construction (gdn_tree_build): the tree, the tokens
and the scores must equal the oracle's bit for bit.  The selections are
decided in fp32 on both sides (the same one addition per score), so this is
an exact comparison.  Tables are either quantised (many equal scores, so the
parent / rank tie rules decide) or drawn from the synthetic drafter.  A built
tree then runs through verification and commit like any other."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import rel_l2

pytestmark = pytest.mark.gpu


def _announce(what):
    print(f"[gpu-build] {what}", flush=True)


def tables(seed, B, N, K, quantised):
    rng = np.random.default_rng(seed)
    if quantised:
        lp = (-rng.integers(0, 6, size=(B, N + 1, K)) / 2.0).astype(np.float32)
        tk = rng.integers(0, 1 << 20, size=(B, N + 1, K)).astype(np.int32)
        return lp, tk
    return W.draft_scores(rng, B, N, K)


def gpu_build(lp, tk, N, w):
    import torch
    import tree_masked_gated_amd as T
    B, _, K = lp.shape
    bd = T.build_dims(B, N, K, w)
    outs = [torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, N), -7.0, dtype=torch.float32, device="cuda")]
    T.gdn_tree_build(bd, W.to_device(lp), W.to_device(tk), *outs)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in outs]


@pytest.mark.parametrize("B,N,K,w", [
    (4, 128, 8, 8),        # the 8-wide, 16-step shape of the 128-node drafts
    (8, 512, 8, 8),        # 512-node drafts, 64 steps
    (2, 1024, 16, 64),     # the largest tree, wide steps
    (3, 1, 1, 1),
    (2, 33, 3, 5),
    (2, 100, 2, 1),        # best-first, one node per step
    (2, 20, 8, 64),        # one step covers more than the tree
    (1, 1024, 1, 1),       # one continuation per node: a chain, 1024 steps
    (2, 300, 4, 300),
    (2, 200, 64, 4),       # the widest rows
    (5, 77, 5, 9),
])
@pytest.mark.parametrize("quantised", [True, False])
def test_build_matches_oracle(B, N, K, w, quantised):
    import oracle
    lp, tk = tables(400 + N + K + w, B, N, K, quantised)
    _announce(f"B={B} N={N} K={K} w={w} quantised={quantised}")
    par, tok, sc = gpu_build(lp, tk, N, w)
    rp, rt, rs = oracle.build_tree(lp, tk, N, w)
    assert np.array_equal(par, rp), "parent"
    assert np.array_equal(tok, rt), "token"
    assert np.array_equal(sc.view(np.uint32), rs.view(np.uint32)), "score"


def test_built_tree_verifies():
    """A tree built on the device goes straight into verification and commit
    (parents and draft tokens never leave the GPU), and matches the oracle's
    verification of the oracle-built tree."""
    import torch
    import oracle
    import tree_masked_gated_amd as T
    rng = np.random.default_rng(450)
    B, N, K, w, H, d = 4, 128, 8, 8, 2, 128
    lp, tk = W.draft_scores(rng, B, N, K)
    _announce("build -> verify -> commit")
    bd = T.build_dims(B, N, K, w)
    par = torch.empty((B, N), dtype=torch.int32, device="cuda")
    tok = torch.empty_like(par)
    sc = torch.empty((B, N), dtype=torch.float32, device="cuda")
    T.gdn_tree_build(bd, W.to_device(lp), W.to_device(tk), par, tok, sc)
    lay = W.draw_layer(rng, B, N, 1, H, d, "bf16")
    dims = T.dims(B, N, 1, H, d, d, "bf16")
    dev = lambda a, x="": W.to_device(a, x)
    S0 = dev(lay["S0"])
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    cache = T.TreeCache(dims)
    T.gdn_tree_verify(dims, S0, dev(lay["q"], "bf16"), dev(lay["k"], "bf16"), dev(lay["v"], "bf16"),
                      dev(lay["beta"]), dev(lay["g"]), par, o, cache)
    rp, rt, _ = oracle.build_tree(lp, tk, N, w)
    acc = np.array([W.pick_leaf(rng, rp[b]) for b in range(B)], np.int32)
    S_out = torch.empty_like(S0)
    path = torch.empty((B, N), dtype=torch.int32, device="cuda")
    plen = torch.empty((B,), dtype=torch.int32, device="cuda")
    T.gdn_tree_commit(dims, S0, S_out, dev(lay["k"], "bf16"), cache, dev(acc), path, plen)
    torch.cuda.synchronize()
    assert np.array_equal(par.cpu().numpy(), rp) and np.array_equal(tok.cpu().numpy(), rt)
    f = lambda a: W.io_to_f64(a, "bf16")
    ref = oracle.verify(lay["S0"].astype(np.float64), f(lay["q"]), f(lay["k"]), f(lay["v"]),
                        lay["beta"].astype(np.float64), lay["g"].astype(np.float64), rp, acc,
                        memo=True)
    og = W.from_device_f64(o)
    Sg = S_out.cpu().numpy().astype(np.float64)
    assert np.array_equal(path.cpu().numpy(), ref["path"])
    for b in range(B):
        for h in range(H):
            assert rel_l2(og[b, :, h], ref["o"][b, :, h]) <= 1e-2, (b, h)
            assert rel_l2(Sg[b, h], ref["S_commit"][b, h]) <= 1e-2, (b, h)
