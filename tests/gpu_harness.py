"""Run the HIP library and the oracle on the same seeded inputs and compare.

Shared by the GPU parity tests.  Inputs come from workloads.py only; expected
values come from the oracle only."""
import numpy as np

import workloads as W

# Worst errors per case, written to the file named by GDN_PARITY_JSON (if set)
# when the session ends (tests/conftest.py), so that every run leaves a record
# of the measured errors next to its log.
ERRORS = {}


def record(name, err):
    """Keep the worst value of each error figure seen for case `name`."""
    cur = ERRORS.setdefault(name, {})
    for key, val in err.items():
        cur[key] = max(cur.get(key, 0.0), float(val))


def rel_l2(x, ref):
    """Relative L2 error; infinite when either side holds a NaN or an infinity,
    so that a max over units (which keeps its first argument when the second
    is NaN) and a tolerance check both see it."""
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    e = float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))
    return e if np.isfinite(e) else float("inf")


def gpu_run(parent, accepted, lay, io, Hk, Hv, in_place=False, device="cuda"):
    """One verify + commit through the Python binding; returns numpy results."""
    import torch
    import tree_masked_gated_amd as T
    B, N = parent.shape
    d = lay["S0"].shape[-1]
    dims = T.dims(B, N, Hk, Hv, d, d, io)
    S0 = W.to_device(lay["S0"], device=device)
    S0_before = S0.clone()
    q = W.to_device(lay["q"], io, device)
    k = W.to_device(lay["k"], io, device)
    v = W.to_device(lay["v"], io, device)
    beta = W.to_device(lay["beta"], device=device)
    g = W.to_device(lay["g"], device=device)
    par = W.to_device(parent.astype(np.int32), device=device)
    acc = W.to_device(np.asarray(accepted, np.int32), device=device)
    o = torch.empty((B, N, Hv, d), dtype=q.dtype, device=device)
    cache = T.TreeCache(dims, device)
    T.gdn_tree_verify(dims, S0, q, k, v, beta, g, par, o, cache)
    torch.cuda.synchronize()
    s0_unchanged = bool(torch.equal(S0.view(torch.int32), S0_before.view(torch.int32)))
    S_out = S0 if in_place else torch.empty_like(S0)
    path = torch.empty((B, N), dtype=torch.int32, device=device)
    plen = torch.empty((B,), dtype=torch.int32, device=device)
    T.gdn_tree_commit(dims, S0, S_out, k, cache, acc, path, plen)
    torch.cuda.synchronize()
    return {
        "o": W.from_device_f64(o), "u": cache.u.cpu().numpy(),
        "log_gamma": cache.log_gamma.cpu().numpy(),
        "anc_mask": cache.anc_mask.cpu().numpy().view(np.uint32),
        "depth": cache.depth.cpu().numpy(), "status": cache.tree_status.cpu().numpy(),
        "S_commit": S_out.cpu().numpy().astype(np.float64),
        "path": path.cpu().numpy(), "path_len": plen.cpu().numpy(),
        "s0_unchanged": s0_unchanged,
    }


def oracle_run(parent, accepted, lay, io, memo=True):
    import oracle
    f = lambda a: W.io_to_f64(a, io)
    r = oracle.verify(lay["S0"].astype(np.float64), f(lay["q"]), f(lay["k"]), f(lay["v"]),
                      lay["beta"].astype(np.float64), lay["g"].astype(np.float64),
                      parent, np.asarray(accepted, np.int32), memo=memo)
    mask, depth, status = oracle.tree(parent)
    r.update(anc_mask=mask, depth=depth, tree_status=status)
    return r


def unit_errors(gpu, ref, Hk, Hv):
    """Max over (b, h) units of the relative L2 error of o, u, S_commit, Gamma."""
    B = gpu["o"].shape[0]
    worst = {"o": 0.0, "u": 0.0, "S_commit": 0.0, "log_gamma": 0.0}
    for b in range(B):
        if ref["status"][b]:
            continue
        for h in range(Hv):
            worst["o"] = max(worst["o"], rel_l2(gpu["o"][b, :, h], ref["o"][b, :, h]))
            worst["u"] = max(worst["u"], rel_l2(gpu["u"][b, h], ref["u"][b, h]))
            worst["S_commit"] = max(worst["S_commit"],
                                      rel_l2(gpu["S_commit"][b, h], ref["S_commit"][b, h]))
            worst["log_gamma"] = max(worst["log_gamma"],
                                       rel_l2(gpu["log_gamma"][b, h], ref["log_gamma"][b, h]))
    return worst


def check_exact(gpu, ref):
    """Integer outputs must match bit for bit."""
    assert np.array_equal(gpu["status"], ref["tree_status"]), "tree_status"
    assert np.array_equal(gpu["anc_mask"], ref["anc_mask"]), "anc_mask"
    assert np.array_equal(gpu["depth"], ref["depth"]), "depth"
    assert np.array_equal(gpu["path_len"], ref["path_len"]), "path_len"
    assert np.array_equal(gpu["path"], ref["path"]), "path"
    assert gpu["s0_unchanged"], "verify wrote S0"


def gpu_fused_layer(parent, accepted, lay, io, Hk, Hv, device="cuda"):
    """The benchmark's decode step on one layer: the tree is verified on S0
    (cache A), then one gdn_tree_commit_verify launch commits its accepted
    node (S1) and verifies the same tree again on S1 (cache B), exactly the
    launch sequence of every timed step."""
    import torch
    import tree_masked_gated_amd as T
    B, N = parent.shape
    d = lay["S0"].shape[-1]
    dims = T.dims(B, N, Hk, Hv, d, d, io)
    S0 = W.to_device(lay["S0"], device=device)
    x = {key: W.to_device(lay[key], io, device) for key in ("q", "k", "v")}
    x.update({key: W.to_device(lay[key], device=device) for key in ("beta", "g")})
    par = W.to_device(parent.astype(np.int32), device=device)
    acc = W.to_device(np.asarray(accepted, np.int32), device=device)
    o1 = torch.empty((B, N, Hv, d), dtype=x["q"].dtype, device=device)
    o2 = torch.empty_like(o1)
    ca, cb = T.TreeCache(dims, device), T.TreeCache(dims, device)
    S1 = torch.empty_like(S0)
    path = torch.full((B, N), -7, dtype=torch.int32, device=device)
    plen = torch.full((B,), -7, dtype=torch.int32, device=device)
    T.gdn_tree_verify(dims, S0, x["q"], x["k"], x["v"], x["beta"], x["g"], par, o1, ca)
    T.gdn_tree_commit_verify(dims, S0, S1, x["k"], ca, acc, path, plen, x["q"], x["k"],
                             x["v"], x["beta"], x["g"], par, o2, cb)
    torch.cuda.synchronize()
    cache = lambda c: {"u": c.u.cpu().numpy(), "log_gamma": c.log_gamma.cpu().numpy(),
                       "anc_mask": c.anc_mask.cpu().numpy().view(np.uint32),
                       "depth": c.depth.cpu().numpy(), "status": c.tree_status.cpu().numpy()}
    return {"o1": W.from_device_f64(o1), "o2": W.from_device_f64(o2), "A": cache(ca),
            "B": cache(cb), "S1": S1.cpu().numpy().astype(np.float64),
            "path": path.cpu().numpy(), "path_len": plen.cpu().numpy()}


def oracle_paths(parent, accepted):
    """The oracle's committed path and its length for every sequence.  The
    path depends on the tree alone, so the oracle runs on a one-dimensional
    head with zero values."""
    import oracle
    B, N = parent.shape
    z = np.zeros((B, N, 1, 1))
    r = oracle.verify(np.zeros((B, 1, 1, 1)), z, z, z, np.zeros((B, N, 1)), np.ones((B, N, 1)),
                      parent, np.asarray(accepted, np.int32))
    return r["path"], r["path_len"]


def oracle_commit(parent, accepted, lay, io, S0):
    """The oracle's committed state of every sequence's accepted node, from
    the nodes of its root-to-node path alone: the state of a node is the
    sequential rule applied along that path, so the path, relabelled as a
    chain, reaches the same state.  Sequences with shorter paths fill the
    remaining chain slots with independent roots that nothing reads."""
    import oracle
    paths, plen = oracle_paths(parent, accepted)
    B = parent.shape[0]
    P = max(1, int(plen.max()))
    f = lambda a: W.io_to_f64(a, io)
    q, k, v = f(lay["q"]), f(lay["k"]), f(lay["v"])
    Hk, Hv = q.shape[2], v.shape[2]
    cq = np.zeros((B, P) + q.shape[2:]); ck = np.zeros_like(cq)
    cv = np.zeros((B, P) + v.shape[2:])
    cb = np.zeros((B, P, Hv)); cg = np.ones((B, P, Hv))
    cpar = np.full((B, P), -1, np.int32)
    cacc = np.full(B, -1, np.int32)
    for b in range(B):
        n = int(plen[b])
        if n <= 0:
            continue
        nodes = paths[b, :n]
        cq[b, :n], ck[b, :n], cv[b, :n] = q[b, nodes], k[b, nodes], v[b, nodes]
        cb[b, :n], cg[b, :n] = lay["beta"][b, nodes], lay["g"][b, nodes]
        cpar[b, :n] = np.arange(-1, n - 1)
        cacc[b] = n - 1
    r = oracle.verify(np.asarray(S0, np.float64), cq, ck, cv, cb, cg, cpar, cacc, memo=True)
    return r["S_commit"], paths, plen
