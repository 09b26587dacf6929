"""Run the HIP library and the oracle on the same seeded inputs and compare.

Shared by the GPU parity tests.  Inputs come from workloads.py only; expected
values come from the oracle only."""
import numpy as np

import workloads as W


def rel_l2(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


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
