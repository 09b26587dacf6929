"""Benchmark: tree nodes verified per second per GDN layer on one MI355X.

A step is one decode iteration of the 36-layer stack: for every layer, verify
all 64 draft trees (128 nodes, M = 8 wide, 16 deep; 16 key / 32 value heads,
d = 128, bf16 q/k/v, fp32 state) and commit each sequence's accepted node,
found on the device by the greedy acceptance walk over synthetic draft and
verifier tokens (once per step; the tokens make it accept a random leaf).
The committed states of step t are the prefix states of step t + 1, as in a
decode loop.  By default each layer is one launch of gdn_tree_commit_verify:
the commit of the tree verified at the previous step, then this step's
verification on the committed state (the tree verified before the first timed
step is primed untimed).  --unfused times gdn_tree_verify + gdn_tree_commit
per layer instead.  All inputs are synthetic (workloads.py) and resident in HBM
before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--unfused]

Prints one JSON line.  value = B * N * layer calls * K / elapsed, i.e. nodes
per second per layer (each layer call verifies B * N nodes and commits B
paths).  A workload whose inputs would fit in the last-level cache runs
copies of its layers on separate buffers (config.input_copies), so that
repeated steps read HBM, not that cache.
The roofline block reports the dominant kernel (the fused launch, or the
verification when unfused): algorithmic bytes per launch over its average
launch time, measured with HIP events recorded on the launch stream around
each timed step's block of those launches.  The
cpu_baseline block times the fp64 oracle (path-walk mode) on a bounded sample
of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- byte model

def verify_bytes(s, e, sizes):
    """Algorithmic HBM bytes of one verify launch, summed over the sequences (a
    tree of n nodes): S0 read once, q/k read once per key head, v read,
    beta/g/parent read, o written, the cache rows of the n nodes written (u,
    Gamma, ancestor rows, depth) and the status; a ragged batch also reads its
    two offsets per sequence."""
    Hk, Hv, d = s.h_k, s.h_v, s.d
    Wd = (s.n_nodes + 31) // 32
    tot = 0
    for n in sizes:
        n = int(n)
        tot += (4 * Hv * d * d + 2 * n * Hk * d * e + n * Hv * d * e + 8 * n * Hv + 4 * n
                + n * Hv * d * e + 4 * n * Hv * d + 4 * n * Hv + 4 * n * Wd + 4 * n + 4
                + (8 if s.depths else 0))
    return tot


def commit_bytes(s, e, path_lens, sizes):
    """Algorithmic bytes of one commit launch: S in + out, and per path node its
    u row, k row and Gamma, plus the accepted row of the ancestor mask, the
    path written (the tree's n slots) and the small per-sequence scalars."""
    Hk, Hv, d = s.h_k, s.h_v, s.d
    Wd = (s.n_nodes + 31) // 32
    tot = 0
    for P, n in zip(path_lens, sizes):
        P = max(int(P), 0)
        tot += (8 * Hv * d * d + P * (4 * Hv * d + Hk * d * e + 4 * Hv) + 4 * Hv
                + 4 * Wd + 4 * int(n) + 12 + (8 if s.depths else 0))
    return tot


# ---------------------------------------------------------------- GPU run

def run_gpu(args, s):
    import torch
    import tree_masked_gated_amd as T

    dev = torch.device("cuda:0")
    e = 2 if s.io == "bf16" else 4
    parent, accepted = W.make_trees(s)
    sizes = W.tree_sizes(s)
    ragged = bool(s.depths)
    # a ragged batch: per-node arrays packed tree after tree, located by offsets
    pack = (lambda a: W.pack_rows(a, sizes)) if ragged else (lambda a: a)
    L = s.layers
    log(f"generating {L} layers of {s.name} on the host")
    t0 = time.time()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, L)) as ex:
        futs = [ex.submit(W.make_layer, s, l) for l in range(L)]
        layers = []
        for l, f in enumerate(futs):
            lay = f.result()
            if ragged:
                lay.update({key: pack(lay[key]) for key in ("q", "k", "v", "beta", "g")})
            layers.append({
                "q": W.to_device(lay["q"], s.io, dev), "k": W.to_device(lay["k"], s.io, dev),
                "v": W.to_device(lay["v"], s.io, dev),
                "beta": W.to_device(lay["beta"], device=dev),
                "g": W.to_device(lay["g"], device=dev),
                "S": [W.to_device(lay["S0"], device=dev), None],
            })
            layers[-1]["S"][1] = torch.empty_like(layers[-1]["S"][0])
            del lay
    log(f"generated and uploaded in {time.time() - t0:.1f} s")
    dims = T.dims(s.batch, s.n_nodes, s.h_k, s.h_v, s.d, s.d, s.io)
    # A workload whose inputs fit in the 256 MB last-level (Infinity) cache
    # would be served from it on repeated steps.  Its layers are then
    # replicated on the device into copies that together hold at least
    # 512 MiB, and a step runs every copy in turn: each copy is one more
    # layer call of the same work on different buffers.
    nbytes = lambda t: t.numel() * t.element_size()
    cache_b = sum(T.gdn_tree_cache_bytes(dims).values()) * (2 if args.fused else 1)
    rows_n = int(sizes.sum()) if ragged else s.batch * s.n_nodes
    o_b = rows_n * s.h_v * s.d * e
    per_layer = (sum(nbytes(layers[0][k]) for k in ("q", "k", "v", "beta", "g"))
                 + 2 * nbytes(layers[0]["S"][0]) + cache_b + o_b)
    copies = min(64, max(1, math.ceil(512 * 2**20 / (L * per_layer))))
    for _ in range(copies - 1):
        for l in range(L):
            x = layers[l]
            layers.append({k: x[k].clone() for k in ("q", "k", "v", "beta", "g")})
            layers[-1]["S"] = [x["S"][0].clone(), torch.empty_like(x["S"][0])]
    if copies > 1:
        log(f"{copies} copies of the layer inputs ({copies * L * per_layer / 2**20:.0f} MiB resident)")
    L = L * copies
    par = W.to_device(pack(parent), device=dev)
    # the acceptance walk runs on the device each step and writes acc; the
    # synthetic tokens make it accept the workload's chosen leaf
    draft, target, troot = W.make_tokens(s, parent, accepted)
    draft, target, troot = (W.to_device(x, device=dev) for x in (pack(draft), pack(target), troot))
    if ragged:
        offs = W.to_device(W.ragged_offsets(sizes), device=dev)
        T.check_offsets(offs, dims, int(sizes.sum()))
    acc = torch.empty((s.batch,), dtype=torch.int32, device=dev)
    alen = torch.empty((s.batch,), dtype=torch.int32, device=dev)
    nxt = torch.empty((s.batch,), dtype=torch.int32, device=dev)
    # two caches per layer: the fused step reads the previous tree's while it
    # writes the new tree's
    caches2 = [[T.TreeCache(dims, dev), T.TreeCache(dims, dev) if args.fused else None]
               for _ in range(L)]
    caches = [c[0] for c in caches2]
    rows = (int(sizes.sum()),) if ragged else (s.batch, s.n_nodes)
    o = [torch.empty(rows + (s.h_v, s.d), dtype=layers[0]["q"].dtype, device=dev)
         for _ in range(L)]
    path = torch.empty(rows, dtype=torch.int32, device=dev)
    plen = torch.empty((s.batch,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    phase = [0]
    # (ragged: the same trees every step, so the previous tree's offsets are
    # this step's)
    R = (lambda name: getattr(T, name + "_ragged")) if ragged else (lambda name: getattr(T, name))
    O = (lambda: (offs,)) if ragged else (lambda: ())

    def verify(l):
        x = layers[l]
        R("gdn_tree_verify")(dims, *O(), x["S"][phase[0]], x["q"], x["k"], x["v"], x["beta"],
                             x["g"], par, o[l], caches[l], sptr)

    def commit(l):
        x = layers[l]
        R("gdn_tree_commit")(dims, *O(), x["S"][phase[0]], x["S"][1 - phase[0]], x["k"],
                             caches[l], acc, path, plen, sptr)

    cur = [0]

    def commit_verify(l):
        x = layers[l]
        R("gdn_tree_commit_verify")(dims, *O(), x["S"][phase[0]], x["S"][1 - phase[0]], x["k"],
                                    caches2[l][cur[0]], acc, path, plen, *O(), x["q"], x["k"],
                                    x["v"], x["beta"], x["g"], par, o[l], caches2[l][1 - cur[0]],
                                    sptr)

    def accept(_l=0):
        R("gdn_tree_accept")(dims, *O(), par, draft, target, troot, acc, alen, nxt, sptr)

    # events around each step's block of dominant-kernel launches (the fused
    # launches, or the verifications when unfused), recorded on the launch
    # stream inside the timed region: the roofline's launch time
    marks = []

    def step(mark=False):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if mark else None
        if args.fused:
            # commit of the tree verified last step, then this step's tree,
            # then its acceptance walk (read by the next step's commits)
            if ev: ev[0].record(stream)
            for l in range(L):
                commit_verify(l)
            if ev: ev[1].record(stream)
            accept()
            cur[0] ^= 1
        else:
            if ev: ev[0].record(stream)
            for l in range(L):
                verify(l)
            if ev: ev[1].record(stream)
            accept()
            for l in range(L):
                commit(l)
        phase[0] ^= 1
        if ev: marks.append(ev)

    if args.fused:
        for l in range(L):            # the first tree has no commit before it
            verify(l)
    accept()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step(mark=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    per_step = sorted(a.elapsed_time(b) / L for a, b in marks)
    live_ms = sum(per_step) / len(per_step)
    live_med_ms = per_step[len(per_step) // 2]
    log(f"timed {args.steps} steps: {total_ms:.3f} ms; dominant launch {live_ms * 1e3:.1f} us in the timed region")

    # per-kernel averages, same stream, same launch configuration
    reps = max(1, args.steps)

    def timed(fn):
        for l in range(L):          # untimed: a kernel's first launch loads its code
            fn(l)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            for l in range(L):
                fn(l)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * L)

    fused_ms = timed(commit_verify) if args.fused else None
    verify_ms = timed(verify)
    commit_ms = timed(commit)
    accept_ms = timed(accept)
    log(f"verify {verify_ms * 1e3:.1f} us/launch, commit {commit_ms * 1e3:.1f} us/launch"
        + (f", commit+verify {fused_ms * 1e3:.1f} us/launch" if args.fused else "")
        + f", accept {accept_ms * 1e3:.1f} us/launch")
    path_lens = plen.cpu().numpy()
    assert np.array_equal(acc.cpu().numpy(), accepted), "the acceptance walk missed the chosen leaf"
    build = time_tree_build(s, stream, reps)
    return {
        "total_ms": total_ms, "verify_ms": verify_ms, "commit_ms": commit_ms,
        "fused_ms": fused_ms, "accept_ms": accept_ms, "live_ms": live_ms, "live_med_ms": live_med_ms,
        "verify_bytes": verify_bytes(s, e, sizes),
        "commit_bytes": commit_bytes(s, e, path_lens, sizes),
        "path_lens": path_lens, "parent": parent, "accepted": accepted, "sizes": sizes,
        "build": build, "layer_calls": L, "copies": copies,
    }


def time_tree_build(s, stream, reps, topk=8):
    """The step before verification: building the batch's draft trees from the
    drafter's top-k continuations with w = M expansions per step (a tree of the
    workload's largest size; synthetic drafter scores).  Timed with HIP events
    on the launch stream, like the other kernels."""
    import torch
    import tree_masked_gated_amd as T
    w = s.width or 8
    N = s.n_nodes
    lp, tk = W.draft_scores(np.random.default_rng(s.seed + 1000), s.batch, N, topk)
    bd = T.build_dims(s.batch, N, topk, w)
    lp_d, tk_d = W.to_device(lp), W.to_device(tk)
    par = torch.empty((s.batch, N), dtype=torch.int32, device="cuda")
    tok = torch.empty_like(par)
    sc = torch.empty((s.batch, N), dtype=torch.float32, device="cuda")
    sptr = stream.cuda_stream
    T.gdn_tree_build(bd, lp_d, tk_d, par, tok, sc, sptr)     # untimed: code load
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        T.gdn_tree_build(bd, lp_d, tk_d, par, tok, sc, sptr)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    log(f"tree build {ms * 1e3:.1f} us/launch ({s.batch} trees of {N} nodes, k {topk}, w {w})")
    return {"launch_us": ms * 1e3, "batch": s.batch, "n_nodes": N, "topk": topk, "width": w,
            "steps": -(-N // w), "trees_per_s": s.batch / (ms * 1e-3)}


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(s, budget_s):
    """The fp64 oracle, path-walk mode, on the first sequences of layer 0 (all
    value heads), growing the sample until it took about budget_s seconds.  A
    ragged batch's trees each run at their own size."""
    import oracle
    lib = oracle.load()
    parent, accepted = W.make_trees(s)
    sizes = W.tree_sizes(s)
    lay = W.make_layer(s, 0)
    f = lambda a: W.io_to_f64(a, s.io)

    def run(b0, b1, n):
        sl = slice(b0, b1)
        oracle.verify(lay["S0"][sl].astype(np.float64), f(lay["q"][sl, :n]), f(lay["k"][sl, :n]),
                      f(lay["v"][sl, :n]), lay["beta"][sl, :n].astype(np.float64),
                      lay["g"][sl, :n].astype(np.float64), parent[sl, :n], accepted[sl],
                      memo=False, lib=lib)

    nb = 1
    while True:
        t0 = time.perf_counter()
        if s.depths:
            for b in range(nb):
                run(b, b + 1, int(sizes[b]))
        else:
            run(0, nb, s.n_nodes)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or nb >= s.batch:
            break
        nb = min(s.batch, nb * 2)
    nodes = int(sizes[:nb].sum())
    return {"value": nodes / dt, "unit": "nodes/s/layer", "cores": oracle.max_threads(lib),
            "kind": "oracle",
            "sample": f"layer 0, sequences 0..{nb - 1} (all {s.h_v} value heads, "
                      f"{nodes} nodes), fp64 path walk, {dt:.2f} s"}


# ---------------------------------------------------------------- copy

def copy_bandwidth(mib):
    """A plain device-to-device copy of a known size (torch's copy kernel): the
    reference for scaling FETCH_SIZE / WRITE_SIZE counters and the achievable
    streaming bandwidth on this machine.  Returns what it measured."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = 2 * n * 4
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4,
            "us_per_copy": ms * 1e3, "GBs": moved / (ms * 1e-3) / 1e9}


# ---------------------------------------------------------------- traffic

def profiled_traffic(kernel, workload):
    """HBM bytes per launch of kernel measured by the FETCH_SIZE / WRITE_SIZE
    counter passes (profiles/<kernel>_traffic_<workload>.txt), or None when there
    is no such record or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    traffic, ok = None, True
    for line in open(path):
        line = line.strip()
        if line.startswith("traffic_bytes="):
            traffic = int(line.split("=", 1)[1])
        elif line.startswith("sha256 "):
            rel, digest = line[len("sha256 "):].split("=", 1)
            with open(os.path.join(ROOT, rel), "rb") as f:
                ok &= hashlib.sha256(f.read()).hexdigest() == digest
    return traffic if ok else None


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mary128_b64_l36")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--unfused", dest="fused", action="store_false",
                    help="verify and commit as two launches per layer")
    args = ap.parse_args()
    if args.copy_calibration:
        print(json.dumps(copy_bandwidth(args.copy_calibration)), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every (sequence, value head) unit is "
              "independent, so the path shards across GPUs without exchange; run it "
              "with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    s = W.spec(args.workload)
    r = run_gpu(args, s)
    L = s.layers
    nodes = int(r["sizes"].sum())
    value = nodes * r["layer_calls"] * args.steps / (r["total_ms"] * 1e-3)
    # the dominant kernel's launch time, measured in the timed region
    launch_ms = r["live_ms"]
    if args.fused:
        # the fused launch reads the state once for both halves
        kernel = "commit_verify"
        vb = r["verify_bytes"] + r["commit_bytes"] - 4 * s.batch * s.h_v * s.d * s.d
    else:
        kernel = "verify"
        vb = r["verify_bytes"]
    achieved = vb / (launch_ms * 1e-3) / 1e9
    # what plain streaming reaches here: 1 GiB read + 1 GiB written, after the
    # timed region
    copy_gbs = copy_bandwidth(1024)["GBs"]
    base = None
    if args.cpu_budget > 0:
        log("timing the oracle on the host")
        base = cpu_baseline(s, args.cpu_budget)

    out = {
        "metric": "tree nodes verified/sec per GDN layer",
        "value": value,
        "unit": "nodes/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["total_ms"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-io/f32-state" if s.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": s.name, "batch": s.batch, "n_nodes": s.n_nodes, "layers": L,
            "tree": (f"{s.width}-ary x depth {'/'.join(map(str, s.depths))} (ragged, "
                     f"{nodes} nodes)" if s.depths else
                     f"{s.width}-ary x depth {s.depth}" if s.tree == "mary" else s.tree),
            "h_k": s.h_k, "h_v": s.h_v, "d_k": s.d, "d_v": s.d, "io": s.io,
            "state": "f32", "launches": "commit_verify" if args.fused else "verify+commit",
            "input_copies": r["copies"],
        },
        "roofline": {
            "bound": "hbm", "kernel": kernel, "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": profiled_traffic(kernel, s.name), "alg_bytes_per_launch": vb,
            "launch_us": launch_ms * 1e3,
            "launch_us_median_step": r["live_med_ms"] * 1e3,
            "copy_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs,
        },
        "verify": {
            "launch_us": r["verify_ms"] * 1e3, "alg_bytes_per_launch": r["verify_bytes"],
            "achieved_GBs": r["verify_bytes"] / (r["verify_ms"] * 1e-3) / 1e9,
        },
        "commit": {
            "launch_us": r["commit_ms"] * 1e3, "alg_bytes_per_launch": r["commit_bytes"],
            "achieved_GBs": r["commit_bytes"] / (r["commit_ms"] * 1e-3) / 1e9,
        },
        "accept": {"launch_us": r["accept_ms"] * 1e3, "per": "step"},
        "tree_build": r["build"],
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
