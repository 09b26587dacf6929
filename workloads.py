"""Seeded synthetic inputs for GDN draft-tree verification.

This module only draws random numbers and shapes them into trees and tensors.
It holds none of the verification arithmetic, so both the fp64 CPU oracle
(``oracle/``) and the HIP library (``tree_masked_gated_amd``) can be fed from it
without sharing any of the method's code.

Value recipe (the same for every workload; the pages fix none of it, so these
are readings of the workload descriptions):

* q, k ~ N(0, 1), then L2-normalised per node and head (the caller of the
  library normalises; the library applies no scale);
* v ~ N(0, 1);
* beta = sigmoid(N(mu_beta, 1)) with mu_beta = 0, or 2 for the deep-tree
  stress workloads ("beta pushed toward 1");
* g = exp(-softplus(N(0, 1))) = sigmoid(-x), strictly inside (0, 1);
* S0 ~ N(0, 1/d), fp32, layout [d_v][d_k] per value head;
* bf16 workloads round q, k, v from fp32 to bf16 with round-to-nearest-even.

Draws happen in float32 in a fixed order per layer (q, k, v, beta, g, S0), from
``numpy.random.default_rng`` seeded as stated per workload, so every machine
gets the same bytes.

Tree shapes:

* M-ary draft tree of width M and depth gamma (the TreeFlash page's stage-1
  tree keeps exactly M tokens at every depth): node index (j-1)*M + m for depth
  j = 1..gamma; depth-1 nodes hang off the prefix state (parent -1); a depth-j
  node's parent is uniform over the M depth-(j-1) nodes;
* chain: parent[i] = i - 1;
* random recursive tree: parent[0] = -1, parent[i] uniform over [0, i);
* the accepted node is a leaf (a node without children) drawn uniformly.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Spec", "WORKLOADS", "spec", "bf16_bits", "bf16_to_f32", "io_to_f64",
    "tree_binary7", "tree_mary", "tree_chain", "tree_random_recursive",
    "tree_star", "leaves", "pick_leaf", "make_trees", "make_layer",
    "draw_layer", "tree_sizes", "ragged_offsets", "pack_rows", "draft_scores",
]


@dataclasses.dataclass(frozen=True)
class Spec:
    """One synthetic workload: sizes, tree kind, value recipe and seed."""
    name: str
    batch: int
    n_nodes: int
    h_k: int
    h_v: int
    d: int
    io: str            # "f32" or "bf16" for q/k/v/o
    layers: int
    tree: str          # "binary7", "mary", "chain", "rrt"
    seed: int
    width: int = 0     # M for M-ary trees
    depth: int = 0     # gamma for M-ary trees
    beta_mu: float = 0.0
    shared_tree: bool = False   # one tree per sequence shared by all layers
    depths: tuple = ()          # ragged: each M-ary tree's depth drawn from these

    @property
    def group(self) -> int:
        return self.h_v // self.h_k


WORKLOADS: Dict[str, Spec] = {
    # 1 sequence, 1 head, d=16, fp32, 7-node binary tree, accepted node 5.
    "tiny7": Spec("tiny7", 1, 7, 1, 1, 16, "f32", 1, "binary7", 0),
    # 1 sequence, 16 heads, d=128, bf16 q/k/v, M=4 x gamma=16 tree (64 nodes).
    "mary64_b1": Spec("mary64_b1", 1, 64, 16, 16, 128, "bf16", 1, "mary", 1,
                      width=4, depth=16),
    # 32 sequences, 16 key / 32 value heads, 64-node M=4 trees.
    "mary64_b32": Spec("mary64_b32", 32, 64, 16, 32, 128, "bf16", 1, "mary", 2,
                       width=4, depth=16),
    # 36 layers back to back, 64 sequences, 128-node M=8 trees shared by layers.
    "mary128_b64_l36": Spec("mary128_b64_l36", 64, 128, 16, 32, 128, "bf16", 36,
                            "mary", 3, width=8, depth=16, shared_tree=True),
    # The 36-layer step with a ragged batch: 64 sequences whose M=8 trees have
    # depth 2, 4, 8 or 16 (draft budgets of 16 .. 128 nodes), packed by offsets.
    "maryragged_b64_l36": Spec("maryragged_b64_l36", 64, 128, 16, 32, 128, "bf16", 36,
                               "mary", 6, width=8, depth=16, shared_tree=True,
                               depths=(2, 4, 8, 16)),
    # 8 sequences, 16 heads, 256-node chain, beta pushed toward 1.
    "chain256_b8": Spec("chain256_b8", 8, 256, 16, 16, 128, "bf16", 1, "chain", 4,
                        beta_mu=2.0),
    # 8 sequences, 16 heads, 512-node random recursive trees, beta toward 1.
    "rrt512_b8": Spec("rrt512_b8", 8, 512, 16, 16, 128, "bf16", 1, "rrt", 5,
                      beta_mu=2.0),
    # The same two shapes at the largest supported tree, 1024 nodes.
    "chain1024_b8": Spec("chain1024_b8", 8, 1024, 16, 16, 128, "bf16", 1, "chain", 7,
                         beta_mu=2.0),
    "rrt1024_b8": Spec("rrt1024_b8", 8, 1024, 16, 16, 128, "bf16", 1, "rrt", 8,
                       beta_mu=2.0),
}


def spec(name: str) -> Spec:
    return WORKLOADS[name]


# ---------------------------------------------------------------- bf16 codec

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they encode (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def io_to_f64(arr: np.ndarray, io: str) -> np.ndarray:
    """The exact values the library reads, widened to float64."""
    if io == "bf16":
        return bf16_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- trees

def tree_binary7() -> np.ndarray:
    return np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)


def tree_mary(rng: np.random.Generator, width: int, depth: int) -> np.ndarray:
    """M-ary draft tree, node (j-1)*M + m at depth j (1-based)."""
    parent = np.full(width * depth, -1, dtype=np.int32)
    for j in range(2, depth + 1):
        lo = (j - 2) * width
        parent[(j - 1) * width: j * width] = lo + rng.integers(0, width, size=width)
    return parent


def tree_chain(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_random_recursive(rng: np.random.Generator, n: int) -> np.ndarray:
    parent = np.empty(n, dtype=np.int32)
    parent[0] = -1
    for i in range(1, n):
        parent[i] = rng.integers(0, i)
    return parent


def tree_star(n: int) -> np.ndarray:
    """Node 0 under the prefix, every other node a child of node 0."""
    parent = np.zeros(n, dtype=np.int32)
    parent[0] = -1
    return parent


def leaves(parent: np.ndarray) -> np.ndarray:
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    p = parent[parent >= 0]
    has_child[p] = True
    return np.nonzero(~has_child)[0].astype(np.int32)


def pick_leaf(rng: np.random.Generator, parent: np.ndarray) -> int:
    lv = leaves(parent)
    return int(lv[rng.integers(0, len(lv))])


def make_trees(s: Spec):
    """(parent [B][N] int32, accepted [B] int32) for a workload.  A ragged
    workload's sequence b fills its first tree_sizes(s)[b] entries; the rest
    are -1 and belong to no tree."""
    rng = np.random.default_rng(s.seed)
    parent = np.full((s.batch, s.n_nodes), -1, dtype=np.int32)
    accepted = np.empty(s.batch, dtype=np.int32)
    for b in range(s.batch):
        if s.depths:
            p = tree_mary(rng, s.width, int(rng.choice(s.depths)))
            parent[b, :len(p)] = p
            accepted[b] = pick_leaf(rng, p)
            continue
        if s.tree == "binary7":
            p, a = tree_binary7(), 5
        elif s.tree == "mary":
            p = tree_mary(rng, s.width, s.depth)
            a = pick_leaf(rng, p)
        elif s.tree == "chain":
            p, a = tree_chain(s.n_nodes), s.n_nodes - 1
        elif s.tree == "rrt":
            p = tree_random_recursive(rng, s.n_nodes)
            a = pick_leaf(rng, p)
        else:
            raise ValueError(s.tree)
        parent[b] = p
        accepted[b] = a
    return parent, accepted


def tree_sizes(s: Spec) -> np.ndarray:
    """Node count of each sequence's tree (n_nodes unless the workload is
    ragged), int64 [B]."""
    if not s.depths:
        return np.full(s.batch, s.n_nodes, dtype=np.int64)
    rng = np.random.default_rng(s.seed)
    sizes = np.empty(s.batch, dtype=np.int64)
    for b in range(s.batch):          # the same draws as make_trees
        p = tree_mary(rng, s.width, int(rng.choice(s.depths)))
        pick_leaf(rng, p)
        sizes[b] = len(p)
    return sizes


def make_tokens(s: Spec, parent: np.ndarray, accepted: np.ndarray, vocab: int = 32000):
    """Synthetic draft and verifier tokens under which greedy acceptance walks
    exactly to `accepted`: (draft [B][N], target [B][N], target_root [B]),
    int32.  A node on the accepted path carries its predecessor's verifier
    token, every other node a different token."""
    rng = np.random.default_rng(np.random.SeedSequence(s.seed).spawn(2)[1])
    B, N = parent.shape
    target = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
    root = rng.integers(0, vocab, size=B).astype(np.int32)
    draft = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        on_path = np.zeros(N, dtype=bool)
        j = int(accepted[b])
        while j >= 0:
            on_path[j] = True
            j = int(parent[b, j])
        pred = np.where(parent[b] < 0, root[b], target[b, np.maximum(parent[b], 0)])
        draft[b] = np.where(on_path, pred, (pred + 1) % vocab)
    return draft, target, root


# ---------------------------------------------------------------- values

def _normalise(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    x64 /= np.linalg.norm(x64, axis=-1, keepdims=True)
    return x64.astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def draw_layer(rng: np.random.Generator, batch: int, n: int, h_k: int, h_v: int,
               d: int, io: str = "bf16", beta_mu: float = 0.0) -> dict:
    """One layer of inputs. q/k/v are float32 arrays (io "f32") or bf16 bit
    patterns (io "bf16"); beta, g, S0 are float32."""
    q = _normalise(rng.standard_normal((batch, n, h_k, d), dtype=np.float32))
    k = _normalise(rng.standard_normal((batch, n, h_k, d), dtype=np.float32))
    v = rng.standard_normal((batch, n, h_v, d), dtype=np.float32)
    beta = _sigmoid(rng.standard_normal((batch, n, h_v), dtype=np.float32) + beta_mu)
    g = _sigmoid(-rng.standard_normal((batch, n, h_v), dtype=np.float32))
    s0 = (rng.standard_normal((batch, h_v, d, d), dtype=np.float32)
          * np.float32(1.0 / np.sqrt(d)))
    if io == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return {"q": q, "k": k, "v": v, "beta": beta, "g": g, "S0": s0}


def layer_rng(s: Spec, layer: int) -> np.random.Generator:
    if s.layers == 1:
        # single-layer workloads continue from the tree generator's seed space
        return np.random.default_rng(np.random.SeedSequence(s.seed).spawn(1)[0])
    return np.random.default_rng(np.random.SeedSequence(s.seed).spawn(s.layers)[layer])


def make_layer(s: Spec, layer: int = 0) -> dict:
    return draw_layer(layer_rng(s, layer), s.batch, s.n_nodes, s.h_k, s.h_v, s.d,
                      s.io, s.beta_mu)


def unit_slice(s: Spec, lay: dict, parent: np.ndarray, accepted: np.ndarray,
               b: int, h: int) -> dict:
    """Inputs of one (sequence b, value head h) unit as float64, for the oracle.
    Value head h reads key head h // (h_v / h_k)."""
    hk = h // s.group
    return {
        "q": io_to_f64(lay["q"][b:b + 1, :, hk:hk + 1], s.io),
        "k": io_to_f64(lay["k"][b:b + 1, :, hk:hk + 1], s.io),
        "v": io_to_f64(lay["v"][b:b + 1, :, h:h + 1], s.io),
        "beta": lay["beta"][b:b + 1, :, h:h + 1].astype(np.float64),
        "g": lay["g"][b:b + 1, :, h:h + 1].astype(np.float64),
        "S0": lay["S0"][b:b + 1, h:h + 1].astype(np.float64),
        "parent": parent[b:b + 1],
        "accepted": accepted[b:b + 1],
    }


# ---------------------------------------------------------------- ragged batches

def ragged_offsets(lens) -> np.ndarray:
    """int32 [B + 1] first rows of B packed trees of sizes lens."""
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def pack_rows(dense: np.ndarray, lens) -> np.ndarray:
    """Rows 0 .. lens[b] - 1 of every sequence b of a [B][N][...] array, packed
    sequence after sequence into [sum(lens)][...]."""
    parts = [dense[b, :n] for b, n in enumerate(lens)]
    return np.ascontiguousarray(np.concatenate(parts, axis=0)) if parts else dense[:0, 0]


# ---------------------------------------------------------------- drafter scores

def draft_scores(rng: np.random.Generator, batch: int, n: int, k: int, vocab: int = 32000,
                 sigma: float = 2.0):
    """Synthetic drafter outputs for tree construction: for the prefix and each
    of n node indices, the top-k continuations of a distribution over `vocab`
    tokens whose k candidates have logits ln(vocab) + N(0, sigma^2) and whose
    other vocab - k tokens have logit 0 (so the candidates hold most of the
    mass, the best one typically well over half, as a confident drafter's
    would).  Returns (logp [batch][n + 1][k] float32, descending per row; tok
    [batch][n + 1][k] int32, distinct per row)."""
    z = np.log(vocab) + rng.standard_normal((batch, n + 1, k)) * sigma
    zmax = np.maximum(z.max(axis=-1, keepdims=True), 0.0)
    denom = np.exp(z - zmax).sum(axis=-1, keepdims=True) + (vocab - k) * np.exp(-zmax)
    logp = np.sort(z - zmax - np.log(denom), axis=-1)[..., ::-1].astype(np.float32)
    tok = np.empty((batch, n + 1, k), dtype=np.int32)
    for b in range(batch):
        for r in range(n + 1):
            tok[b, r] = rng.choice(vocab, size=k, replace=False)
    return np.ascontiguousarray(logp), tok


# ---------------------------------------------------------------- upload

def to_device(arr: np.ndarray, io: str = "", device="cuda"):
    """numpy -> torch device tensor.  io="bf16" reinterprets uint16 bit
    patterns as torch.bfloat16; everything else keeps its dtype."""
    import torch
    a = np.ascontiguousarray(arr)
    if io == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def from_device_f64(t, io: str = "") -> np.ndarray:
    """torch tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)
