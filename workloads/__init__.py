"""Seeded synthetic inputs for the verify-and-resample step.

This module is the one piece shared by the CPU oracle's tests and the GPU path's
tests and benchmark.  It only *constructs inputs*: logit tensors, draft tokens,
uniform random numbers and draft trees.  It holds none of the verification
arithmetic (no acceptance test, no residual, no tree acceptance); the draft
tokens come from a stand-in drafter (`drafter_tokens`, `greedy_drafter_tokens`)
that plays the role of the draft model, which sits upstream of verification.

Workload shapes follow the five settings the pages' experiments imply:

* sampling verify of a T5-sized vocabulary (32000) in fp32;
* greedy verify and sampling verify of a Llama-3-sized vocabulary (128256) in bf16;
* large-batch sampling with temperature and top-p on a Qwen2.5-sized vocabulary
  (152064) in fp32 with Zipf-shaped logits;
* greedy verification of merged two-drafter trees (TAPS, aitrends.kr, section
  "방법론": two drafters' trees under one shared root, one target pass).

No dataset item is used or needed: verification never sees text, only logits and
token ids.  Every array is drawn from numpy's PCG64 seeded by a SeedSequence
built from (20261202 + config index, user seed), spawned into named streams.

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even from
an fp32 draw); uniforms lie on the grid k * 2**-24, k in [0, 2**24), so they are
exact in fp32 and fp64 and never equal 1.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BASE_SEED = 20261202
STREAMS = ("logits", "noise", "tokens", "uniforms", "tree")

SAMPLE, GREEDY, TREE = "sample", "greedy", "tree"


# --------------------------------------------------------------------------
# basic helpers (input construction only)
# --------------------------------------------------------------------------

def rngs(config_index: int, seed: int = 0) -> Dict[str, np.random.Generator]:
    ss = np.random.SeedSequence([BASE_SEED + int(config_index), int(seed)])
    return {name: np.random.Generator(np.random.PCG64(child))
            for name, child in zip(STREAMS, ss.spawn(len(STREAMS)))}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms_on_grid(rng: np.random.Generator, shape) -> np.ndarray:
    """U[0,1) on the 2**-24 grid, as float32 (exact)."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def logits_as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float32)


# --------------------------------------------------------------------------
# stand-in drafters (they play the draft model; verification never calls them)
# --------------------------------------------------------------------------

def drafter_tokens(draft_f32: np.ndarray, temperature: float, top_p: float,
                   rng: np.random.Generator) -> np.ndarray:
    """Draw one token per draft row, as a sampling drafter at `temperature`
    (and nucleus `top_p`) would.  Uses the Gumbel-max trick, so no normalised
    distribution is formed; with top_p < 1 the draw is restricted to the
    drafter's own nucleus (largest logits whose tempered mass first reaches
    top_p).  draft_f32: [..., V] -> int32 [...]."""
    lead = draft_f32.shape[:-1]
    V = draft_f32.shape[-1]
    rows = draft_f32.reshape(-1, V)
    out = np.empty(rows.shape[0], dtype=np.int32)
    for r in range(rows.shape[0]):
        l = rows[r].astype(np.float64) / float(temperature)
        if top_p < 1.0:
            order = np.argsort(-l, kind="stable")
            w = np.exp(l[order] - l[order[0]])
            cum = np.cumsum(w) / w.sum()
            keep = int(np.searchsorted(cum, top_p)) + 1
            allowed = np.full(V, -np.inf)
            allowed[order[:keep]] = 0.0
            l = l + allowed
        g = -np.log(-np.log(rng.uniform(np.finfo(np.float64).tiny, 1.0, size=V)))
        out[r] = int(np.argmax(l + g))
    return out.reshape(lead)


def greedy_drafter_tokens(target_f32: np.ndarray, agree: float,
                          rng: np.random.Generator) -> np.ndarray:
    """Greedy drafter stand-in: per row, the target's top choice (first
    occurrence) with probability `agree`, else a uniform id in [0, V)."""
    V = target_f32.shape[-1]
    top = np.argmax(target_f32, axis=-1).astype(np.int32)
    coin = rng.random(size=top.shape) < agree
    rand = rng.integers(0, V, size=top.shape, dtype=np.int64).astype(np.int32)
    return np.where(coin, top, rand).astype(np.int32)


# --------------------------------------------------------------------------
# draft trees (two drafters, merged under one root)
# --------------------------------------------------------------------------

def grow_tree(rng: np.random.Generator, n_nonroot: int, max_depth: int = 8,
              max_children: int = 4) -> np.ndarray:
    """Random draft tree: repeatedly attach a child to a uniformly chosen node
    with depth < max_depth and < max_children children; then renumber in BFS
    order so that every parent index is smaller than its child's.
    Returns parents[n_nonroot + 1] with parents[0] = -1."""
    parent, depth, nchild = [-1], [0], [0]
    while len(parent) < n_nonroot + 1:
        eligible = [i for i in range(len(parent))
                    if depth[i] < max_depth and nchild[i] < max_children]
        p = eligible[int(rng.integers(len(eligible)))]
        parent.append(p)
        depth.append(depth[p] + 1)
        nchild[p] += 1
        nchild.append(0)
    n = len(parent)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    order, head = [0], 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new_index = {old: new for new, old in enumerate(order)}
    out = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        out[new_index[old]] = new_index[parent[old]]
    return out


def ancestor_mask(parents: np.ndarray) -> np.ndarray:
    """Ancestor-or-self matrix of one tree (row i has a 1 at i and at every
    ancestor of i), the per-tree attention mask a drafter hands over."""
    n = len(parents)
    m = np.zeros((n, n), dtype=np.uint8)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j] = 1
            j = int(parents[j])
    return m


def merge_two_trees(parents1, tokens1, parents2, tokens2):
    """Two drafters' trees under one shared root (TAPS, aitrends.kr, section
    "방법론": both trees verified in one target pass under a mask that keeps
    each branch blind to the other).  Node numbering: the shared root first
    (it carries tree 1's root token), then tree 1's non-root nodes in their
    own order, then tree 2's; a tree-2 node hanging from its root hangs from
    the shared root, any other tree-2 parent index moves up by n1 (tree 1's
    non-root node count).  The mask is the ancestor-or-self closure of the
    merged parents.  Returns (parents[N], tokens[N], mask[N, N]), N = n1 + n2 + 1."""
    p1 = np.asarray(parents1, np.int64)
    p2 = np.asarray(parents2, np.int64)
    n1 = len(p1) - 1
    moved = np.where(p2[1:] == 0, 0, p2[1:] + n1)
    parents = np.concatenate([p1, moved]).astype(np.int32)
    tokens = np.concatenate([np.asarray(tokens1, np.int32), np.asarray(tokens2, np.int32)[1:]])
    return parents, tokens, ancestor_mask(parents)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    kind: str                    # SAMPLE | GREEDY | TREE
    name: str
    B: int
    K: int                       # draft positions (TREE: N nodes)
    V: int
    dtype: str                   # "f32" | "bf16"
    target: np.ndarray           # [B, K+1, V] (TREE: [B, N, V]); float32 or uint16 bits
    draft: Optional[np.ndarray] = None        # [B, K, V]   (SAMPLE)
    tokens: Optional[np.ndarray] = None       # [B, K] int32 (TREE: node tokens [B, N])
    u_accept: Optional[np.ndarray] = None     # [B, K] float32
    u_sample: Optional[np.ndarray] = None     # [B] float32
    temperature: float = 1.0
    top_p: float = 1.0
    parents: Optional[np.ndarray] = None      # [B, N] int32 (TREE)
    anc_mask: Optional[np.ndarray] = None     # [B, N, N] uint8 (TREE)

    @property
    def rows(self) -> int:
        if self.kind == SAMPLE:
            return self.B * (2 * self.K + 1)
        if self.kind == GREEDY:
            return self.B * (self.K + 1)
        return self.B * self.K

    @property
    def logit_bytes(self) -> int:
        return self.rows * self.V * (2 if self.dtype == "bf16" else 4)

    @property
    def positions(self) -> int:
        """Target positions whose outcome one call decides."""
        return self.B * (self.K if self.kind == TREE else self.K + 1)


def _to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def sample_gaussian(cfg: int, B: int, K: int, V: int, dtype: str, sigma: float,
                    noise: float, temperature: float, seed: int = 0,
                    name: str = "sample") -> Workload:
    """Sampling verify: target ~ N(0, sigma^2) for K+1 positions; draft = the
    first K target rows + N(0, noise^2); each tensor rounded to `dtype`
    independently; draft tokens drawn from the tempered draft."""
    r = rngs(cfg, seed)
    t32 = (r["logits"].standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(sigma))
    d32 = t32[:, :K] + r["noise"].standard_normal((B, K, V), dtype=np.float32) * np.float32(noise)
    target = _to_dtype(t32, dtype)
    draft = _to_dtype(d32, dtype)
    T = float(np.float32(temperature))
    toks = drafter_tokens(logits_as_f32(draft, dtype), T, 1.0, r["tokens"])
    return Workload(SAMPLE, name, B, K, V, dtype, target, draft, toks,
                    uniforms_on_grid(r["uniforms"], (B, K)),
                    uniforms_on_grid(r["uniforms"], (B,)), T, 1.0)


def sample_zipf_topp(cfg: int, B: int, K: int, V: int, temperature: float,
                     top_p: float, seed: int = 0, name: str = "topp",
                     dtype: str = "f32") -> Workload:
    """Large-batch sampling with top-p: per row an independent random
    permutation pi of [0, V); base_j = -1.1 ln(pi(j) + 1); target = base +
    N(0, 1); draft = target + N(0, 1.5^2); tokens from the drafter's own
    tempered nucleus."""
    r = rngs(cfg, seed)
    t32 = np.empty((B, K + 1, V), dtype=np.float32)
    for b in range(B):
        for i in range(K + 1):
            perm = r["logits"].permutation(V).astype(np.float64)
            t32[b, i] = (-1.1 * np.log(perm + 1.0)).astype(np.float32)
    t32 += r["noise"].standard_normal((B, K + 1, V), dtype=np.float32)
    d32 = t32[:, :K] + r["noise"].standard_normal((B, K, V), dtype=np.float32) * np.float32(1.5)
    target = _to_dtype(t32, dtype)
    draft = _to_dtype(d32, dtype)
    T = float(np.float32(temperature))
    P = float(np.float32(top_p))
    toks = drafter_tokens(logits_as_f32(draft, dtype), T, P, r["tokens"])
    return Workload(SAMPLE, name, B, K, V, dtype, target, draft, toks,
                    uniforms_on_grid(r["uniforms"], (B, K)),
                    uniforms_on_grid(r["uniforms"], (B,)), T, P)


def greedy_gaussian(cfg: int, B: int, K: int, V: int, dtype: str = "bf16",
                    sigma: float = 2.5, agree: float = 0.7, seed: int = 0,
                    name: str = "greedy") -> Workload:
    r = rngs(cfg, seed)
    t32 = r["logits"].standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(sigma)
    target = _to_dtype(t32, dtype)
    toks = greedy_drafter_tokens(logits_as_f32(target[:, :K], dtype), agree, r["tokens"])
    return Workload(GREEDY, name, B, K, V, dtype, target, tokens=toks)


def tree_merged(cfg: int, B: int, n_per_tree: int, V: int, dtype: str = "bf16",
                sigma: float = 2.5, agree: float = 0.6, seed: int = 0,
                max_depth: int = 8, max_children: int = 4,
                name: str = "tree") -> Workload:
    """Greedy tree verify: per request two random trees of `n_per_tree`
    non-root nodes, merged under one root (N = 2 n_per_tree + 1).  Target
    logits per merged node ~ N(0, sigma^2); each child's token is the target's
    top choice at its parent with probability `agree`, else a uniform id; the
    root token is uniform."""
    r = rngs(cfg, seed)
    N = 2 * n_per_tree + 1
    t32 = r["logits"].standard_normal((B, N, V), dtype=np.float32) * np.float32(sigma)
    target = _to_dtype(t32, dtype)
    top = np.argmax(logits_as_f32(target, dtype), axis=-1)  # [B, N], the drafter's view
    parents = np.empty((B, N), np.int32)
    tokens = np.empty((B, N), np.int32)
    masks = np.empty((B, N, N), np.uint8)
    for b in range(B):
        p1 = grow_tree(r["tree"], n_per_tree, max_depth, max_children)
        p2 = grow_tree(r["tree"], n_per_tree, max_depth, max_children)
        zeros1 = np.zeros(len(p1), np.int32)
        zeros2 = np.zeros(len(p2), np.int32)
        par, _, mask = merge_two_trees(p1, zeros1, p2, zeros2)
        tok = np.empty(N, np.int32)
        tok[0] = int(r["tokens"].integers(0, V))
        for i in range(1, N):
            if r["tokens"].random() < agree:
                tok[i] = int(top[b, par[i]])
            else:
                tok[i] = int(r["tokens"].integers(0, V))
        parents[b], tokens[b], masks[b] = par, tok, mask
    return Workload(TREE, name, B, N, V, dtype, target, tokens=tokens,
                    parents=parents, anc_mask=masks)


# The five settings (index 0..4).  `scale` shrinks B and V for quick parity
# runs while keeping the recipe; K / tree shape are kept.
CONFIG_NAMES = (
    "sample B4 K4 V32000 f32 T1",
    "greedy B64 K5 V128256 bf16",
    "sample B64 K8 V128256 bf16 T0.7",
    "sample+top-p B256 K4 V152064 f32 T0.8 p0.95",
    "greedy tree B32 N63 V128256 bf16",
)


def make_config(index: int, seed: int = 0, B: Optional[int] = None,
                V: Optional[int] = None, K: Optional[int] = None) -> Workload:
    if index == 0:
        return sample_gaussian(0, B or 4, K or 4, V or 32000, "f32", 3.0, 1.0, 1.0,
                               seed, CONFIG_NAMES[0])
    if index == 1:
        return greedy_gaussian(1, B or 64, K or 5, V or 128256, "bf16", 2.5, 0.7, seed,
                               name=CONFIG_NAMES[1])
    if index == 2:
        return sample_gaussian(2, B or 64, K or 8, V or 128256, "bf16", 3.0, 0.5, 0.7,
                               seed, CONFIG_NAMES[2])
    if index == 3:
        return sample_zipf_topp(3, B or 256, K or 4, V or 152064, 0.8, 0.95, seed,
                                CONFIG_NAMES[3])
    if index == 4:
        n = 31 if K is None else (K - 1) // 2
        return tree_merged(4, B or 32, n, V or 128256, "bf16", 2.5, 0.6, seed,
                           name=CONFIG_NAMES[4])
    raise ValueError(f"no workload {index}")


def subset(w: "Workload", requests) -> "Workload":
    """The same workload restricted to some of its requests."""
    import dataclasses
    r = np.asarray(requests)
    kw = dict(B=len(r), target=w.target[r])
    for name in ("draft", "tokens", "u_accept", "u_sample", "parents", "anc_mask"):
        v = getattr(w, name)
        if v is not None:
            kw[name] = v[r]
    return dataclasses.replace(w, **kw)


@dataclasses.dataclass
class KVWorkload:
    """A KV-cache commit: cache [L, 2, B, H, S, D] of 16-bit words (each
    row distinct), per-request committed length, and the accepted path of
    the cycle (tree node ids by depth, or None for a linear draft)."""
    name: str
    kv: np.ndarray
    cache_len: np.ndarray
    path_len: np.ndarray
    path_nodes: Optional[np.ndarray]
    N: int
    mirror: Optional[np.ndarray]

    @property
    def shape(self):
        return self.kv.shape


def random_paths(rng: np.random.Generator, B: int, n_per_tree: int):
    """Accepted paths in merged trees of 2 n_per_tree + 1 nodes: per request
    a random node of a random merged tree, the path being its ancestors below
    the root and itself, by depth.  Returns (path_len[B], path_nodes[B, N])."""
    N = 2 * n_per_tree + 1
    plen = np.zeros(B, np.int32)
    nodes = np.full((B, N), -1, np.int32)
    for b in range(B):
        p1 = grow_tree(rng, n_per_tree)
        p2 = grow_tree(rng, n_per_tree)
        zeros = np.zeros(n_per_tree + 1, np.int32)
        par, _, _ = merge_two_trees(p1, zeros, p2, zeros)
        node = int(rng.integers(N))
        chain = []
        while node > 0:
            chain.append(node)
            node = int(par[node])
        chain.reverse()
        plen[b] = len(chain)
        nodes[b, :len(chain)] = chain
    return plen, nodes


def kv_commit_workload(seed: int = 0, L: int = 32, B: int = 32, H: int = 8, S: int = 256,
                       D: int = 128, n_per_tree: int = 31, tree: bool = True,
                       mirror: bool = True, name: str = "kv") -> KVWorkload:
    """Cache of a Llama-3-8B-shaped target (32 layers, 8 KV heads of 128)
    in bf16 bits; a cycle of N = 2 n_per_tree + 1 slots (tree) or N slots of
    a linear draft with n_per_tree accepted at most."""
    ss = np.random.SeedSequence([20261202 + 50, seed])
    r_kv, r_len, r_tree = [np.random.default_rng(x) for x in ss.spawn(3)]
    N = 2 * n_per_tree + 1
    kv = r_kv.integers(0, 1 << 16, size=(L, 2, B, H, S, D), dtype=np.uint16)
    cache_len = r_len.integers(0, S - N + 1, size=B).astype(np.int32)
    if tree:
        path_len, path_nodes = random_paths(r_tree, B, n_per_tree)
    else:
        path_len = r_tree.integers(0, N, size=B).astype(np.int32)
        path_nodes = None
    mir = r_kv.integers(0, 1 << 16, size=kv.shape, dtype=np.uint16) if mirror else None
    return KVWorkload(name, kv, cache_len, path_len, path_nodes, N, mir)


# --------------------------------------------------------------------------
# hidden states and a vocabulary matrix for the fused LM-head front end
# --------------------------------------------------------------------------

LMHEAD_CFG = 7  # seed-sequence slot of the LM-head workload


@dataclasses.dataclass
class LMHeadWorkload:
    name: str
    hidden: np.ndarray        # [B, K+1, d] uint16 (bf16 bits)
    weight: np.ndarray        # [V, d] uint16 (bf16 bits)
    tokens: np.ndarray        # [B, K] int32 draft tokens
    intended: np.ndarray      # [B, K+1] int32: the token each row was built to favour

    @property
    def B(self) -> int:
        return self.hidden.shape[0]

    @property
    def K(self) -> int:
        return self.hidden.shape[1] - 1

    @property
    def d(self) -> int:
        return self.hidden.shape[2]

    @property
    def V(self) -> int:
        return self.weight.shape[0]


def lmhead_workload(seed: int = 0, B: int = 64, K: int = 5, d: int = 4096, V: int = 128256,
                    integer: bool = False, signal: float = 0.75, agree: float = 0.7,
                    name: str = "lmhead") -> LMHeadWorkload:
    """Final hidden states and an LM-head matrix (Llama-3-8B-sized by
    default: d = 4096, V = 128256, bf16) for B requests of K drafts.

    Real-valued: W ~ N(0, 1/d); each row of H is N(0, 1) noise, plus, with
    probability `signal`, 0.5 sqrt(d) times the weight row of a uniformly
    drawn intended token (which then stands far above the rest); rows without
    it have Gaussian logits with close runners-up.  Integer-valued
    (`integer`): W in [-3, 3], noise in [-3, 3] plus twice the intended
    token's row, so that every logit is an integer below 2^24 and any fp32
    evaluation is exact.  Draft tokens: the intended token of the position
    with probability `agree`, else a uniform id (the stand-in drafter)."""
    r = rngs(LMHEAD_CFG, seed)
    g_w, g_h, g_t = r["logits"], r["noise"], r["tokens"]
    intended = g_t.integers(0, V, size=(B, K + 1)).astype(np.int32)
    has = g_t.random((B, K + 1)) < signal
    if integer:
        w32 = g_w.integers(-3, 4, size=(V, d)).astype(np.float32)
        h32 = g_h.integers(-3, 4, size=(B, K + 1, d)).astype(np.float32)
        h32 += np.where(has[..., None], 2.0 * w32[intended], 0.0).astype(np.float32)
        weight = f32_to_bf16_bits(w32)
    else:
        w32 = g_w.standard_normal((V, d), dtype=np.float32)
        w32 *= np.float32(1.0 / np.sqrt(d))
        weight = f32_to_bf16_bits(w32)
        del w32
        h32 = g_h.standard_normal((B, K + 1, d), dtype=np.float32)
        h32 += np.where(has[..., None], np.float32(0.5 * np.sqrt(d)) * bf16_bits_to_f32(weight[intended]),
                        np.float32(0.0)).astype(np.float32)
    hidden = f32_to_bf16_bits(h32)
    agree_mask = g_t.random((B, K)) < agree
    uniform = g_t.integers(0, V, size=(B, K)).astype(np.int32)
    tokens = np.where(agree_mask, intended[:, :K], uniform).astype(np.int32)
    return LMHeadWorkload(name, hidden, weight, tokens, intended)
