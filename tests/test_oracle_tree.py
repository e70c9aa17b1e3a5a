"""Pins of the oracle's merged-tree verification (TAPS, aitrends.kr:
section "방법론", merged-tree verification, and section "코드 예제", the merged
mask layout)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_tree(target_f32, parents, tokens):
    """Independent of masks: walk each node's parent chain explicitly; a node
    is accepted when every node on the chain (root excluded) equals numpy's
    first-occurrence argmax of its parent's row.  Deepest accepted node, lowest
    index on ties; path ordered root-side first."""
    N = len(parents)
    top = np.argmax(target_f32, axis=-1)
    best, best_depth = 0, 0
    for i in range(N):
        chain = []
        j = i
        while j > 0:
            chain.append(j)
            j = int(parents[j])
        ok = all(tokens[c] == top[parents[c]] for c in chain)
        if ok and len(chain) > best_depth:
            best, best_depth = i, len(chain)
    path = []
    j = best
    while j > 0:
        path.append(j)
        j = int(parents[j])
    path = path[::-1]
    return best_depth, path, [int(tokens[p]) for p in path] + [int(top[best])]


@pytest.mark.parametrize("seed", range(6))
def test_tree_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    B, V = 40, 6
    for dtype in ("f32", "bf16"):
        for b in range(B):
            n_nodes = int(rng.integers(1, 9))  # <= 8 nodes
            parents = W.grow_tree(rng, n_nodes - 1, max_depth=5, max_children=3)
            mask = W.ancestor_mask(parents)
            t32 = rng.normal(0, 1, (1, n_nodes, V)).astype(np.float32)
            t = W.f32_to_bf16_bits(t32) if dtype == "bf16" else t32
            tf = W.logits_as_f32(t, dtype)
            top = np.argmax(tf[0], axis=-1)
            toks = np.empty(n_nodes, np.int32)
            toks[0] = rng.integers(0, V)
            for i in range(1, n_nodes):
                toks[i] = top[parents[i]] if rng.random() < 0.7 else rng.integers(0, V)
            out = oracle.verify_tree(t, parents[None], toks[None], mask[None])
            d, path, emitted = brute_force_tree(tf[0], parents, toks)
            assert out["valid"][0] == 1
            assert out["path_len"][0] == d
            assert list(out["path_nodes"][0, :d]) == path
            assert (out["path_nodes"][0, d:] == -1).all()
            assert list(out["tokens"][0, :d + 1]) == emitted
            assert (out["tokens"][0, d + 1:] == -1).all()


def test_chain_tree_equals_linear_greedy():
    w = W.make_config(1, B=16, V=300)
    K = w.K
    g = oracle.verify_greedy(w.target, w.tokens)
    N = K + 1
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (w.B, 1))
    node_tokens = np.concatenate([np.zeros((w.B, 1), np.int32), w.tokens], axis=1)
    mask = np.tile(np.tril(np.ones((N, N), np.uint8)), (w.B, 1, 1))
    t = oracle.verify_tree(w.target, parents, node_tokens, mask)
    np.testing.assert_array_equal(t["path_len"], g["accepted"])
    np.testing.assert_array_equal(t["tokens"], g["tokens"])


def test_merged_mask_layout_golden():
    g = json.load(open(os.path.join(GOLDEN, "merged_mask_layout.json")))
    p1 = np.array(g["tree1_parents"], np.int32)
    p2 = np.array(g["tree2_parents"], np.int32)
    par, tok, mask = W.merge_two_trees(p1, np.arange(len(p1)), p2, 100 + np.arange(len(p2)))
    np.testing.assert_array_equal(mask, np.array(g["merged_mask"], np.uint8))
    np.testing.assert_array_equal(par, np.array(g["merged_parents"], np.int32))
    assert list(tok) == [0, 1, 2, 3, 101, 102]
    assert oracle.tree_is_valid(par, mask)


def test_merged_masks_are_ancestor_closures_and_corruption_is_caught():
    w = W.make_config(4, B=4, V=64)
    rng = np.random.default_rng(0)
    for b in range(w.B):
        assert oracle.tree_is_valid(w.parents[b], w.anc_mask[b])
        bad = w.anc_mask[b].copy()
        i = int(rng.integers(1, w.K))
        j = int(rng.integers(0, w.K))
        bad[i, j] ^= 1
        assert not oracle.tree_is_valid(w.parents[b], bad)
    out = oracle.verify_workload(w)
    assert (out["valid"] == 1).all()


def test_tree_workload_shape():
    w = W.make_config(4, B=3, V=32)
    assert w.K == 63 and w.parents.shape == (3, 63) and w.anc_mask.shape == (3, 63, 63)
    depth = w.anc_mask.sum(-1) - 1
    assert depth.max() <= 8
    for b in range(3):
        counts = np.bincount(w.parents[b, 1:], minlength=63)
        # root has children from both trees (<= 4 each); others <= 4
        assert counts[1:].max() <= 4 and counts[0] <= 8
        assert (w.parents[b, 1:] < np.arange(1, 63)).all()
