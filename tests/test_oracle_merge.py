"""Pins of the tree-merge / confidence-routing oracle (oracle.c,
oracle_tree_merge): TAPS on aitrends.kr, section "코드 예제" (the merged
tree's block layout) and "방법론" (merged-tree verification; routing to the
tree with the higher mean confidence)."""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_block_layout():
    g = json.load(open(os.path.join(GOLDEN, "merged_mask_layout.json")))
    p1 = np.array([g["tree1_parents"]], np.int32)
    p2 = np.array([g["tree2_parents"]], np.int32)
    t1 = np.arange(p1.shape[1], dtype=np.int32)[None]
    t2 = 100 + np.arange(p2.shape[1], dtype=np.int32)[None]
    o = oracle.tree_merge(p1, t1, np.zeros(p1.shape, np.float32), p2, t2,
                          np.zeros(p2.shape, np.float32))
    np.testing.assert_array_equal(o["parents"][0], g["merged_parents"])
    np.testing.assert_array_equal(o["mask"][0], np.array(g["merged_mask"], np.uint8))
    assert o["tokens"][0].tolist() == [0, 1, 2, 3, 101, 102]


def test_route_by_mean_confidence():
    p1 = np.array([[-1, 0, 0, 1]], np.int32)
    p2 = np.array([[-1, 0, 1]], np.int32)
    t1 = np.array([[5, 6, 7, 8]], np.int32)
    t2 = np.array([[9, 10, 11]], np.int32)
    o = oracle.tree_merge(p1, t1, [[0.0, 0.5, 0.25, 0.75]], p2, t2, [[0.0, 0.875, 0.625]])
    assert o["conf"][0].tolist() == [0.5, 0.75] and o["route"][0] == 1
    o = oracle.tree_merge(p1, t1, [[0.9, 0.5, 0.5, 0.5]], p2, t2, [[0.0, 0.5, 0.5]])
    assert o["route"][0] == 0  # equal means: the first tree
    e = np.array([[-1]], np.int32)
    o = oracle.tree_merge(e, [[3]], [[0.0]], p2, t2, [[0.0, 0.25, 0.25]])
    assert o["conf"][0].tolist() == [0.0, 0.25] and o["route"][0] == 1
    assert o["parents"][0].tolist() == [-1, 0, 1]


def test_invalid_trees_are_marked():
    p2 = np.array([[-1, 0, 1]], np.int32)
    for bad in ([0, 0, 0, 1], [-1, 0, 2, 1], [-1, 0, 0, 3]):
        o = oracle.tree_merge(np.array([bad], np.int32), [[1, 2, 3, 4]], [[0, .1, .1, .1]],
                              p2, [[5, 6, 7]], [[0, .2, .2]])
        assert o["route"][0] == -1 and (o["parents"][0] == -1).all() and o["mask"].sum() == 0


def test_random_trees_match_the_generator_layout_and_are_valid():
    rng = np.random.default_rng(8)
    B, n = 6, 31
    p1 = np.stack([W.grow_tree(rng, n) for _ in range(B)])
    p2 = np.stack([W.grow_tree(rng, n) for _ in range(B)])
    t1 = rng.integers(0, 1000, (B, n + 1)).astype(np.int32)
    t2 = rng.integers(0, 1000, (B, n + 1)).astype(np.int32)
    c1 = rng.random((B, n + 1)).astype(np.float32)
    c2 = rng.random((B, n + 1)).astype(np.float32)
    o = oracle.tree_merge(p1, t1, c1, p2, t2, c2)
    for b in range(B):
        par, tok, mask = W.merge_two_trees(p1[b], t1[b], p2[b], t2[b])
        np.testing.assert_array_equal(o["parents"][b], par)
        np.testing.assert_array_equal(o["tokens"][b], tok)
        np.testing.assert_array_equal(o["mask"][b], mask)
        # the block structure, as properties: the root sees only itself;
        # each tree's rows keep that tree's own ancestor sets (the root
        # standing for both roots) and see nothing of the other tree
        m = o["mask"][b]
        m1, m2 = W.ancestor_mask(p1[b]), W.ancestor_mask(p2[b])
        assert m[0].tolist() == [1] + [0] * (2 * n)
        np.testing.assert_array_equal(m[1:n + 1, :n + 1], m1[1:])
        assert not m[1:n + 1, n + 1:].any() and not m[n + 1:, 1:n + 1].any()
        np.testing.assert_array_equal(m[n + 1:, 0], m2[1:, 0])
        np.testing.assert_array_equal(m[n + 1:, n + 1:], m2[1:, 1:])
        assert oracle.tree_is_valid(o["parents"][b], o["mask"][b])
        m1, m2 = c1[b, 1:].astype(np.float64).mean(), c2[b, 1:].astype(np.float64).mean()
        assert abs(o["conf"][b, 0] - m1) < 1e-15 and abs(o["conf"][b, 1] - m2) < 1e-15
        assert o["route"][b] == (1 if o["conf"][b, 1] > o["conf"][b, 0] else 0)
