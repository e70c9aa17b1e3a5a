"""Pins of the KV-cache commit oracle (oracle.c, oracle_kv_commit).

The operation: after a cycle, the cache keeps the root and the accepted
path's entries in consecutive slots and drops the rest (lotook.com explainer,
section on the KV cache: rejected entries are cut from both caches; SubSpec
review, Method part 2, step 4: the drafter's temporary entries are
overwritten with the target's; TAPS on aitrends.kr, "방법론": the longest
accepted path of a merged tree)."""
import numpy as np
import pytest

import oracle
import workloads as W


def slot_coded_cache(L, B, H, S, D):
    """Every element encodes (l, kv, b, h, slot) so moves can be read back."""
    kv = np.zeros((L, 2, B, H, S, D), np.int32)
    l, k, b, h, s = np.meshgrid(np.arange(L), np.arange(2), np.arange(B), np.arange(H),
                                np.arange(S), indexing="ij")
    code = ((((l * 2 + k) * B + b) * H + h) * S + s)
    kv[...] = code[..., None] * 16 + np.arange(D)
    return kv


def test_hand_case_tree_path():
    # one row of slots 0..7 (coded by slot id), cycle at slot 1 with N = 5
    # slots (nodes 0..4), accepted path root, node 2, node 4
    kv = np.arange(8, dtype=np.int32).reshape(1, 1, 1, 1, 8, 1).repeat(2, axis=1)
    out, mir, new_len = oracle.kv_commit(kv, [1], [2], np.array([[2, 4, -1, -1, -1]], np.int32),
                                         mirror=np.full_like(kv, -7))
    assert out[0, 0, 0, 0, :, 0].tolist() == [0, 1, 3, 5, 4, 5, 6, 7]
    assert mir[0, 1, 0, 0, :, 0].tolist() == [-7, 1, 3, 5, -7, -7, -7, -7]
    assert new_len.tolist() == [4]


def test_linear_draft_keeps_the_cache_and_sets_the_length():
    kv = slot_coded_cache(2, 3, 2, 12, 3)
    out, mir, new_len = oracle.kv_commit(kv, [0, 4, 7], [0, 3, 4], None, N=5,
                                         mirror=np.zeros_like(kv))
    np.testing.assert_array_equal(out, kv)
    assert new_len.tolist() == [1, 8, 12]
    for b, (c, d) in enumerate([(0, 0), (4, 3), (7, 4)]):
        np.testing.assert_array_equal(mir[:, :, b, :, c:c + d + 1], kv[:, :, b, :, c:c + d + 1])
        assert (mir[:, :, b, :, :c] == 0).all() and (mir[:, :, b, :, c + d + 1:] == 0).all()


def test_chain_path_equals_linear():
    kv = slot_coded_cache(1, 2, 2, 10, 2)
    chain = np.array([[1, 2, 3, -1, -1], [1, -1, -1, -1, -1]], np.int32)
    a = oracle.kv_commit(kv, [2, 5], [3, 1], chain)
    b = oracle.kv_commit(kv, [2, 5], [3, 1], None, N=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[2], b[2])


def test_same_slot_move_in_every_layer_and_head_and_nothing_else():
    L, B, H, S, D = 2, 4, 3, 40, 2
    kv = slot_coded_cache(L, B, H, S, D)
    rng = np.random.default_rng(3)
    plen, nodes = W.random_paths(rng, B, 6)
    N = nodes.shape[1]
    cache_len = np.array([0, 5, 20, S - N], np.int32)
    out, _, new_len = oracle.kv_commit(kv, cache_len, plen, nodes)
    code = out[..., 0] // 16
    slot = code % S
    rest = code // S
    # no element moved across layers, K/V, requests or heads
    np.testing.assert_array_equal(rest, kv[..., 0] // 16 // S)
    for b in range(B):
        c, d = int(cache_len[b]), int(plen[b])
        want = np.arange(S)
        want[c] = c
        want[c + 1:c + 1 + d] = c + nodes[b, :d]
        assert (slot[:, :, b] == want).all()
        assert new_len[b] == c + 1 + d


@pytest.mark.parametrize("case", ["long", "overflow", "order", "range", "negative"])
def test_inconsistent_requests_are_left_alone(case):
    kv = slot_coded_cache(1, 2, 1, 12, 1)
    nodes = np.array([[1, 3, -1, -1, -1], [2, 4, -1, -1, -1]], np.int32)
    cache_len = np.array([0, 2], np.int32)
    plen = np.array([2, 2], np.int32)
    if case == "long":
        plen[1] = 5           # more than N - 1 path nodes
    elif case == "overflow":
        cache_len[1] = 8      # 8 + 5 > 12 slots
    elif case == "order":
        nodes[1] = [4, 2, -1, -1, -1]
    elif case == "range":
        nodes[1] = [2, 5, -1, -1, -1]
    else:
        plen[1] = -2          # a failed verify
    out, _, new_len = oracle.kv_commit(kv, cache_len, plen, nodes)
    assert new_len[1] == -1 and new_len[0] == 3
    np.testing.assert_array_equal(out[:, :, 1], kv[:, :, 1])


def test_commit_of_a_verified_tree_keeps_the_path_rows():
    w = W.make_config(4, B=3, V=300)
    res = oracle.verify_tree(w.target, w.parents, w.tokens, w.anc_mask)
    N = w.K
    kv = slot_coded_cache(1, 3, 1, N + 4, 1)
    cache_len = np.array([0, 2, 4], np.int32)
    out, _, new_len = oracle.kv_commit(kv, cache_len, res["path_len"], res["path_nodes"])
    for b in range(3):
        d = int(res["path_len"][b])
        got = out[0, 0, b, 0, cache_len[b]:cache_len[b] + d + 1, 0] // 16 % (N + 4)
        want = cache_len[b] + np.concatenate([[0], res["path_nodes"][b, :d]])
        np.testing.assert_array_equal(got, want)
        # every kept node is an ancestor of the next one (a root-to-node path)
        for j in range(1, d):
            assert w.anc_mask[b, res["path_nodes"][b, j], res["path_nodes"][b, j - 1]] == 1
