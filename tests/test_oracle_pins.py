"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: the pages' worked
example and narrative (tests/golden/), the losslessness invariant, closed-form
acceptance laws, textbook routines (scipy softmax, numpy argmax, inverse CDF by
searchsorted) and special cases that reduce to them.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def grid(G):
    """Midpoints (k + 0.5) / G: on the 2**-24 grid for G <= 2**23, never on a
    rational threshold with small denominator."""
    return ((np.arange(G) + 0.5) / G).astype(np.float32)


def tempered_nucleus(logits, T, top_p):
    """Test-side target law: scipy softmax at temperature T, then the nucleus
    (largest logits, tie groups whole, first reaching top_p), renormalised."""
    l = np.asarray(logits, np.float64)
    p = special.softmax(l / T)
    if top_p >= 1.0:
        return p
    vals = np.unique(l)[::-1]
    cum = 0.0
    for v in vals:
        cum += p[l == v].sum()
        if cum >= top_p:
            keep = l >= v
            break
    out = np.where(keep, p, 0.0)
    return out / out.sum()


def run_sample(target, draft, tokens, ua, us, T, top_p=1.0):
    return oracle.verify_sample(np.asarray(target, np.float32), np.asarray(draft, np.float32),
                                tokens, ua, us, T, top_p)


# ---------------------------------------------------------------------------
# ariser.io worked example: p = [0.6, 0.4], q = [0.8, 0.2]
# ---------------------------------------------------------------------------

def test_worked_example_probabilities():
    g = golden("worked_example.json")
    p = np.array(g["p_target"])
    q = np.array(g["q_draft"])
    pt, info_p = oracle.row_distribution(np.log(p).astype(np.float64).astype(np.float32), 1.0)
    # float32 logits of ln p reproduce p to ~1e-7; use fp64-exact target below
    np.testing.assert_allclose(pt, p, atol=1e-7)


def _worked_example_batch(x, ua, us):
    """K = 1, V = 2; row 1 of the target (bonus) is the same p."""
    g = golden("worked_example.json")
    lp = np.log(np.array(g["p_target"])).astype(np.float32)
    lq = np.log(np.array(g["q_draft"])).astype(np.float32)
    n = len(ua)
    target = np.broadcast_to(np.stack([lp, lp]), (n, 2, 2)).copy()
    draft = np.broadcast_to(lq[None, None, :], (n, 1, 2)).copy()
    tokens = np.full((n, 1), x, np.int32)
    return run_sample(target, draft, tokens, np.asarray(ua, np.float32).reshape(n, 1),
                      np.asarray(us, np.float32), 1.0)


def test_worked_example_accept_and_residual():
    g = golden("worked_example.json")
    G = 4096
    u = grid(G)
    # the float32 logits give p, q within ~1e-7 of the page's numbers; the
    # midpoint grid keeps every u at least 1/(2G) away from 0.75
    outA = _worked_example_batch(0, u, np.full(G, 0.5, np.float32))
    outB = _worked_example_batch(1, u, np.full(G, 0.5, np.float32))
    accA = (outA["accepted"] == 1).mean()
    accB = (outB["accepted"] == 1).mean()
    assert accA == pytest.approx(g["accept_probability"]["A"], abs=0)
    assert accB == pytest.approx(g["accept_probability"]["B"], abs=0)
    qA, qB = g["q_draft"]
    assert qA * accA == pytest.approx(g["immediate_accept_mass"]["A"], abs=1e-12)
    assert qB * accB == pytest.approx(g["immediate_accept_mass"]["B"], abs=1e-12)
    assert qA * (1 - accA) + qB * (1 - accB) == pytest.approx(g["rejection_mass"], abs=1e-12)
    # every rejection of A resamples from normalize(max(0, p - q)) = [0, 1]
    rej = outA["accepted"] == 0
    assert rej.sum() == G // 4
    np.testing.assert_allclose(outA["S"][rej], sum(g["residual_unnormalised"]), atol=1e-7)
    sweep = _worked_example_batch(0, np.full(G, 0.999, np.float32), u)
    assert (sweep["accepted"] == 0).all()
    assert (sweep["tokens"][:, 0] == 1).all(), "residual must be [0, 1] -> always B"
    np.testing.assert_allclose(sweep["p"][:, 0], g["p_target"][0], atol=1e-7)
    np.testing.assert_allclose(sweep["q"][:, 0], g["q_draft"][0], atol=1e-7)


def test_worked_example_final_law_by_quadrature():
    """Law of the emitted first token, integrating x ~ q and both uniforms on
    grids: exactly the target's [0.6, 0.4] (up to the grid resolution)."""
    g = golden("worked_example.json")
    G = 1024
    u = grid(G)
    ua = np.repeat(u, G)
    us = np.tile(u, G)
    law = np.zeros(2)
    for x, qx in enumerate(g["q_draft"]):
        out = _worked_example_batch(x, ua, us)
        first = out["tokens"][:, 0]
        law += qx * np.bincount(first, minlength=2) / len(first)
    np.testing.assert_allclose(law, g["final_law"], atol=2.0 / G)


# ---------------------------------------------------------------------------
# losslessness: Monte-Carlo, 10**6 trials, chi-square per emitted slot
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,K,T,top_p", [(8, 3, 0.7, 1.0), (16, 2, 1.3, 0.8), (5, 3, 1.0, 0.9)])
def test_losslessness_chi_square(V, K, T, top_p):
    rng = np.random.default_rng(1000 + V + K)
    tl = (rng.normal(0, 1.5, (K + 1, V))).astype(np.float32)
    dl = (tl[:K] + rng.normal(0, 1.0, (K, V))).astype(np.float32)
    Tf = float(np.float32(T))
    P = np.stack([tempered_nucleus(tl[i], Tf, top_p) for i in range(K + 1)])
    Qd = np.stack([tempered_nucleus(dl[i], Tf, top_p) for i in range(K)])
    trials = 1_000_000
    tokens = np.stack([rng.choice(V, size=trials, p=Qd[i]) for i in range(K)], axis=1).astype(np.int32)
    ua = (rng.integers(0, 1 << 24, (trials, K)) * 2.0 ** -24).astype(np.float32)
    us = (rng.integers(0, 1 << 24, trials) * 2.0 ** -24).astype(np.float32)
    target = np.broadcast_to(tl, (trials, K + 1, V))
    draft = np.broadcast_to(dl, (trials, K, V))
    out = run_sample(target, draft, tokens, ua, us, Tf, top_p)
    n = out["accepted"]
    for i in range(K + 1):
        sel = n >= i
        counts = np.bincount(out["tokens"][sel, i], minlength=V)
        expected = P[i] * sel.sum()
        support = expected > 0
        assert counts[~support].sum() == 0, "emitted a token outside the target's support"
        chi = stats.chisquare(counts[support], expected[support])
        assert chi.pvalue > 1e-4, (i, chi)
    # the law of the accepted length: P(n = i) = prod_{k<i} beta_k (1 - beta_i)
    beta = np.minimum(P[:K], Qd).sum(axis=1)
    law = np.array([np.prod(beta[:i]) * (1 - beta[i]) for i in range(K)] + [np.prod(beta)])
    chi = stats.chisquare(np.bincount(n, minlength=K + 1), law * trials)
    assert chi.pvalue > 1e-4, chi


# ---------------------------------------------------------------------------
# brute force (K <= 3, V <= 4): exact acceptance / residual laws via u-grids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,K,T,top_p,seed", [(3, 2, 1.0, 1.0, 0), (4, 3, 0.7, 1.0, 1),
                                             (4, 3, 1.0, 0.85, 2), (2, 1, 2.0, 1.0, 3)])
def test_brute_force_acceptance_law(V, K, T, top_p, seed):
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.2, (K + 1, V)).astype(np.float32)
    dl = (tl[:K] + rng.normal(0, 1.0, (K, V))).astype(np.float32)
    Tf = float(np.float32(T))
    P = np.stack([tempered_nucleus(tl[i], Tf, top_p) for i in range(K + 1)])
    Qd = np.stack([tempered_nucleus(dl[i], Tf, top_p) for i in range(K)])
    G = 8192
    u = grid(G)
    # measured per-position accept probability of the oracle for every (i, x)
    acc = np.zeros((K, V))
    resid_law = np.zeros((K, V))
    for i in range(K):
        for x in range(V):
            tokens = np.zeros((G, K), np.int32)
            for k in range(K):
                tokens[:, k] = int(np.argmax(P[k]))  # earlier positions: p > 0, u = 0 -> accept
            tokens[:, i] = x
            ua = np.zeros((G, K), np.float32)
            ua[:, i] = u
            out = run_sample(np.broadcast_to(tl, (G, K + 1, V)), np.broadcast_to(dl, (G, K, V)),
                             tokens, ua, np.full(G, 0.5, np.float32), Tf, top_p)
            assert (out["accepted"] >= i).all()
            acc[i, x] = (out["accepted"] > i).mean()
            if Qd[i, x] > 0:
                expect = min(1.0, P[i, x] / Qd[i, x])
                assert abs(acc[i, x] - expect) <= 1.0 / G, (i, x, acc[i, x], expect)
        # residual law at a rejection at i: sweep u_sample, force a rejecting x
        xs = [x for x in range(V) if Qd[i, x] > P[i, x]]
        if not xs:
            continue
        x = xs[0]
        tokens = np.tile(np.array([int(np.argmax(P[k])) for k in range(K)], np.int32), (G, 1))
        tokens[:, i] = x
        ua = np.zeros((G, K), np.float32)
        ua[:, i] = np.float32(1.0 - 2.0 ** -24)
        out = run_sample(np.broadcast_to(tl, (G, K + 1, V)), np.broadcast_to(dl, (G, K, V)),
                         tokens, ua, u, Tf, top_p)
        assert (out["accepted"] == i).all()
        resid_law[i] = np.bincount(out["tokens"][:, i], minlength=V) / G
        r = np.maximum(P[i] - Qd[i], 0.0)
        np.testing.assert_allclose(resid_law[i], r / r.sum(), atol=1.5 / G)
    # enumerate every draft sequence: law of n from the measured accept
    # probabilities against the closed form prod beta
    law = np.zeros(K + 1)
    for seq in np.ndindex(*([V] * K)):
        w = np.prod([Qd[k, seq[k]] for k in range(K)])
        alive = 1.0
        for k in range(K):
            a = acc[k, seq[k]]
            law[k] += w * alive * (1 - a)
            alive *= a
        law[K] += w * alive
    beta = np.minimum(P[:K], Qd).sum(axis=1)
    closed = np.array([np.prod(beta[:i]) * (1 - beta[i]) for i in range(K)] + [np.prod(beta)])
    np.testing.assert_allclose(law, closed, atol=K * 1.0 / G)


# ---------------------------------------------------------------------------
# textbook routines
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(7)
    l = rng.normal(0, 4, 1000).astype(np.float32)
    Tf = float(np.float32(T))
    prob, info = oracle.row_distribution(l, Tf)
    ref = special.softmax(l.astype(np.float64) / Tf)
    np.testing.assert_allclose(prob, ref, rtol=1e-12, atol=1e-15)
    assert info["max"] == float(l.max())


def test_bf16_widening_and_argmax_match_numpy():
    import workloads as W
    rng = np.random.default_rng(3)
    B, K, V = 6, 3, 257
    t = W.f32_to_bf16_bits(rng.normal(0, 2.5, (B, K + 1, V)).astype(np.float32))
    # plant exact ties at the maximum in several rows
    tf = W.bf16_bits_to_f32(t)
    for b in range(B):
        i = b % (K + 1)
        j = int(np.argmax(tf[b, i]))
        t[b, i, (j + 17) % V] = t[b, i, j]
        t[b, i, (j + 101) % V] = t[b, i, j]
    tf = W.bf16_bits_to_f32(t)
    out = oracle.verify_greedy(t, np.zeros((B, K), np.int32))
    np.testing.assert_array_equal(out["argmax"], np.argmax(tf, axis=-1))
    # and the fp32 path
    out32 = oracle.verify_greedy(tf, np.zeros((B, K), np.int32))
    np.testing.assert_array_equal(out32["argmax"], np.argmax(tf, axis=-1))
    # the bf16 distribution equals the softmax of the exactly widened values
    prob, _ = oracle.row_distribution(t[0, 0], float(np.float32(0.9)))
    np.testing.assert_allclose(prob, special.softmax(tf[0, 0].astype(np.float64) / float(np.float32(0.9))),
                               rtol=1e-12, atol=1e-15)


def test_bonus_is_inverse_cdf_of_last_target_row():
    """p = q accepts every draft (u q < q for u < 1); the bonus then is the
    textbook inverse-CDF draw from p_K: searchsorted(cumsum(p), u, 'right')."""
    rng = np.random.default_rng(11)
    B, K, V = 2000, 3, 50
    tl = rng.normal(0, 2, (K + 1, V)).astype(np.float32)
    target = np.broadcast_to(tl, (B, K + 1, V))
    draft = np.broadcast_to(tl[:K], (B, K, V))
    T = float(np.float32(0.8))
    P = np.stack([special.softmax(tl[i].astype(np.float64) / T) for i in range(K + 1)])
    tokens = np.stack([rng.choice(V, size=B, p=P[i]) for i in range(K)], axis=1).astype(np.int32)
    ua = (rng.integers(0, 1 << 24, (B, K)) * 2.0 ** -24).astype(np.float32)
    us = (rng.integers(0, 1 << 24, B) * 2.0 ** -24).astype(np.float32)
    out = run_sample(target, draft, tokens, ua, us, T)
    assert (out["accepted"] == K).all()
    expect = np.searchsorted(np.cumsum(P[K]), us.astype(np.float64) * P[K].sum(), side="right")
    ok = (out["flags"] & oracle.FLAG_CDF_NEAR) == 0
    np.testing.assert_array_equal(out["tokens"][ok, K], expect[ok])
    np.testing.assert_array_equal(out["tokens"][:, :K], tokens)
    np.testing.assert_allclose(out["S"], 1.0, atol=1e-12)


# ---------------------------------------------------------------------------
# special cases
# ---------------------------------------------------------------------------

def test_one_hot_sampling_reduces_to_greedy():
    rng = np.random.default_rng(5)
    B, K, V = 200, 4, 12
    top_t = rng.integers(0, V, (B, K + 1))
    top_d = np.where(rng.random((B, K)) < 0.6, top_t[:, :K], rng.integers(0, V, (B, K)))
    target = np.full((B, K + 1, V), -1.0e4, np.float32)
    draft = np.full((B, K, V), -1.0e4, np.float32)
    np.put_along_axis(target, top_t[..., None], 0.0, axis=-1)
    np.put_along_axis(draft, top_d[..., None], 0.0, axis=-1)
    tokens = top_d.astype(np.int32)  # the one-hot draft always proposes its top token
    ua = (rng.integers(0, 1 << 24, (B, K)) * 2.0 ** -24).astype(np.float32)
    us = (rng.integers(0, 1 << 24, B) * 2.0 ** -24).astype(np.float32)
    s = run_sample(target, draft, tokens, ua, us, 1.0)
    g = oracle.verify_greedy(target, tokens)
    np.testing.assert_array_equal(s["accepted"], g["accepted"])
    np.testing.assert_array_equal(s["tokens"], g["tokens"])


def test_top_p_edges():
    rng = np.random.default_rng(9)
    l = rng.normal(0, 1, 64).astype(np.float32)
    full, _ = oracle.row_distribution(l, 0.9, 1.0)
    # a nucleus that must keep every token (smallest token mass >> 1e-9)
    keep_all, info = oracle.row_distribution(l, 0.9, 1.0 - 1e-9)
    assert (keep_all > 0).all()
    np.testing.assert_allclose(keep_all, full, rtol=1e-8)
    # top_p -> 0 keeps only the maximum's tie group
    l2 = l.copy()
    l2[10] = l2[20] = l.max() + 1.0
    tiny, info = oracle.row_distribution(l2, 0.9, 1e-9)
    expect = np.zeros(64)
    expect[[10, 20]] = 0.5
    np.testing.assert_allclose(tiny, expect, atol=1e-15)
    assert info["tau"] == float(l2[10])


def test_top_p_hand_case():
    """p = [0.5, 0.3, 0.15, 0.05]: top_p 0.7 keeps {0, 1} -> [5/8, 3/8];
    top_p 0.85 keeps {0, 1, 2} -> [0.5, 0.3, 0.15] / 0.95."""
    p = np.array([0.5, 0.3, 0.15, 0.05])
    l = np.log(p)  # as float32 logits below; p within 1e-7
    a, _ = oracle.row_distribution(l.astype(np.float32), 1.0, 0.7)
    np.testing.assert_allclose(a, [5 / 8, 3 / 8, 0, 0], atol=1e-7)
    b, _ = oracle.row_distribution(l.astype(np.float32), 1.0, 0.85)
    np.testing.assert_allclose(b, [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0], atol=1e-7)
    # a tie across the cut is kept whole: [0.4, 0.3, 0.3] at top_p 0.5 keeps all three
    c, _ = oracle.row_distribution(np.log(np.array([0.4, 0.3, 0.3])).astype(np.float32), 1.0, 0.5)
    assert (c > 0).all()


def test_replacement_never_equals_rejected_draft():
    import workloads as W
    for cfg, kw in ((0, dict(B=64, V=300)), (2, dict(B=32, V=500)), (3, dict(B=16, V=400))):
        w = W.make_config(cfg, **kw)
        out = oracle.verify_workload(w)
        n = out["accepted"]
        rej = (n < w.K) & ((out["flags"] & oracle.FLAG_FALLBACK) == 0)
        assert rej.any()
        assert (out["tokens"][rej, n[rej]] != w.tokens[rej, n[rej]]).all()
        assert ((out["tokens"] >= -1) & (out["tokens"] < w.V)).all()
        for b in range(w.B):
            np.testing.assert_array_equal(out["tokens"][b, :n[b]], w.tokens[b, :n[b]])
            assert (out["tokens"][b, n[b] + 1:] == -1).all()


def test_k1_and_out_of_range_token():
    rng = np.random.default_rng(2)
    V = 10
    tl = rng.normal(0, 1, (3, 2, V)).astype(np.float32)
    dl = rng.normal(0, 1, (3, 1, V)).astype(np.float32)
    tokens = np.array([[V], [-1], [3]], np.int32)
    ua = np.zeros((3, 1), np.float32)
    us = np.full(3, 0.25, np.float32)
    out = run_sample(tl, dl, tokens, ua, us, 1.0)
    assert out["accepted"][0] == 0 and out["accepted"][1] == 0
    assert out["flags"][0] & oracle.FLAG_TOKEN_RANGE and out["flags"][1] & oracle.FLAG_TOKEN_RANGE
    assert out["accepted"][2] == 1  # u = 0 accepts whenever p'(x) > 0
    assert out["tokens"][2, 0] == 3


def test_greedy_narrative():
    g = golden("greedy_narrative.json")
    vocab = {w: i for i, w in enumerate(g["vocab"])}
    V = len(vocab)
    tops = [vocab[w] for w in g["target_top_choice_per_position"]]
    K = len(g["draft"])
    target = np.zeros((1, K + 1, V), np.float32)
    for i, t in enumerate(tops):
        target[0, i, t] = 5.0
    tokens = np.array([[vocab[w] for w in g["draft"]]], np.int32)
    out = oracle.verify_greedy(target, tokens)
    assert out["accepted"][0] == g["expected_accepted"]
    emitted = [g["vocab"][t] for t in out["tokens"][0] if t >= 0]
    assert emitted == g["expected_emitted"]
    # same narrative as a chain tree: root = the last prefix token
    N = K + 1
    parents = np.arange(-1, N - 1, dtype=np.int32)[None]
    node_tokens = np.array([[vocab[g["prefix"][-1]]] + [vocab[w] for w in g["draft"]]], np.int32)
    mask = np.tril(np.ones((N, N), np.uint8))[None]
    tr = oracle.verify_tree(target, parents, node_tokens, mask)
    assert tr["path_len"][0] == g["expected_accepted"]
    assert [g["vocab"][t] for t in tr["tokens"][0] if t >= 0] == g["expected_emitted"]
