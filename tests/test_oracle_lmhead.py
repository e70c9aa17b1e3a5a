"""Pins of the fused LM-head oracle (oracle.c, oracle_lmhead_logits and
oracle_lmhead_greedy): the logits are the product of the target's final
hidden states with the vocabulary matrix (lotook.com explainer, the four
steps: one target pass gives the K+1 distributions), and greedy
verification takes the top choice of each (lotook.com FAQ)."""
import numpy as np

import oracle
import workloads as W


def bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_hand_case():
    h = bits([[1.0, 2.0]])
    w = bits([[1.0, 0.0], [0.5, 1.0], [-1.0, 3.0]])
    logits, ad = oracle.lmhead_logits(h, w, absdot=True)
    assert logits.tolist() == [[1.0, 2.5, 5.0]]
    assert ad.tolist() == [[1.0, 2.5, 7.0]]


def test_integer_logits_equal_integer_matmul():
    wl = W.lmhead_workload(seed=3, B=2, K=3, d=48, V=257, integer=True)
    h = wl.hidden.reshape(-1, wl.d)
    got = oracle.lmhead_logits(h, wl.weight)
    hi = W.bf16_bits_to_f32(h).astype(np.int64)
    wi = W.bf16_bits_to_f32(wl.weight).astype(np.int64)
    ref = hi @ wi.T
    assert (W.bf16_bits_to_f32(h) == hi).all() and (W.bf16_bits_to_f32(wl.weight) == wi).all()
    np.testing.assert_array_equal(got, ref.astype(np.float64))
    assert np.abs(ref).max() < 2 ** 24


def test_real_logits_match_float64_matmul():
    wl = W.lmhead_workload(seed=4, B=2, K=2, d=96, V=300)
    h = wl.hidden.reshape(-1, wl.d)
    got, ad = oracle.lmhead_logits(h, wl.weight, absdot=True)
    ref = W.bf16_bits_to_f32(h).astype(np.float64) @ W.bf16_bits_to_f32(wl.weight).astype(np.float64).T
    assert (np.abs(got - ref) <= 1e-13 * ad).all()
    assert (ad >= np.abs(got)).all()


def test_greedy_equals_plain_greedy_on_exact_logits():
    # integer-valued inputs: the logits are exact in fp32, so the fused
    # verification must equal greedy verification of the materialised logits
    wl = W.lmhead_workload(seed=5, B=6, K=4, d=64, V=700, integer=True, agree=0.8)
    logits = oracle.lmhead_logits(wl.hidden.reshape(-1, wl.d), wl.weight)
    lf32 = logits.astype(np.float32).reshape(wl.B, wl.K + 1, wl.V)
    assert (lf32.astype(np.float64) == logits.reshape(lf32.shape)).all()
    plain = oracle.verify_greedy(lf32, wl.tokens)
    fused = oracle.lmhead_greedy(wl.hidden, wl.weight, wl.tokens)
    for k in ("accepted", "tokens", "argmax"):
        np.testing.assert_array_equal(fused[k], plain[k])
    np.testing.assert_array_equal(fused["argmax"], np.argmax(lf32, axis=2))


def test_ties_take_the_lowest_id():
    wl = W.lmhead_workload(seed=6, B=1, K=1, d=32, V=50, integer=True)
    w = wl.weight.copy()
    h = wl.hidden.copy()
    top = int(np.argmax(oracle.lmhead_logits(h[0, :1], w)[0]))
    w[49] = w[top]            # a later duplicate of the top row: still `top`
    out = oracle.lmhead_greedy(h, w, np.array([[top]], np.int32))
    assert out["argmax"][0, 0] == top and out["accepted"][0] == 1
    if top > 0:
        w2 = w.copy()
        w2[0] = w[top]        # an earlier duplicate wins
        out2 = oracle.lmhead_greedy(h, w2, np.array([[top]], np.int32))
        assert out2["argmax"][0, 0] == 0 and out2["accepted"][0] == 0
        assert out2["tokens"][0].tolist() == [0, -1]


def test_signal_rows_pick_the_intended_token():
    wl = W.lmhead_workload(seed=7, B=4, K=3, d=128, V=2000, signal=1.0)
    out = oracle.lmhead_greedy(wl.hidden, wl.weight, wl.tokens)
    np.testing.assert_array_equal(out["argmax"], wl.intended)
