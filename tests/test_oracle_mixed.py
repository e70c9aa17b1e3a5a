"""Pins of the per-request oracle (oracle.verify_mixed): each request is
verified on its own with its own temperature and top-p; temperature 0 is the
greedy rule (lotook.com explainer, FAQ), any other value the sampling rule
(ariser.io review, section "같은 분포를 지키는 작은 장치")."""
import numpy as np

import oracle
import workloads as W


def test_equal_temperatures_reduce_to_the_batch_call():
    w = W.make_config(2, B=6, V=3001)
    ref = oracle.verify_sample(w.target, w.draft, w.tokens, w.u_accept, w.u_sample,
                               w.temperature, 0.9)
    got = oracle.verify_mixed(w.target, w.draft, w.tokens, w.u_accept, w.u_sample,
                              np.full(6, w.temperature, np.float32), np.full(6, 0.9, np.float32))
    for key in ("accepted", "tokens", "p", "q", "S", "flags"):
        np.testing.assert_array_equal(got[key], ref[key])


def test_zero_temperatures_reduce_to_greedy():
    w = W.make_config(2, B=5, V=2000)
    ref = oracle.verify_greedy(w.target, w.tokens)
    got = oracle.verify_mixed(w.target, w.draft, w.tokens, w.u_accept, w.u_sample,
                              np.zeros(5, np.float32))
    np.testing.assert_array_equal(got["accepted"], ref["accepted"])
    np.testing.assert_array_equal(got["tokens"], ref["tokens"])
    assert (got["S"] == 0).all() and (got["p"] == 0).all()


def test_each_request_uses_only_its_own_parameters():
    w = W.make_config(2, B=4, V=1500)
    temps = np.array([0.0, 0.7, 1.3, 0.7], np.float32)
    topps = np.array([1.0, 0.8, 1.0, 1.0], np.float32)
    got = oracle.verify_mixed(w.target, w.draft, w.tokens, w.u_accept, w.u_sample, temps, topps)
    for b in range(4):
        one = oracle.verify_mixed(w.target[b:b + 1], w.draft[b:b + 1], w.tokens[b:b + 1],
                                  w.u_accept[b:b + 1], w.u_sample[b:b + 1], temps[b:b + 1],
                                  topps[b:b + 1])
        assert got["accepted"][b] == one["accepted"][0]
        np.testing.assert_array_equal(got["tokens"][b], one["tokens"][0])


def test_out_of_range_parameters_are_marked():
    w = W.make_config(2, B=5, V=500)
    temps = np.array([-1.0, np.nan, np.inf, 0.7, 0.7], np.float32)
    topps = np.array([1.0, 1.0, 1.0, 0.0, 1.5], np.float32)
    got = oracle.verify_mixed(w.target, w.draft, w.tokens, w.u_accept, w.u_sample, temps, topps)
    assert (got["accepted"] == -3).all() and (got["tokens"] == -1).all()
