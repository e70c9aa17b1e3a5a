"""The GPU parity checker (tests/parity.py, check_sample) on made-up GPU
outputs, on the CPU: it must accept the oracle's outcome and, where a nucleus
edge lies within 1e-6 of top_p, the oracle's alternative, and reject anything
else.  Mistakes are planted in the outputs handed to the checker, never in a
kernel."""
import numpy as np
import pytest
from scipy import special

import oracle
import workloads as W
from parity import check_sample, flag_counts

torch = pytest.importorskip("torch")

RAMP = np.array([3.0, 2.0, 1.0, 0.0], np.float32)
CUM = np.cumsum(special.softmax(RAMP.astype(np.float64)))


def edge_workload():
    """Two requests of K = 1, V = 4: request 0 has its bonus row's nucleus
    edge within 1e-6 of top_p (the alternative draws token 2, the defined
    nucleus token 1); request 1 is the same rows with the ramp far from the
    edge (a steeper ramp)."""
    target = np.zeros((2, 2, 4), np.float32)
    target[0, 1] = RAMP
    target[1, 1] = 3 * RAMP
    draft = np.zeros((2, 1, 4), np.float32)
    return W.Workload("sample", "edge", 2, 1, 4, "f32", target, draft,
                      np.zeros((2, 1), np.int32), np.zeros((2, 1), np.float32),
                      np.full(2, 0.999, np.float32), 1.0, float(CUM[1] - 0.5e-6))


def fake(ref, n=None, tok=None, p=None, q=None, S=None):
    acc = ref["accepted"].copy() if n is None else np.asarray(n, np.int32)
    tokens = ref["tokens"].copy() if tok is None else np.asarray(tok, np.int32)
    return dict(accepted=torch.from_numpy(acc), tokens=torch.from_numpy(tokens),
                p=torch.from_numpy((ref["p"] if p is None else np.asarray(p)).astype(np.float32)),
                q=torch.from_numpy((ref["q"] if q is None else np.asarray(q)).astype(np.float32)),
                residual_mass=torch.from_numpy(
                    (ref["S"] if S is None else np.asarray(S)).astype(np.float32)))


def test_checker_accepts_the_defined_and_the_alternative_outcome():
    w = edge_workload()
    ref = oracle.verify_workload(w)
    assert ref["flags"][0] & oracle.FLAG_TOPP_NEAR and not ref["flags"][1]
    assert ref["tokens"][0].tolist() == [0, 1] and ref["alt_token"][0, 1, 1] == 2
    counts = check_sample(w, fake(ref), ref)
    assert counts == flag_counts(ref["flags"]) and counts["topp_near"] == 1
    assert counts["excluded"] == 0
    alt_tokens = ref["tokens"].copy()
    alt_tokens[0, 1] = 2
    S = ref["S"].copy()
    S[0] = ref["alt_S"][0, 1, 1]
    check_sample(w, fake(ref, tok=alt_tokens, S=S), ref)


@pytest.mark.parametrize("req", [0, 1])
def test_checker_rejects_a_token_no_variant_draws(req):
    w = edge_workload()
    ref = oracle.verify_workload(w)
    bad = ref["tokens"].copy()
    bad[req, 1] = 3
    with pytest.raises(AssertionError):
        check_sample(w, fake(ref, tok=bad), ref)


def test_checker_rejects_the_alternative_where_no_edge_is_near():
    # request 1's alternative would be token 2 too, but its edge is far away
    w = edge_workload()
    ref = oracle.verify_workload(w)
    bad = ref["tokens"].copy()
    bad[1, 1] = 2 if ref["tokens"][1, 1] != 2 else 1
    with pytest.raises(AssertionError):
        check_sample(w, fake(ref, tok=bad), ref)


@pytest.mark.parametrize("field", ["p", "q", "S"])
def test_checker_rejects_probabilities_off_by_2e5(field):
    w = edge_workload()
    ref = oracle.verify_workload(w)
    off = {field: (ref["S"] if field == "S" else ref[field]) + 2e-5}
    with pytest.raises(AssertionError):
        check_sample(w, fake(ref, **off), ref)


def test_checker_skips_only_flagged_uniforms():
    """A uniform 0.5e-6 relative from its accept threshold: the request is
    counted as excluded and a flipped decision passes; at 2e-6 it does not."""
    tgt = np.zeros((1, 2, 4), np.float32)
    dft = np.array([[[0.0, 0.0, 0.0, -np.inf]]], np.float32)  # ratio 3/4
    for rel, excluded in ((0.5e-6, True), (2e-6, False)):
        w = W.Workload("sample", "near", 1, 1, 4, "f32", tgt, dft, np.zeros((1, 1), np.int32),
                       np.array([[0.75 * (1 + rel)]], np.float32), np.array([0.3], np.float32),
                       1.0, 1.0)
        ref = oracle.verify_workload(w)
        assert ref["accepted"][0] == 0
        flipped = np.array([[0, 1]], np.int32)  # accepted, then the bonus draw's token 1
        got = fake(ref, n=[1], tok=flipped, S=[1.0])
        if excluded:
            assert check_sample(w, got, ref)["excluded"] == 1
        else:
            with pytest.raises(AssertionError):
                check_sample(w, got, ref)
