"""Pins of the oracle's ambiguity flags and of its nucleus alternatives.

A request leaves the exact GPU comparison only when the oracle flags it, so
the flags must fire where the rule says and nowhere else:
  - the accept test: a uniform within 1e-6 relative of p'(x)/q'(x);
  - the inverse CDF: u * S within 1e-6 relative of a CDF step;
  - top-p: a row whose cumulative mass before or after its cut group lies
    within 1e-6 of top_p; the oracle then verifies the request again with
    that row's cut moved by one tie group, and marks it only if the emitted
    outcome changes.
The inputs here have probabilities known exactly (equal logits give exact
quarters and thirds), so each uniform is placed at a known relative offset
from its threshold: 0.5e-6 must flag, 2e-6 must not.  The top-p cases take
cumulative masses from scipy's softmax (a textbook routine, not the oracle)
and check each alternative against the defined rule at a top_p that makes
the alternative membership the defined one.
(ariser.io review, section "같은 분포를 지키는 작은 장치": accept with
probability min(1, p/q), residual normalize(max(0, p - q)), temperature and
top-p applied to p and q.)
"""
import numpy as np
import pytest
from scipy import special

import oracle

NEG = -np.inf


def run(target, draft, tokens, ua, us, T=1.0, top_p=1.0):
    t = np.asarray(target, np.float32)
    d = np.asarray(draft, np.float32)
    return oracle.verify_sample(t[None], d[None], np.asarray([tokens], np.int32),
                                np.asarray([ua], np.float32), np.asarray([us], np.float32),
                                T, top_p)


def f32(x):
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# accept test: p'(0) = 1/4, q'(0) = 1/3, ratio 3/4
# ---------------------------------------------------------------------------

TGT_QUARTERS = [[0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]
DFT_THIRDS = [[0.0, 0.0, 0.0, NEG]]


@pytest.mark.parametrize("rel,flagged,accepted", [
    (-0.5e-6, True, True), (+0.5e-6, True, False),
    (-2e-6, False, True), (+2e-6, False, False),
    (-0.9e-6, True, True), (+0.9e-6, True, False),
])
def test_accept_near_flag(rel, flagged, accepted):
    u = 0.75 * (1.0 + rel)
    assert abs(f32(u) / 0.75 - 1.0 - rel) < 6e-8  # the offset survives fp32 rounding
    out = run(TGT_QUARTERS, DFT_THIRDS, [0], [u], 0.3)
    assert out["p"][0, 0] == pytest.approx(0.25, abs=1e-15)
    assert out["q"][0, 0] == pytest.approx(1 / 3, abs=1e-15)
    assert bool(out["flags"][0] & oracle.FLAG_ACCEPT_NEAR) == flagged
    assert (out["accepted"][0] == 1) == accepted
    # nothing else is flagged
    assert out["flags"][0] & ~oracle.FLAG_ACCEPT_NEAR == 0


@pytest.mark.parametrize("rel,flagged", [(0.5e-6, True), (-0.5e-6, True), (2e-6, False),
                                         (-2e-6, False)])
def test_accept_near_flag_is_relative(rel, flagged):
    # p'(0) = e / (e + 3) with e = exp(fp32 ln 2^-10) ~ 2^-10, q'(0) = 1/3: a
    # ratio near 0.003, where an absolute 1e-6 window would be 300 times too wide
    l0 = np.float32(np.log(2.0 ** -10))
    target = [[l0, 0.0, 0.0, 0.0]] * 2
    e0 = np.exp(np.float64(l0))
    p0 = e0 / (e0 + 3.0)
    ratio = p0 * 3.0
    assert abs(f32(ratio * (1.0 + rel)) / ratio - 1.0 - rel) < 6e-8
    out = run(target, DFT_THIRDS, [0], [ratio * (1.0 + rel)], 0.3)
    assert out["p"][0, 0] == pytest.approx(p0, rel=1e-12)
    assert bool(out["flags"][0] & oracle.FLAG_ACCEPT_NEAR) == flagged
    assert (out["accepted"][0] == 1) == (rel < 0)


def test_accept_near_flag_needs_positive_q():
    # q'(x) = 0: the ratio is unbounded, accepted iff p'(x) > 0, never flagged
    out = run(TGT_QUARTERS, [[NEG, 0.0, 0.0, 0.0]], [0], [0.75], 0.3)
    assert out["accepted"][0] == 1 and out["flags"][0] == 0


# ---------------------------------------------------------------------------
# inverse CDF: the bonus draw from p' = quarters (steps at 1/4, 1/2, 3/4), and
# the residual max(0, p' - q') = [0, 0, 1/4, 1/4] (S = 1/2, one inner step)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("step", [0.25, 0.5, 0.75])
@pytest.mark.parametrize("rel,flagged", [(-0.5e-6, True), (0.5e-6, True), (-2e-6, False),
                                         (2e-6, False)])
def test_cdf_near_flag_bonus(step, rel, flagged):
    u = step * (1.0 + rel)
    out = run(TGT_QUARTERS, DFT_THIRDS, [0], [0.0], u)
    assert out["accepted"][0] == 1 and out["S"][0] == pytest.approx(1.0, abs=1e-15)
    assert bool(out["flags"][0] & oracle.FLAG_CDF_NEAR) == flagged
    # the smallest j with C_j > u S: below a step the token before it
    want = int(step * 4) - 1 if rel < 0 else int(step * 4)
    assert out["tokens"][0, 1] == want


@pytest.mark.parametrize("rel,flagged", [(-0.5e-6, True), (0.5e-6, True), (-2e-6, False),
                                         (2e-6, False)])
def test_cdf_near_flag_residual(rel, flagged):
    # q' = [1/2, 1/2, 0, 0]: x = 0 has ratio 1/2, rejected at u = 0.9
    out = run(TGT_QUARTERS, [[0.0, 0.0, NEG, NEG]], [0], [0.9], 0.5 * (1.0 + rel))
    assert out["accepted"][0] == 0
    assert out["S"][0] == pytest.approx(0.5, abs=1e-15)
    assert bool(out["flags"][0] & oracle.FLAG_CDF_NEAR) == flagged
    assert out["tokens"][0, 0] == (2 if rel < 0 else 3)


def test_cdf_flag_is_relative_to_t():
    # a step at t = 2^-20 of S: 0.5e-6 relative is far below any absolute scale
    t = np.zeros((2, 3), np.float32)
    t[1] = [np.log(2.0 ** -20), 0.0, NEG]
    p = special.softmax(t[1].astype(np.float64))
    for rel, flagged in ((0.5e-6, True), (2e-6, False)):
        out = run(t, [[0.0, 0.0, 0.0]], [0], [0.0], p[0] * (1.0 + rel))
        assert bool(out["flags"][0] & oracle.FLAG_CDF_NEAR) == flagged


# ---------------------------------------------------------------------------
# top-p near its threshold: one row with logits [3, 2, 1, 0]
# ---------------------------------------------------------------------------

RAMP = np.array([3.0, 2.0, 1.0, 0.0], np.float32)
CUM = np.cumsum(special.softmax(RAMP.astype(np.float64)))  # a1, a2, a3, 1


def bonus_case(top_p, us):
    """K = 1: target row 0 and the draft row flat (their nucleus is one tie
    group of mass 1: never near top_p < 1 - 1e-6), the draft accepted at
    u = 0; the bonus row 1 is the ramp."""
    target = np.stack([np.zeros(4, np.float32), RAMP])
    return run(target, [np.zeros(4, np.float32)], [0], [0.0], us, 1.0, top_p)


@pytest.mark.parametrize("which,offset,shift", [
    (1, -0.5e-6, 1),   # after = a2 just above top_p: one group later adds token 2
    (0, +0.5e-6, 0),   # before = a1 just below top_p: one group earlier drops token 1
])
def test_topp_alternative_changes_the_bonus(which, offset, shift):
    top_p = CUM[which] + offset
    out = bonus_case(top_p, 0.999)
    f = out["flags"][0]
    assert f & oracle.FLAG_TOPP_EDGE and f & oracle.FLAG_TOPP_NEAR
    assert out["accepted"][0] == 1 and out["tokens"][0, 1] == 1  # defined nucleus {0, 1}
    an = out["alt_n"][0]
    assert (an >= 0).sum() == 1 and an[1, shift] == 1  # only target row 1 moved
    # the alternative equals the defined rule at a top_p that takes its membership
    membership_top_p = CUM[2] - 0.01 if shift == 1 else CUM[0] - 0.01
    alt_ref = bonus_case(membership_top_p, 0.999)
    assert out["alt_token"][0, 1, shift] == alt_ref["tokens"][0, 1] == (2 if shift else 0)
    assert out["alt_S"][0, 1, shift] == pytest.approx(alt_ref["S"][0], abs=1e-15)
    np.testing.assert_allclose(out["alt_p"][0, 1, shift], alt_ref["p"][0], atol=1e-15)


def test_topp_alternative_without_effect_is_not_flagged():
    # the same edge, but u = 0.1 draws token 0 under either nucleus
    out = bonus_case(CUM[1] - 0.5e-6, 0.1)
    f = out["flags"][0]
    assert f & oracle.FLAG_TOPP_EDGE and not f & oracle.FLAG_TOPP_NEAR
    assert out["alt_n"][0, 1, 1] == 1 and out["alt_token"][0, 1, 1] == 0


@pytest.mark.parametrize("offset", [-2e-6, 2e-6, -1e-4])
def test_topp_edge_outside_the_band_takes_no_alternative(offset):
    out = bonus_case(CUM[1] + offset, 0.999)
    assert out["flags"][0] & (oracle.FLAG_TOPP_EDGE | oracle.FLAG_TOPP_NEAR) == 0
    assert (out["alt_n"] == -1).all()


def test_topp_alternative_on_a_draft_row_changes_acceptance():
    """The draft row is the ramp with top_p just below a2: q'(0) = p0 / a2
    under the defined nucleus, p0 / a3 under the alternative; the target row
    is flat (p'(0) = 1/4).  u between the two ratios accepts only under the
    alternative."""
    top_p = CUM[1] - 0.5e-6
    p0 = special.softmax(RAMP.astype(np.float64))[0]
    r_def, r_alt = 0.25 / (p0 / CUM[1]), 0.25 / (p0 / CUM[2])
    u = 0.5 * (r_def + r_alt)
    target = np.zeros((2, 4), np.float32)
    out = run(target, [RAMP], [0], [u], 0.5, 1.0, top_p)
    f = out["flags"][0]
    assert f & oracle.FLAG_TOPP_NEAR
    assert out["accepted"][0] == 0
    row = 2  # draft row 0 of K = 1 is row K + 1
    assert out["alt_n"][0, row, 1] == 1
    assert out["q"][0, 0] == pytest.approx(p0 / CUM[1], rel=1e-12)
    assert out["alt_q"][0, row, 1, 0] == pytest.approx(p0 / CUM[2], rel=1e-12)
    assert out["alt_p"][0, row, 1, 0] == pytest.approx(0.25, abs=1e-15)


def test_flags_are_rare_on_the_reduced_workloads():
    """The exact comparison keeps nearly every request: at most one flagged
    request in 50 on reduced copies of the sampling settings."""
    import workloads as W
    total = flagged = 0
    for cfg, kw in ((0, {}), (2, dict(B=16, V=20011)), (3, dict(B=8, V=20011))):
        for seed in (0, 1):
            w = W.make_config(cfg, seed=seed, **kw)
            f = oracle.verify_workload(w)["flags"]
            total += w.B
            flagged += int(((f & oracle.FLAG_AMBIGUOUS) != 0).sum())
    assert flagged <= total // 50


# ---------------------------------------------------------------------------
# residual mass near the level below which the draw falls back to p'
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S_target,fallback,flagged", [
    (2.0 ** -26, True, False), (0.5 * oracle.S_RESOLUTION, True, True),
    (2.0 * oracle.S_RESOLUTION, False, True), (2.0 ** -16, False, False),
])
def test_small_residual_mass(S_target, fallback, flagged):
    """p' = [2d, 1 - 3d, d] and q' = [d, 1 - 3d, 2d]: token 2 (ratio 1/2)
    rejected at u = 3/4 leaves the residual [d, 0, 0], S = d.  At or below
    2^-20 the draw takes p' (token 1 at u_sample = 1/2), above it the
    residual (token 0); within a factor 4 of the level the request is
    flagged."""
    d = S_target
    lt = np.log(np.array([2 * d, 1 - 3 * d, d])).astype(np.float32)
    ld = np.log(np.array([d, 1 - 3 * d, 2 * d])).astype(np.float32)
    p = special.softmax(lt.astype(np.float64))
    q = special.softmax(ld.astype(np.float64))
    S = np.maximum(p - q, 0.0).sum()
    assert 0.5 < S / S_target < 2.0
    out = run([lt, lt], [ld], [2], [0.75], 0.5)
    assert out["accepted"][0] == 0
    assert bool(out["flags"][0] & oracle.FLAG_FALLBACK) == fallback
    assert bool(out["flags"][0] & oracle.FLAG_S_NEAR) == flagged
    if fallback:
        assert out["tokens"][0, 0] == 1 and out["S"][0] == pytest.approx(1.0, abs=1e-12)
    else:
        assert out["tokens"][0, 0] == 0 and out["S"][0] == pytest.approx(S, rel=1e-6)
