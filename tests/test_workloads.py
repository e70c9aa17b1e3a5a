"""Input generators: determinism, dtype handling, uniform grid, shapes."""
import numpy as np

import workloads as W


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38, 1e-30], np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert back[1] == 1.0
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    assert back[3] == -2.5
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_uniforms_on_grid():
    r = W.rngs(0, 0)["uniforms"]
    u = W.uniforms_on_grid(r, 100000)
    k = u.astype(np.float64) * 2 ** 24
    assert np.all(k == np.floor(k)) and u.min() >= 0 and u.max() < 1


def test_deterministic_and_seeded():
    a = W.make_config(2, B=2, V=300)
    b = W.make_config(2, B=2, V=300)
    c = W.make_config(2, B=2, V=300, seed=1)
    np.testing.assert_array_equal(a.target, b.target)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    assert not np.array_equal(a.target, c.target)


def test_shapes_and_dtypes():
    for i in range(5):
        w = W.make_config(i, B=2, V=257)
        assert w.target.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
        if w.kind == "sample":
            assert w.target.shape == (2, w.K + 1, 257) and w.draft.shape == (2, w.K, 257)
            assert w.u_accept.shape == (2, w.K) and w.u_sample.shape == (2,)
            assert ((w.tokens >= 0) & (w.tokens < 257)).all()
        elif w.kind == "greedy":
            assert w.target.shape == (2, w.K + 1, 257) and w.tokens.shape == (2, w.K)
        else:
            assert w.target.shape == (2, w.K, 257)


def test_draft_tokens_follow_drafter_nucleus():
    w = W.make_config(3, B=4, V=2000)
    d = w.draft.astype(np.float64)
    for b in range(4):
        for i in range(w.K):
            l = d[b, i]
            x = w.tokens[b, i]
            order = np.argsort(-l)
            rank = int(np.where(order == x)[0][0])
            e = np.exp((l[order] - l[order[0]]) / w.temperature)
            cum = np.cumsum(e) / e.sum()
            assert rank == 0 or cum[rank - 1] < w.top_p
