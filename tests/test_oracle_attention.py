"""Pins for the oracle's verify attention (CPU only).

"In full" item 6 of the optimisations page describes a multi-query verify
attention (several query tokens of one sequence at once); the oracle's
reading is causal attention over the cache with grouped-query heads.  Pinned
by a scalar evaluation of the definition on tiny inputs, closed forms and
invariants (what a query may not see does not matter, heads of a group with
equal queries agree, equal keys give the mean of the visible values).

The score scale 1/sqrt(D) is a reading (the page gives head_dim 256 but not
the scale); it is pinned by a closed form that does not restate the
formula: with two visible keys whose dot products with the query differ by
d, the two softmax weights stand in the ratio e^(d / sqrt(D)), read off an
output whose value rows are unit vectors.  Planted scales (1/D, none) fail.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float16)


def test_matches_a_scalar_evaluation():
    T, Hq, Hkv, L, D = 3, 4, 2, 7, 8
    q, k, v = _rand((T, Hq, D), 1), _rand((L, Hkv, D), 2), _rand((L, Hkv, D), 3)
    got = oracle.ref_verify_attention(q, k, v)
    for t in range(T):
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            ps = list(range(L - T + t + 1))
            s = [sum(float(q[t, h, d]) * float(k[p, kv, d]) for d in range(D)) / math.sqrt(D) for p in ps]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for d in range(D):
                want = sum(wi * float(v[p, kv, d]) for wi, p in zip(w, ps)) / sum(w)
                assert abs(got[t, h, d] - want) <= 1e-12 * max(1.0, abs(want))


def test_invisible_positions_do_not_matter():
    T, Hq, Hkv, L, D = 5, 6, 3, 40, 16
    q, k, v = _rand((T, Hq, D), 4), _rand((L, Hkv, D), 5), _rand((L, Hkv, D), 6)
    base = oracle.ref_verify_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[L - T + 1:] = 7.0          # positions after query 0's own
    v2[L - T + 1:] = -3.0
    alt = oracle.ref_verify_attention(q, k2, v2)
    assert np.array_equal(alt[0], base[0])
    assert not np.allclose(alt[1:], base[1:])


def test_equal_keys_average_the_visible_values():
    T, Hq, Hkv, L, D = 4, 2, 1, 9, 8
    q = _rand((T, Hq, D), 7)
    k = np.repeat(_rand((1, Hkv, D), 8), L, axis=0)
    v = _rand((L, Hkv, D), 9)
    got = oracle.ref_verify_attention(q, k, v)
    for t in range(T):
        want = v[: L - T + t + 1, 0].astype(np.float64).mean(axis=0)
        assert np.allclose(got[t, 0], want, rtol=0, atol=1e-12)
        assert np.allclose(got[t, 1], want, rtol=0, atol=1e-12)


def test_one_query_sees_everything_and_groups_share_values():
    T, Hq, Hkv, L, D = 1, 8, 2, 33, 256
    q, k, v = _rand((T, Hq, D), 10), _rand((L, Hkv, D), 11), _rand((L, Hkv, D), 12)
    q[0, 1] = q[0, 0]             # heads 0 and 1 share key/value head 0
    got = oracle.ref_verify_attention(q, k, v)
    assert np.array_equal(got[0, 0], got[0, 1])
    # a dominant score picks out one value row
    k2 = k.copy()
    k2[17, 0] = (q[0, 0].astype(np.float32) * 8).astype(np.float16)
    got2 = oracle.ref_verify_attention(q, k2, v)
    assert np.allclose(got2[0, 0], v[17, 0].astype(np.float64), atol=1e-6)


def _two_key_weight_ratios(attn, D, scale_q=1.0):
    """For (a, b) pairs: q = a e0 (times scale_q), keys 0 and b e0, values
    e0 and e1.  The output's first two entries are the two softmax weights,
    so out[1] / out[0] = exp((q . k1 - q . k0) * scale) = exp(a b * scale).
    Returns [(ratio seen, a * b)]."""
    out = []
    for a, b in ((2.0, 4.0), (1.0, -8.0), (4.0, 8.0), (0.5, 3.0), (-2.0, 6.0)):
        q = np.zeros((1, 1, D), np.float16)
        q[0, 0, 0] = np.float16(a * scale_q)
        k = np.zeros((2, 1, D), np.float16)
        k[1, 0, 0] = b
        v = np.zeros((2, 1, D), np.float16)
        v[0, 0, 0] = 1.0
        v[1, 0, 1] = 1.0
        o = attn(q, k, v)
        assert o[0, 0, 0] + o[0, 0, 1] == pytest.approx(1.0, abs=1e-15)
        out.append((o[0, 0, 1] / o[0, 0, 0], a * b))
    return out


@pytest.mark.parametrize("D", [256, 64])
def test_score_scale_closed_form(D):
    for ratio, ab in _two_key_weight_ratios(oracle.ref_verify_attention, D):
        assert ratio == pytest.approx(math.exp(ab / math.sqrt(D)), rel=1e-12), (D, ab)


@pytest.mark.parametrize("planted,scale_q", [("1/D", 1.0 / 16.0), ("no scale", 16.0)])
def test_planted_score_scales_fail_the_closed_form(planted, scale_q):
    # q scaled by 1/16 (exact in fp16 for these values) is attention with
    # scale 1/256 = 1/D at D = 256; q scaled by 16 is attention with no scale
    got = _two_key_weight_ratios(oracle.ref_verify_attention, 256, scale_q)
    assert all(q == pytest.approx(math.exp(ab * scale_q / 16.0), rel=1e-12) for q, ab in got)
    assert not any(q == pytest.approx(math.exp(ab / 16.0), rel=1e-6) for q, ab in got), planted
