"""Pins for the oracle's RMSNorm and fused normalise-and-quantise step (CPU only).

The pages name no norm, so ``oracle.rmsnorm`` is a reading (its docstring has
the definition): parity unpinned as to the pages.  These tests pin the oracle
to that definition by other means: an exact-rational evaluation of every
rounding on small rows, closed forms, an exact invariance under power-of-two
scaling, padding invariance of the tree sum, and a float64 bound.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import synth
from tests import exact


def _ulp32(f: Fraction) -> Fraction:
    a = abs(f)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return Fraction(2) ** (max(e, -126) - 23)


def _rn_sqrt32(t: Fraction) -> Fraction:
    """Correctly rounded float32 square root of t, checked exactly: the
    candidate's half-ulp neighbourhood must contain sqrt(t)."""
    f = Fraction(float(np.sqrt(np.float32(float(t)))))
    for cand in (f, f + _ulp32(f), f - _ulp32(f)):
        half_lo = _ulp32(cand - _ulp32(cand) / 4) / 2 if cand > 0 else Fraction(0)
        half_hi = _ulp32(cand) / 2
        if (cand - half_lo) ** 2 <= t <= (cand + half_hi) ** 2:
            return cand
    raise AssertionError("no correctly rounded square root found")


def _exact_factor(x, eps):
    """r of the definition for one row, with exact rationals, rounding by hand."""
    H = len(x)
    sq = [Fraction(float(v)) ** 2 for v in x]
    assert all(exact.round_f32(s) == s for s in sq)        # squares are exact in fp32
    p = 1
    while p < H:
        p *= 2
    level = sq + [Fraction(0)] * (p - H)
    while len(level) > 1:
        level = [exact.round_f32(level[i] + level[i + 1]) for i in range(0, len(level), 2)]
    t = exact.round_f32(exact.round_f32(level[0] / H) + Fraction(float(np.float32(eps))))
    return exact.round_f32(1 / _rn_sqrt32(t)) if t > 0 else Fraction(0)


@pytest.mark.parametrize("H,eps", [(5, 1e-6), (8, 0.25), (13, 3e-3), (16, 0.0)])
def test_rmsnorm_factor_matches_an_exact_evaluation(H, eps):
    rng = np.random.default_rng(H)
    mags = np.exp(rng.uniform(np.log(1e-3), np.log(30.0), size=(1500, 1)))
    x = (rng.standard_normal((1500, H)) * mags).astype(np.float16)
    r = oracle.rmsnorm_factor(x, eps)
    for m in range(len(x)):
        assert Fraction(float(r[m])) == _exact_factor(x[m], eps), (H, eps, m)


@pytest.mark.parametrize("H,seed", [(5, 1), (8, 2), (13, 3), (128, 4)])
def test_rmsnorm_products_match_an_exact_evaluation(H, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, H)) * np.array([[0.01], [1.0], [300.0]])).astype(np.float16)
    w = (1.0 + 0.5 * rng.standard_normal(H)).astype(np.float16)
    for eps in (1e-6, 0.25):
        y32 = oracle.rmsnorm_f32(x, w, eps)
        y16 = oracle.rmsnorm(x, w, eps)
        for m in range(3):
            r = _exact_factor(x[m], eps)
            want = [exact.round_f32(exact.round_f32(Fraction(float(v)) * r) * Fraction(float(wv)))
                    for v, wv in zip(x[m], w)]
            assert [Fraction(float(v)) for v in y32[m]] == want, (H, m, eps)
            assert [Fraction(float(v)) for v in y16[m]] == [exact.round_f16(v) for v in want]


def test_tree_sum_closed_form_and_padding():
    v = np.array([[1e8, 1.0, -1e8, 1.0, 3.0]], np.float32)
    # ((v0 + v1) + (v2 + v3)) + (v4 + 0): fp32(1e8 + 1) = 1e8, so the 1s vanish
    a = np.float32(np.float32(1e8) + np.float32(1.0))
    b = np.float32(np.float32(-1e8) + np.float32(1.0))
    want = np.float32(np.float32(a + b) + np.float32(3.0))
    assert oracle.tree_sum_f32(v)[0] == want == np.float32(3.0)
    rng = np.random.default_rng(7)
    w = rng.standard_normal((4, 37)).astype(np.float32)
    padded = np.concatenate([w, np.zeros((4, 91), np.float32)], axis=1)
    assert np.array_equal(oracle.tree_sum_f32(w), oracle.tree_sum_f32(padded))
    ints = rng.integers(-1000, 1000, size=(3, 640)).astype(np.float32)     # every partial sum exact
    assert np.array_equal(oracle.tree_sum_f32(ints), ints.sum(axis=1))


def test_tree_sum_error_bound_against_exact_sum():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal((6, 5120)) ** 2).astype(np.float32)
    got = oracle.tree_sum_f32(v)
    for m in range(6):
        ex = math.fsum(float(t) for t in v[m])
        bound = math.ceil(math.log2(5120)) * 2.0 ** -24 * math.fsum(abs(float(t)) for t in v[m])
        assert abs(float(got[m]) - ex) <= bound


def test_constant_rows_normalise_to_the_weight():
    H = 256
    x = np.zeros((3, H), np.float16)
    x[0] = np.float16(4.0)
    x[1] = np.float16(-0.125)
    w = np.full(H, np.float16(1.5))
    y = oracle.rmsnorm(x, w, 0.0)
    assert (y[0] == np.float16(1.5)).all() and (y[1] == np.float16(-1.5)).all()
    assert not y[2].any()                                    # zero row, eps = 0: r = 0
    assert not oracle.rmsnorm(x[2:], w, 1e-6).any()


def test_power_of_two_scaling_is_exact_without_eps():
    rng = np.random.default_rng(9)
    # magnitudes in [0.5, 1.5]: every scaled value below stays a normal fp16
    x = (np.where(rng.random((4, 256)) < 0.5, -1.0, 1.0) * (0.5 + rng.random((4, 256)))).astype(np.float16)
    w = synth.acts(1, x.shape[1], 1.0, 0.0, 1.0, seed=3)[0]
    y = oracle.rmsnorm(x, w, 0.0)
    for k in (-8, -1, 3, 7):
        xs = (x.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16)
        assert np.array_equal(xs.astype(np.float32), x.astype(np.float32) * np.float32(2.0 ** k))
        assert np.array_equal(oracle.rmsnorm(xs, w, 0.0).view(np.uint16), y.view(np.uint16)), k


def test_rmsnorm_within_one_fp16_ulp_of_float64():
    x = synth.acts(16, 5120, 1.0, 0.01, 20.0, seed=11)
    w = (1.0 + 0.1 * synth.acts(1, 5120, 1.0, 0.0, 1.0, seed=12)[0].astype(np.float32)).astype(np.float16)
    y = oracle.rmsnorm(x, w, 1e-6).astype(np.float64)
    xf = x.astype(np.float64)
    y64 = xf / np.sqrt((xf * xf).mean(axis=1, keepdims=True) + 1e-6) * w.astype(np.float64)[None, :]
    ulp = np.spacing(np.abs(y64).astype(np.float16)).astype(np.float64)
    assert (np.abs(y - y64) <= ulp * 1.01).all()


def test_fused_step_is_the_quantiser_on_the_normalised_rows():
    x = synth.acts(5, 640, 1.0, 0.01, 20.0, seed=13)
    w = synth.acts(1, 640, 1.0, 0.0, 1.0, seed=14)[0]
    y, q, s = oracle.rmsnorm_quant(x, w, 1e-5)
    assert np.array_equal(y.view(np.uint16), oracle.rmsnorm(x, w, 1e-5).view(np.uint16))
    assert (np.abs(q).max(axis=1) == 127).all()
    assert np.array_equal(s, np.abs(y.astype(np.float32)).max(axis=1) / np.float32(127.0))
