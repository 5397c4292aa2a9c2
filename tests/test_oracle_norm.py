"""Pins for the oracle's RMSNorm and fused normalise-and-quantise step (CPU only).

The pages name no norm, so ``oracle.rmsnorm`` is a reading (its docstring has
the definition: the float64 value of x * w / sqrt(mean(x^2) + eps), rounded
once to fp16): parity unpinned as to the pages.  These tests pin the oracle
to that definition by other means: a 60-digit decimal evaluation rounded to
fp16 by hand, closed forms (constant rows, with and without eps), exact
invariances (power-of-two scaling of x without eps, the sign of x, doubling
the weight), and planted mistakes in the norm (mean over H - 1, a dropped
eps, a dropped square root) that the closed forms reject.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact


def _decimal_norm_row(x, w, eps):
    """fp16 values (as Fractions) of one row by 60-digit decimal arithmetic:
    y = fp16(x * w / sqrt(sum(x^2) / H + eps)), rounded by hand."""
    getcontext().prec = 60
    xs = [Decimal(float(v)) for v in x]                      # fp16 -> float -> Decimal: exact
    ws = [Decimal(float(v)) for v in w]
    H = len(xs)
    t = sum(v * v for v in xs) / H + Decimal(float(np.float32(eps)))
    if t == 0:
        return [Fraction(0)] * H
    r = 1 / t.sqrt()
    return [exact.round_f16(Fraction(v * r * wv)) for v, wv in zip(xs, ws)]


def _as_fractions(y):
    return [Fraction(float(v)) for v in y]


@pytest.mark.parametrize("H,eps,seed", [(5, 1e-6, 1), (8, 0.25, 2), (13, 3e-3, 3), (128, 0.0, 4), (640, 1e-5, 5)])
def test_matches_a_decimal_evaluation(H, eps, seed):
    rng = np.random.default_rng(seed)
    rows = 400 if H <= 128 else 40
    mags = np.exp(rng.uniform(np.log(1e-3), np.log(30.0), size=(rows, 1)))
    x = (rng.standard_normal((rows, H)) * mags).astype(np.float16)
    w = (1.0 + 0.5 * rng.standard_normal(H)).astype(np.float16)
    y = oracle.rmsnorm(x, w, eps)
    for m in range(rows):
        assert _as_fractions(y[m]) == _decimal_norm_row(x[m], w, eps), (H, eps, m)


def test_decimal_evaluation_on_workload_rows():
    x = synth.acts(3, 5120, 1.0, 0.01, 20.0, seed=11)
    w = (1.0 + 0.1 * synth.acts(1, 5120, 1.0, 0.0, 1.0, seed=12)[0].astype(np.float32)).astype(np.float16)
    y = oracle.rmsnorm(x, w, 1e-6)
    for m in range(3):
        assert _as_fractions(y[m]) == _decimal_norm_row(x[m], w, 1e-6), m


def _planted(kind):
    """Norms with one planted mistake each, for the closed-form pins to reject."""
    def f(x, w, eps):
        xf = x.astype(np.float64)
        H = xf.shape[1]
        ss = (xf * xf).sum(axis=1, keepdims=True)
        if kind == "mean over H-1":
            t = ss / (H - 1) + eps
        elif kind == "no eps":
            t = ss / H
        elif kind == "no sqrt":
            return (xf / (ss / H + eps) * w.astype(np.float64)).astype(np.float16)
        return (xf / np.sqrt(t) * w.astype(np.float64)).astype(np.float16)
    return f


def _constant_row_pins(norm):
    """Closed forms: a constant row c gives r = 1 / sqrt(c^2 + eps), so
    y = w * sign(c) at eps = 0 and fp16(w * c / sqrt(c^2 + eps)) otherwise."""
    H = 256
    x = np.zeros((3, H), np.float16)
    x[0] = np.float16(4.0)
    x[1] = np.float16(-0.125)
    x[2] = np.float16(1.0)
    w = np.full(H, np.float16(1.5))
    y0 = norm(x, w, 0.0)
    ok = bool((y0[0] == np.float16(1.5)).all() and (y0[1] == np.float16(-1.5)).all())
    # c = 1, eps = 0.25: y = 1.5 / sqrt(1.25) = 1.5 * 2 / sqrt(5) = 3 / sqrt(5)
    getcontext().prec = 60
    want = exact.round_f16(Fraction(Decimal(3) / Decimal(5).sqrt()))
    ye = norm(x, w, 0.25)
    ok = ok and all(Fraction(float(v)) == want for v in ye[2])
    return ok


def test_constant_rows_normalise_to_the_weight():
    assert _constant_row_pins(oracle.rmsnorm)
    H = 256
    z = np.zeros((2, H), np.float16)
    w = np.full(H, np.float16(1.5))
    assert not oracle.rmsnorm(z, w, 0.0).astype(np.float32).any()   # zero row, eps = 0: r = 0
    assert not oracle.rmsnorm(z, w, 1e-6).astype(np.float32).any()


@pytest.mark.parametrize("kind", ["mean over H-1", "no eps", "no sqrt"])
def test_planted_mistakes_fail_the_closed_forms(kind):
    assert not _constant_row_pins(_planted(kind))


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


def test_sign_and_weight_doubling_are_exact():
    x = synth.acts(6, 384, 1.0, 0.01, 20.0, seed=15)
    w = synth.acts(1, 384, 0.5, 0.0, 1.0, seed=16)[0]
    y = oracle.rmsnorm(x, w, 1e-5).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(-x, w, 1e-5).astype(np.float32), -y)
    w2 = (w.astype(np.float32) * 2).astype(np.float16)
    y2 = oracle.rmsnorm(x, w2, 1e-5).astype(np.float32)
    normal = np.abs(y) >= 2.0 ** -14                         # doubling is exact outside the subnormals
    assert normal.mean() > 0.9 and np.array_equal(y2[normal], 2 * y[normal])


def test_fused_step_is_the_quantiser_on_the_normalised_rows():
    x = synth.acts(5, 640, 1.0, 0.01, 20.0, seed=13)
    w = synth.acts(1, 640, 1.0, 0.0, 1.0, seed=14)[0]
    y, q, s = oracle.rmsnorm_quant(x, w, 1e-5)
    assert np.array_equal(y.view(np.uint16), oracle.rmsnorm(x, w, 1e-5).view(np.uint16))
    assert (np.abs(q).max(axis=1) == 127).all()
    assert np.array_equal(s, np.abs(y.astype(np.float32)).max(axis=1) / np.float32(127.0))
