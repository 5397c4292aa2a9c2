"""Pins for the oracle's W4A8 / W4A16 / W8A16 references (CPU only).

The references follow "In full" item 4 of the optimisations page (int4
weights with signed group scales, int8 per-token activations, integer
accumulation per 128-wide group) and the project README's "What each step
buys" (W4A16 body).  Each is checked against brute force with exact
rationals, closed forms and invariants that a dropped term, a wrong sign or a
transposed operand would break.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact


def _exact_w4a8(x, codes, scales):
    M, K = x.shape
    N = codes.shape[0]
    out = []
    for m in range(M):
        q, s = exact.quant_row(x[m])
        row = []
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                P = sum(q[k] * int(codes[n, k]) for k in range(g * 128, g * 128 + 128))
                tot += P * Fraction(float(scales[n, g]))
            row.append(s * tot)
        out.append(row)
    return out


def _exact_w4a16(x, codes, scales):
    M, K = x.shape
    N = codes.shape[0]
    xs = [[Fraction(float(v)) for v in x[m]] for m in range(M)]
    sc = [[Fraction(float(v)) for v in scales[n]] for n in range(N)]
    return [[sum(xs[m][k] * int(codes[n, k]) * sc[n][k // 128] for k in range(K))
             for n in range(N)] for m in range(M)]


def _close(y, ex, rel=2.0 ** -48):
    ex = np.array([[float(v) for v in r] for r in ex])
    scale = max(1e-300, np.abs(ex).max())
    return np.abs(np.asarray(y) - ex).max() <= rel * scale


def test_partials_brute_force_tiny_config():
    cfg = synth.CONFIGS["tiny_w4a8"]
    x, codes, scales = synth.gemm_inputs(cfg)
    q, s = oracle.quant_act(x)
    P = oracle.partials(q, codes)
    qi = q.astype(int).tolist()
    ci = codes.astype(int).tolist()
    M, K = q.shape
    N = codes.shape[0]
    for m in range(M):
        for n in range(N):
            for g in range(K // 128):
                ref = 0
                qm, cn = qi[m], ci[n]
                for k in range(g * 128, g * 128 + 128):
                    ref += qm[k] * cn[k]
                assert P[m, n, g] == ref
    assert np.abs(P).max() <= 127 * 8 * 128


def test_partials_with_unit_codes_are_group_row_sums():
    q, _ = oracle.quant_act(synth.acts(5, 512, 1.0, 0.01, 20.0, seed=8))
    P = oracle.partials(q, np.ones((3, 512), np.int8))
    want = q.astype(np.int64).reshape(5, 4, 128).sum(axis=2)
    assert (P == want[:, None, :]).all()


def test_partials_extreme_bound_is_reached():
    q = np.full((1, 128), -127, np.int8)
    codes = np.full((1, 128), -8, np.int8)
    assert oracle.partials(q, codes)[0, 0, 0] == 127 * 8 * 128


def test_w4a8_matches_exact_rationals():
    x = synth.acts(2, 256, 1.0, 0.01, 20.0, seed=31)
    codes, scales = synth.weights(8, 256, seed=32)
    codes[0, :] = -8
    assert _close(oracle.ref_w4a8(x, codes, scales), _exact_w4a8(x, codes, scales))


def test_w4a16_matches_exact_rationals():
    x = synth.acts(2, 256, 1.0, 0.0, 1.0, seed=33)
    codes, scales = synth.weights(8, 256, seed=34)
    codes[1, :] = -8
    assert _close(oracle.ref_w4a16(x, codes, scales), _exact_w4a16(x, codes, scales))


def test_w8a16_matches_exact_rationals_and_row_subset():
    x = synth.acts(2, 256, 1.0, 0.0, 1.0, seed=35)
    rng = np.random.default_rng(36)
    Q = rng.integers(-127, 128, size=(9, 256)).astype(np.int8)
    S = (rng.uniform(1e-4, 1e-3, size=(9, 2)) * np.where(rng.random((9, 2)) < 0.5, -1, 1)).astype(np.float16)
    ex = _exact_w4a16(x, Q, S)          # same formula, Q in place of int4 codes
    assert _close(oracle.ref_w8a16(x, Q, S), ex)
    rows = [7, 0, 3]
    sub = oracle.ref_w8a16(x, Q, S, rows=rows)
    assert _close(sub, [[r[v] for v in rows] for r in ex])


def test_power_of_two_scales_give_exact_results():
    rng = np.random.default_rng(40)
    x = rng.integers(-20, 21, size=(3, 384)).astype(np.float16)
    codes = rng.integers(-8, 8, size=(5, 384)).astype(np.int8)
    e = rng.integers(-9, -6, size=(5, 3))
    scales = (np.where(rng.random((5, 3)) < 0.5, -1.0, 1.0) * 2.0 ** e).astype(np.float16)
    want = np.zeros((3, 5))
    for m in range(3):
        for n in range(5):
            want[m, n] = sum(float(x[m, k]) * int(codes[n, k]) * float(scales[n, k // 128]) for k in range(384))
    assert (oracle.ref_w4a16(x, codes, scales) == want).all()


@pytest.mark.parametrize("ref", ["w4a8", "w4a16"])
def test_sign_flip_of_a_group_is_invisible_including_minus_8(ref):
    """Negating a group's codes and its scale leaves the product unchanged;
    -8 becomes +8, which int4 cannot hold, so a sign fold into the codes is
    not a valid implementation but the reference value is unchanged."""
    x, codes, scales = synth.gemm_inputs(synth.CONFIGS["tiny_w4a8"])
    codes = codes.copy()
    codes[:, :128][::3] = -8
    f = oracle.ref_w4a8 if ref == "w4a8" else oracle.ref_w4a16
    y0 = f(x, codes, scales)
    c2 = codes.astype(np.int16)
    s2 = scales.copy()
    c2[:, :128] = -c2[:, :128]
    s2[:, 0] = -s2[:, 0]
    assert (c2 == 8).any()
    y1 = f(x, c2, s2)
    assert (y0 == y1).all()
    # element-wise dequantisation identity for every int4 code, -8 included
    for q in range(-8, 8):
        for sv in (np.float16(0.0078125), np.float16(-0.00123), np.float16(0.0099)):
            assert (-q) * -float(sv) == q * float(sv)


def test_w4a8_equals_w4a16_when_activations_sit_on_the_int8_grid():
    rng = np.random.default_rng(41)
    codes_x = rng.integers(-127, 128, size=(4, 512))
    codes_x[:, 0] = 127
    x = (codes_x * 2.0 ** -5).astype(np.float16)
    codes, scales = synth.weights(16, 512, seed=42)
    assert (oracle.ref_w4a8(x, codes, scales) == oracle.ref_w4a16(x, codes, scales)).all()


def test_scale_sign_matters():
    """The pages' failure mode: reading signed scales as unsigned gives a
    different (wrong) result that the fp16 bounds reject."""
    x, codes, scales = synth.gemm_inputs(synth.CONFIGS["tiny_w4a8"])
    good = oracle.ref_w4a8(x, codes, scales)
    bad = oracle.ref_w4a8(x, codes, np.abs(scales))
    assert not oracle.fp16_bounds(bad.astype(np.float16), good)["ok"]
    assert oracle.fp16_bounds(good.astype(np.float16), good)["ok"]


@pytest.mark.parametrize("mistake", ["transposed_group_scale", "dropped_last_group", "token_scale_squared"])
def test_exact_pin_catches_planted_mistakes(mistake):
    x = synth.acts(2, 256, 1.0, 0.01, 20.0, seed=31)
    codes, scales = synth.weights(8, 256, seed=32)
    q, s = oracle.quant_act(x)
    sc = scales.astype(np.float64)
    acc = np.zeros((2, 8))
    for g in range(2):
        if mistake == "dropped_last_group" and g == 1:
            continue
        Pg = q[:, g * 128:(g + 1) * 128].astype(np.float64) @ codes[:, g * 128:(g + 1) * 128].astype(np.float64).T
        col = sc[:, 1 - g] if mistake == "transposed_group_scale" else sc[:, g]
        acc += Pg * col[None, :]
    sv = s.astype(np.float64)
    y = acc * (sv * sv if mistake == "token_scale_squared" else sv)[:, None]
    assert not _close(y, _exact_w4a8(x, codes, scales))


def test_fp16_bounds_accept_fp16_rounding_and_gpu_like_accumulation():
    """The tolerance is reachable by an fp16-dequantising, fp32-accumulating
    implementation, and rejects fp16 accumulation of split partial sums."""
    x = synth.acts(16, 5120, 1.0, 0.0, 1.0, seed=43)
    codes, scales = synth.weights(512, 5120, seed=44)
    ref = oracle.ref_w4a16(x, codes, scales)
    wt = (codes.astype(np.float32) * np.repeat(scales.astype(np.float32), 128, axis=1)).astype(np.float16)
    xf = x.astype(np.float32)
    acc = np.zeros((16, 512), np.float32)
    for k0 in range(0, 5120, 32):
        acc += xf[:, k0:k0 + 32] @ wt[:, k0:k0 + 32].astype(np.float32).T
    r = oracle.fp16_bounds(acc.astype(np.float16), ref)
    assert r["ok"], r
    half = np.zeros((16, 512), np.float16)
    for k0 in range(0, 5120, 640):
        part = (xf[:, k0:k0 + 640] @ wt[:, k0:k0 + 640].astype(np.float32).T).astype(np.float16)
        half = (half.astype(np.float32) + part.astype(np.float32)).astype(np.float16)
    assert not oracle.fp16_bounds(half, ref)["ok"]
