"""Pins for the oracle's per-token int8 activation quantiser (CPU only).

The quantiser follows "In full" item 4 of the optimisations page (activations
quantised to int8 per token) with the readings scale = absmax / 127 in IEEE
fp32 and round-half-to-even codes clamped to +-127.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import exact


def _f32(fr):
    return np.float32(float(fr))


def test_absmax_127_gives_unit_scale_and_ties_to_even():
    row = np.array([127.0, 0.5, 1.5, 2.5, -2.5, -0.5, 3.5, -127.0], np.float16)
    q, s = oracle.quant_act(row[None, :])
    assert s[0] == np.float32(1.0)
    assert q[0].tolist() == [127, 0, 2, 2, -2, 0, 4, -127]


def test_zero_row_constant_row_and_bounds():
    x = np.zeros((3, 256), np.float16)
    x[1] = np.float16(0.3)
    x[2] = np.float16(-7.0)
    q, s = oracle.quant_act(x)
    assert s[0] == 0 and not q[0].any()
    assert (q[1] == 127).all() and (q[2] == -127).all()
    assert s[2] == np.float32(7.0) / np.float32(127.0)


def test_idempotent_on_the_int8_grid():
    rng = np.random.default_rng(5)
    for e in (-6, -3, 0, 2):
        codes = rng.integers(-127, 128, size=(4, 384))
        codes[:, 7] = 127
        codes[1, 7] = -127
        x = (codes * 2.0 ** e).astype(np.float16)
        assert (x.astype(np.float64) == codes * 2.0 ** e).all()
        q, s = oracle.quant_act(x)
        assert (s == np.float32(2.0 ** e)).all()
        assert (q.astype(np.int64) == codes).all()


def test_matches_exact_rational_definition():
    """Brute force: IEEE fp32 division and round-half-even done on Fractions."""
    x = synth.acts(6, 256, 1.0, 0.01, 20.0, seed=11)
    # add hand-made rows: exact ties after the division, subnormal fp16 inputs
    x[3, :] = np.float16(0)
    x[3, :8] = np.array([12.7, 0.05, 0.15, 0.25, 0.35, -0.05, 6e-8, -6e-8], np.float16)
    x[4, :] = np.float16(6e-8)
    x[4, 0] = np.float16(-1e-7)
    q, s = oracle.quant_act(x)
    for m in range(x.shape[0]):
        eq, es = exact.quant_row(x[m])
        assert s[m] == _f32(es), m
        assert q[m].tolist() == eq, m


def test_absmax_element_maps_to_127_and_codes_bounded():
    x = synth.acts(64, 5120, 1.0, 0.01, 20.0, seed=1)
    q, s = oracle.quant_act(x)
    assert np.abs(q.astype(np.int32)).max() <= 127
    am = np.abs(x.astype(np.float32)).argmax(axis=1)
    assert (np.abs(q[np.arange(64), am].astype(np.int32)) == 127).all()
    assert (s > 0).all()


@pytest.mark.parametrize("mistake", ["reciprocal", "round_half_away", "unsigned_abs"])
def test_pin_catches_planted_mistakes(mistake):
    """A quantiser with a plausible mistake disagrees with the exact definition
    on some pinned input, so the exact-definition pin can fail."""
    x = synth.acts(8000, 128, 1.0, 0.01, 20.0, seed=21)
    x[0, :6] = np.array([127.0, 0.5, 1.5, 2.5, -2.5, 3.0], np.float16)

    xf = x.astype(np.float32)
    s = np.abs(xf).max(axis=1) / np.float32(127)
    if mistake == "reciprocal":
        v = np.rint(xf * (np.float32(1) / s)[:, None])
    elif mistake == "round_half_away":
        t = xf / s[:, None]
        v = np.sign(t) * np.floor(np.abs(t) + np.float32(0.5))
    else:  # sign dropped
        v = np.rint(np.abs(xf) / s[:, None])
    qb = np.clip(v, -127, 127).astype(np.int8)
    qo, _ = oracle.quant_act(x)
    rows = np.nonzero((qb != qo).any(axis=1))[0]
    assert rows.size > 0
    m = int(rows[0])
    eq, _ = exact.quant_row(x[m])
    assert qo[m].tolist() == eq
    assert qb[m].tolist() != eq
