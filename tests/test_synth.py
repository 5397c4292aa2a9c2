"""Statistics and determinism of the seeded input generators (CPU only)."""
import json
import os

import numpy as np

import synth


def test_weights_statistics_match_the_pages():
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")) as f:
        neg = json.load(f)["negative_group_scale_share"]
    codes, scales = synth.weights(2048, 5120, seed=1)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    assert set(np.unique(codes).tolist()) == set(range(-8, 8))
    frac = float((scales < 0).mean())
    lo, hi = neg["accept"]
    assert lo <= frac <= hi, frac
    mag = np.abs(scales.astype(np.float64))
    assert mag.min() >= 1e-3 * (1 - 2 ** -11) and mag.max() <= 1e-2 * (1 + 2 ** -11)
    # log-uniform: about half the magnitudes below the geometric midpoint
    assert abs(float((mag < np.sqrt(1e-5)).mean()) - 0.5) < 0.01


def test_activation_outlier_fraction_and_scale():
    x = synth.acts(256, 5120, 1.0, 0.01, 20.0, seed=101).astype(np.float64)
    assert abs(float((np.abs(x) > 6).mean()) - 0.01 * 0.77) < 0.002   # P(|20 z| > 6) = P(|z| > .3)
    assert abs(float(np.median(np.abs(x))) - 0.6745) < 0.02
    y = synth.acts(64, 5120, 0.5, 0.0, 1.0, seed=3).astype(np.float64)
    assert abs(y.std() - 0.5) < 0.01


def test_generation_is_deterministic_and_independent_of_threads(monkeypatch):
    a = synth.weights(3000, 256, seed=9)
    b = synth.weights(3000, 256, seed=9)
    monkeypatch.setattr(synth, "_workers", lambda: 1)
    c = synth.weights(3000, 256, seed=9)
    for u, v, w in zip(a, b, c):
        assert u.tobytes() == v.tobytes() == w.tobytes()
    assert synth.acts(5, 128, 1.0, 0.01, 20.0, seed=2).tobytes() == synth.acts(5, 128, 1.0, 0.01, 20.0, seed=2).tobytes()
    assert not np.array_equal(synth.weights(4, 128, 1)[0], synth.weights(4, 128, 2)[0])


def test_token_ids_in_range():
    ids = synth.token_ids(64, 248320, seed=304)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < 248320


def test_draft_ids_are_distinct_sorted_and_seeded():
    ids = synth.draft_ids(40960, 248320, seed=4)
    assert ids.shape == (40960,) and ids.dtype == np.int64
    assert ids.min() >= 0 and ids.max() < 248320
    assert np.all(np.diff(ids) > 0)
    assert np.array_equal(ids, synth.draft_ids(40960, 248320, seed=4))
