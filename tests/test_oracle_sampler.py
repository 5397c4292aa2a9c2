"""Pins of the oracle's top-k / top-p sampler (``oracle.topk_topp_sample``).

The page ("What this repo does that stock vLLM doesn't", "In full" item 6)
prints no worked example, so the oracle is pinned against arithmetic that
shares nothing with it:
  * a brute force in 60-digit decimal arithmetic over Python lists (its own
    ranking, exponentials, sums and comparisons), on many tiny rows;
  * closed forms: uniform rows (mass 1/k each, so the top-p count, the
    renormalised probabilities, the sampled rank and the log-sum-exp are
    known exactly), the tie rule, k = 1 (the first maximum);
  * invariances: scaling logits and temperature together, shifting logits,
    permuting the vocabulary;
  * the inverse-CDF property: uniforms spread over [0, 1) land on each rank
    in proportion to its probability;
  * scipy's logsumexp for the normaliser.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth


def _brute(row, k, p, T, u):
    """Decimal (60 digits) top-k / top-p / sample / log-sum-exp of one row."""
    getcontext().prec = 60
    vals = [Decimal(float(v)) for v in row]                 # fp16 -> float -> Decimal: exact
    Td = Decimal(float(np.float32(T)))
    order = sorted(range(len(vals)), key=lambda i: (-vals[i], i))
    top = order[:k]
    z = [vals[i] / Td for i in top]
    e = [(zi - z[0]).exp() for zi in z]
    tot = sum(e)
    mass = [ei / tot for ei in e]
    pd = Decimal(float(p))
    kept, before, margin = 0, Decimal(0), Decimal(1)
    for j in range(k):
        margin = min(margin, abs(before - pd))
        if before < pd:
            kept += 1
        before += mass[j]
    ks = sum(mass[:kept])
    probs = [m / ks for m in mass[:kept]]
    ud = Decimal(float(u))
    rank, c, umargin = kept - 1, Decimal(0), Decimal(1)
    for j in range(kept):
        c += probs[j]
        umargin = min(umargin, abs(c - ud))
        if c > ud:
            rank = j
            break
    zall = [v / Td for v in vals]
    zmax = max(zall)
    lse = zmax + sum((zi - zmax).exp() for zi in zall).ln()
    return dict(ids=top, mass=[float(m) for m in mass], probs=[float(q) for q in probs], kept=kept, rank=rank,
                lse=float(lse), margin=float(margin), umargin=float(umargin))


def test_against_decimal_brute_force():
    rng = np.random.default_rng(7)
    for case in range(300):
        V = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(V, 12) + 1))
        grid = [0.0, 0.25, 1.0][case % 3]                    # coarse grids give ties
        v = rng.normal(0, 2.0, V)
        if grid:
            v = np.round(v / grid) * grid
        row = v.astype(np.float16)
        p = float(rng.choice([1.0, rng.uniform(0.05, 1.0)]))
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        u = float(np.float32(rng.random()))
        got = oracle.topk_topp_sample(row[None, :], k, p, T, np.array([u], np.float32))
        want = _brute(row, k, p, T, u)
        assert got["ids"][0].tolist() == want["ids"], case
        np.testing.assert_allclose(got["mass"][0], want["mass"], rtol=1e-12, atol=1e-300)
        if want["margin"] > 1e-12:
            assert got["kept"][0] == want["kept"], case
            np.testing.assert_allclose(got["probs"][0, :want["kept"]], want["probs"], rtol=1e-12, atol=1e-300)
            assert np.all(got["probs"][0, want["kept"]:] == 0)
            if want["umargin"] > 1e-12:
                assert got["rank"][0] == want["rank"], case
                assert got["sampled"][0] == want["ids"][want["rank"]]
        assert abs(got["lse"][0] - want["lse"]) <= 1e-12 * max(1.0, abs(want["lse"]))


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_uniform_row_closed_form(k):
    # Equal logits: mass 1/k for each of the k lowest ids; with k a power of
    # two every partial sum is exact, so rank j is kept iff j/k < p exactly.
    V, c, T = 16, 1.5, 0.75
    row = np.full((1, V), c, np.float16)
    for p in [0.1, 0.25, 0.5, 0.5 + 1e-9, 0.75, 1.0]:
        for u in [0.0, 0.3, 0.49999, 0.5, 0.99]:
            got = oracle.topk_topp_sample(row, k, p, T, np.array([u]))
            kept = sum(1 for j in range(k) if Fraction(j, k) < Fraction(p))
            assert got["ids"][0].tolist() == list(range(k))
            assert got["kept"][0] == kept
            assert np.all(got["probs"][0, :kept] == 1.0 / kept) and np.all(got["probs"][0, kept:] == 0)
            # smallest j with (j + 1) / kept > u
            assert got["rank"][0] == min(int(Fraction(u) * kept), kept - 1)
            assert got["lse"][0] == pytest.approx(c / T + np.log(V), rel=0, abs=1e-14)


def test_tie_rule_lower_index_first():
    row = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float16)
    assert oracle.topk_topp_sample(row, 2, 1.0, 1.0, [0.0])["ids"][0].tolist() == [1, 2]
    assert oracle.topk_topp_sample(row, 4, 1.0, 1.0, [0.0])["ids"][0].tolist() == [1, 2, 4, 3]
    assert oracle.topk_topp_sample(row, 5, 1.0, 1.0, [0.0])["ids"][0].tolist() == [1, 2, 4, 3, 0]


def test_k1_is_first_argmax():
    x, u = synth.sampler_inputs(6, 3000, seed=11, grid=0.5)
    got = oracle.topk_topp_sample(x, 1, 0.3, 0.8, u)
    assert np.array_equal(got["sampled"], np.argmax(x.astype(np.float32), axis=1))
    assert np.all(got["kept"] == 1) and np.all(got["probs"][:, 0] == 1.0)


def test_tiny_top_p_keeps_only_the_first():
    x, u = synth.sampler_inputs(4, 2000, seed=12)
    got = oracle.topk_topp_sample(x, 20, 1e-6, 1.0, u)
    assert np.all(got["kept"] == 1) and np.array_equal(got["sampled"], got["ids"][:, 0])


def test_scale_and_shift_invariance():
    # Integer logits in [-20, 20]: doubling and adding 4 are exact in fp16.
    rng = np.random.default_rng(3)
    x = rng.integers(-20, 21, (5, 700)).astype(np.float16)
    u = rng.random(5)
    a = oracle.topk_topp_sample(x, 24, 0.9, 1.25, u)
    b = oracle.topk_topp_sample((x * 2).astype(np.float16), 24, 0.9, 2.5, u)
    s = oracle.topk_topp_sample((x + 4).astype(np.float16), 24, 0.9, 1.25, u)
    for o in (b, s):
        assert np.array_equal(a["ids"], o["ids"]) and np.array_equal(a["kept"], o["kept"])
        assert np.array_equal(a["rank"], o["rank"])
        np.testing.assert_allclose(a["probs"], o["probs"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=1e-14)
    np.testing.assert_allclose(s["lse"], a["lse"] + 4 / 1.25, rtol=1e-14)


def test_vocabulary_permutation():
    # Distinct values, so the ranking has no ties: permuting the positions
    # permutes the ids and changes nothing else.
    rng = np.random.default_rng(5)
    V = 1024
    row = ((rng.permutation(V) - 512) / 64.0).astype(np.float16)[None, :]   # distinct multiples of 1/64
    perm = rng.permutation(V)
    a = oracle.topk_topp_sample(row, 32, 0.8, 0.9, [0.37])
    b = oracle.topk_topp_sample(row[:, perm], 32, 0.8, 0.9, [0.37])
    assert np.array_equal(perm[b["ids"][0]], a["ids"][0])      # position i of b holds id perm[i]
    assert a["kept"][0] == b["kept"][0] and a["rank"][0] == b["rank"][0]
    np.testing.assert_array_equal(a["probs"], b["probs"])


def test_lse_matches_scipy():
    x, u = synth.sampler_inputs(3, 5000, seed=13)
    for T in (0.6, 1.0, 1.7):
        got = oracle.topk_topp_sample(x, 8, 0.95, T, u)
        want = logsumexp(x.astype(np.float64) / float(np.float32(T)), axis=1)
        np.testing.assert_allclose(got["lse"], want, rtol=1e-13)


def test_inverse_cdf_frequencies():
    # Uniforms at the midpoints of N equal cells: each rank is drawn for a
    # share of the cells equal to its probability, within one cell.
    x, _ = synth.sampler_inputs(1, 4000, seed=14, boosted=30, boost=(3.0, 6.0))
    N = 100_000
    u = (np.arange(N) + 0.5) / N
    got = oracle.topk_topp_sample(np.repeat(x, N, axis=0)[:1], 40, 0.9, 1.0, u[:1])
    probs = got["probs"][0]
    kept = got["kept"][0]
    assert 1 < kept < 40
    cdf = np.cumsum(probs[:kept])
    ranks = np.minimum(np.searchsorted(cdf, u, side="right"), kept - 1)
    # The oracle's own draw at a few of these uniforms agrees with the sweep.
    for i in (0, N // 3, N // 2, N - 1):
        r = oracle.topk_topp_sample(x, 40, 0.9, 1.0, [u[i]])["rank"][0]
        assert r == ranks[i]
    freq = np.bincount(ranks, minlength=kept) / N
    assert np.all(np.abs(freq - probs[:kept]) <= 1.0 / N + 1e-12)


def test_synth_sampler_inputs_shape_and_determinism():
    x1, u1 = synth.sampler_inputs(3, 1000, seed=2)
    x2, u2 = synth.sampler_inputs(3, 1000, seed=2)
    assert x1.dtype == np.float16 and x1.shape == (3, 1000) and u1.dtype == np.float32
    assert np.array_equal(x1.view(np.uint16), x2.view(np.uint16)) and np.array_equal(u1, u2)
    assert np.all((u1 >= 0) & (u1 < 1)) and np.isfinite(x1.astype(np.float32)).all()
    xt, _ = synth.sampler_inputs(2, 5000, seed=2, grid=0.5)
    assert len(np.unique(xt[0])) < 100                   # coarse grid: many equal logits
