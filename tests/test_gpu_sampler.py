"""GPU parity of sample_topk_topp against the oracle (oracle.topk_topp_sample).

What is unique is compared exactly: the top-k ids and their order (fp16
comparisons with ties by lower id, no arithmetic).  The rest is float:
  * probabilities: the kernel's fp32 softmax (exp2 of fp32 differences, k
    terms summed) against float64, rtol 2e-5 / atol 1e-7: the exponent's
    argument carries a relative error of a few 1e-7, which is at most about
    5e-6 relative on any mass above 1e-12 of the largest;
  * the top-p count and the draw are integer decisions taken on fp32 sums:
    they must equal the oracle's unless the oracle's own cumulative mass at
    the boundary between the two answers lies within 1e-5 of p (or of u),
    where both answers are correct readings of the definition;
  * lse: |err| <= 2e-5 + 1e-6 |lse| (fp32 sums over up to 248k terms).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
AMBIG = 1e-5


@pytest.fixture(scope="module")
def qg():
    import spec_verify_amd
    return spec_verify_amd


def run(qg, x, u, k, p, T, ld=None):
    R, V = x.shape
    if ld is None or ld == V:
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    else:
        # Rows of a wider buffer; the padding holds large logits that must
        # never be picked.
        buf = np.full((R, ld), 60000.0, np.float16)
        buf[:, :V] = x
        xd = torch.from_numpy(buf).to(DEV)
    ud = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).to(DEV)
    out = qg.sample_topk_topp(xd, ud, k, p, T, V=V)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check(got, want, u, p):
    ids, probs, kept, sampled, lse = got
    R, k = want["ids"].shape
    assert np.array_equal(ids.astype(np.int64), want["ids"]), "top-k ids differ"
    for r in range(R):
        m = want["mass"][r]
        before = np.concatenate(([0.0], np.cumsum(m)[:-1]))
        kg, kw = int(kept[r]), int(want["kept"][r])
        assert 1 <= kg <= k
        if kg != kw:
            lo, hi = min(kg, kw), max(kg, kw)
            assert np.all(np.abs(before[lo:hi] - p) <= AMBIG), (r, kg, kw, before[lo:hi], p)
        ref = np.zeros(k)
        ref[:kg] = m[:kg] / m[:kg].sum()
        np.testing.assert_allclose(probs[r], ref, rtol=2e-5, atol=1e-7, err_msg=f"row {r}")
        cdf = np.cumsum(ref[:kg])
        rank_ref = min(int(np.count_nonzero(cdf <= float(u[r]))), kg - 1)
        pos = np.nonzero(ids[r] == sampled[r])[0]
        assert pos.size == 1 and pos[0] < kg, (r, sampled[r])
        rank_got = int(pos[0])
        if rank_got != rank_ref:
            lo, hi = min(rank_got, rank_ref), max(rank_got, rank_ref)
            assert np.all(np.abs(cdf[lo:hi] - float(u[r])) <= AMBIG), (r, rank_got, rank_ref)
    err = np.abs(lse.astype(np.float64) - want["lse"])
    assert np.all(err <= 2e-5 + 1e-6 * np.abs(want["lse"])), err.max()


@pytest.mark.parametrize("R,k,p,T", [(1, 20, 0.95, 1.0), (16, 20, 0.95, 1.0), (64, 20, 0.95, 1.0),
                                     (32, 64, 0.8, 0.7), (16, 64, 0.5, 1.5), (64, 1, 0.9, 1.0)])
def test_vocabulary_width_rows(qg, R, k, p, T):
    # The 248,320-wide rows of the lm_head (default sampling: T 1.0, top-p
    # 0.95, top-k 20; and other settings).
    x, u = synth.sampler_inputs(R, 248320, seed=40 + R + k)
    check(run(qg, x, u, k, p, T), oracle.topk_topp_sample(x, k, p, T, u), u, p)


@pytest.mark.parametrize("V,k", [(1, 1), (7, 7), (63, 20), (64, 64), (100, 64), (2049, 33), (2048 * 3 + 5, 64),
                                 (40967, 20), (8192 * 256, 64),
                                 # the widest row: 2048 chunks of 8 candidates (the candidate cap)
                                 (2 ** 24 - 8, 8)])
def test_ragged_widths(qg, V, k):
    R = 3 if V < 1_000_000 else 1
    x, u = synth.sampler_inputs(R, V, seed=V % 1000, boosted=min(8, V))
    ld = (V + 7) // 8 * 8
    check(run(qg, x, u, k, 0.9, 1.0, ld=ld), oracle.topk_topp_sample(x, k, 0.9, 1.0, u), u, 0.9)


def test_most_rows(qg):
    # R = 65536, the most rows one call takes (narrow rows: one chunk each).
    x, u = synth.sampler_inputs(65536, 64, seed=11)
    check(run(qg, x, u, 20, 0.9, 1.0), oracle.topk_topp_sample(x, 20, 0.9, 1.0, u), u, 0.9)


@pytest.mark.parametrize("grid", [0.5, 2.0])
def test_ties_break_by_lower_id(qg, grid):
    x, u = synth.sampler_inputs(8, 248320, seed=50, grid=grid)
    check(run(qg, x, u, 64, 0.95, 1.0), oracle.topk_topp_sample(x, 64, 0.95, 1.0, u), u, 0.95)


def test_constant_and_minus_infinity_rows(qg):
    V = 20000
    x = np.zeros((4, V), np.float16)
    x[0] = 1.25                                      # all equal: ids 0 .. k-1, uniform mass
    x[1, :9000] = -np.inf                            # whole chunks of -inf
    x[1, 9000:] = synth.sampler_inputs(1, V - 9000, seed=51)[0][0]
    x[2] = synth.sampler_inputs(1, V, seed=52)[0][0]
    x[2, ::3] = -np.inf
    x[3] = -np.inf
    x[3, 12345] = 3.0                                # one finite logit
    u = np.array([0.3, 0.999999, 0.0, 0.5], np.float32)
    got = run(qg, x, u, 16, 0.9, 1.0)
    want = oracle.topk_topp_sample(x, 16, 0.9, 1.0, u)
    assert np.array_equal(got[0][0], np.arange(16))
    assert got[3][3] == 12345 and got[2][3] == 1
    check(got, want, u, 0.9)


@pytest.mark.parametrize("p", [1.0, 1e-6])
def test_top_p_extremes(qg, p):
    x, u = synth.sampler_inputs(8, 50000, seed=53)
    got = run(qg, x, u, 32, p, 1.0)
    assert np.all(got[2] == (32 if p == 1.0 else 1))
    check(got, oracle.topk_topp_sample(x, 32, p, 1.0, u), u, p)


def test_repeat_runs_are_bit_identical(qg):
    x, u = synth.sampler_inputs(16, 248320, seed=54)
    a = run(qg, x, u, 20, 0.95, 1.0)
    b = run(qg, x, u, 20, 0.95, 1.0)
    for s, t in zip(a, b):
        assert np.array_equal(s.view(np.uint32), t.view(np.uint32))


def test_same_support_for_target_and_draft_rows(qg):
    # Identical rows with different uniforms: the same ids, kept count and
    # probabilities (the truncated support is a function of the row only).
    x, _ = synth.sampler_inputs(1, 248320, seed=55)
    xx = np.repeat(x, 5, axis=0)
    u = np.array([0.0, 0.2, 0.4, 0.6, 0.8], np.float32)
    ids, probs, kept, sampled, lse = run(qg, xx, u, 20, 0.95, 1.0)
    assert np.all(ids == ids[0]) and np.all(kept == kept[0]) and np.all(probs == probs[0])
    ranks = [int(np.nonzero(ids[0] == s)[0][0]) for s in sampled]
    assert ranks == sorted(ranks)                    # the draw is monotone in u


def test_many_equal_candidates_take_the_radix_select(qg):
    # A constant row of 300,000 logits at k = 64: every chunk's candidates
    # tie, so both passes see far more than 512 survivors of the threshold
    # and select by radix digits; the answer is ids 0 .. 63 in order.
    V = 300_000
    x = np.full((2, V), -0.75, np.float16)
    x[1, ::7] = 0.5                                    # ties among every 7th id
    u = np.array([0.4, 0.9], np.float32)
    got = run(qg, x, u, 64, 0.7, 1.0)
    assert np.array_equal(got[0][0], np.arange(64))
    assert np.array_equal(got[0][1], np.arange(64) * 7)
    check(got, oracle.topk_topp_sample(x, 64, 0.7, 1.0, u), u, 0.7)
