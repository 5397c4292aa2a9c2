"""Pins for the oracle's int8 vocabulary table: requantisation, gather and
the page figures for its format (CPU only).

"In full" items 1 and 2 of the optimisations page: both vocabulary matrices
are requantised from bf16 to int8 group-128 (about 0.6% round-trip error) and
served by a dequant-on-gather kernel.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _roundtrip_error(src_bits, Q, S):
    f = synth.bf16_bits_to_f32(src_bits).astype(np.float64)
    deq = Q.astype(np.float64) * np.repeat(S.astype(np.float64), 128, axis=1)
    return np.linalg.norm(deq - f) / np.linalg.norm(f)


def test_quant_table_matches_exact_rationals():
    src = synth.table_source(6, 384, seed=50)
    src[2, :128] = 0                                   # an all-zero group
    Q, S = oracle.quant_table(src)
    vals = synth.bf16_bits_to_f32(src)
    for v in range(6):
        for g in range(3):
            eq, es = exact.quant_group(vals[v, g * 128:(g + 1) * 128])
            assert float(S[v, g]) == float(es)
            assert Q[v, g * 128:(g + 1) * 128].tolist() == eq
    assert S[2, 0] == 0 and not Q[2, :128].any()


def test_roundtrip_error_matches_page_and_closed_form():
    """Measured round-trip error is the pages' ~0.6%, and agrees with the
    uniform-rounding closed form sqrt(E[a^2] / (127^2 * 12)) / sigma where a is
    the absmax of 128 standard normals."""
    g = _golden()["int8_table_roundtrip_error"]
    src = synth.table_source(2048, 5120, seed=204)
    Q, S = oracle.quant_table(src)
    err = _roundtrip_error(src, Q, S)
    lo, hi = g["accept"]
    assert lo <= err <= hi, err
    from scipy import integrate, special
    # E[a^2] = int_0^inf 2 t (1 - F(t)) dt with F(t) = erf(t / sqrt 2)^128
    ea2, _ = integrate.quad(lambda t: 2 * t * (1 - special.erf(t / math.sqrt(2)) ** 128), 0, 12)
    closed = math.sqrt(ea2 / (127 ** 2 * 12))
    assert abs(err - closed) / closed < 0.03, (err, closed)


def test_every_nonzero_group_uses_code_127():
    src = synth.table_source(512, 5120, seed=205)
    Q, S = oracle.quant_table(src)
    gm = np.abs(Q.astype(np.int32)).reshape(512, 40, 128).max(axis=2)
    assert (gm[S != 0] == 127).all()
    assert (S > 0).all()


def test_gather_matches_exact_rounding_and_zero_rows():
    src = synth.table_source(50, 256, seed=51)
    Q, S = oracle.quant_table(src)
    S = S.copy()
    S[3, 1] = np.float16(3e-7)                        # product lands in fp16 subnormals
    ids = np.array([3, -1, 49, 50, 0, 3, 10 ** 6], np.int32)
    out = oracle.ref_gather(ids, Q, S)
    for t, i in enumerate(ids):
        if not 0 <= i < 50:
            assert not out[t].astype(np.float32).any()
            continue
        for h in range(256):
            want = exact.round_f16(int(Q[i, h]) * Fraction(float(S[i, h // 128])))
            assert float(out[t, h]) == float(want), (t, h)


def test_bf16_rounding_of_table_source_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(52)
    v = (rng.standard_normal(100000) * 0.02).astype(np.float32)
    # exact ties between two bf16 values, both parities
    v[:4] = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80C000], np.uint32).view(np.float32)
    ours = synth.bf16_bits_from_f32(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == theirs).all()


def test_page_figures_for_the_table_geometry():
    """V = 248,320 rows x 5,120 hidden: a 1.3 GB int8 head (plus group
    scales) and a 2.5 GB bf16 matrix, as the pages print."""
    g = _golden()
    cfg = synth.CONFIGS["vocab_int8"]
    V, H = cfg["V"], cfg["H"]
    assert V // 1000 == g["vocab_rows_thousands"]["value"]
    assert H % g["table_group"]["value"] == 0
    int8_gb = (V * H + V * (H // 128) * 2) / 1e9
    lo, hi = g["lm_head_int8_gb"]["accept"]
    assert lo <= int8_gb <= hi, int8_gb
    lo, hi = g["bf16_table_gb"]["accept"]
    assert lo <= V * H * 2 / 1e9 <= hi
