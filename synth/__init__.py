"""Seeded synthetic inputs for the weight-only-int4 GEMM path.

This module only draws random numbers and stores them in the formats the
path consumes (int8 codes in [-8, 7], fp16 group scales, fp16 activations,
bf16 table source values, int32 token ids).  It holds none of the path's
arithmetic: no quantisation, no dequantisation, no contraction.  Both the
CPU oracle (``oracle/``) and the GPU path's tests and benchmark take their
inputs from here, so the two sides see byte-identical tensors.

Every array is produced in row chunks of ``CHUNK_ROWS`` rows.  Chunk ``c`` of
stream ``s`` under seed ``seed`` is drawn from
``numpy.random.default_rng(SeedSequence([seed, s, c]))`` (PCG64), so the bytes
depend only on (seed, shape) and not on how many threads fill them.

Value distributions follow the workloads the pages describe:

* weights: AutoRound symmetric int4 with signed group scales, about half of
  them negative (page "What this repo does that stock vLLM doesn't",
  "In full" item 4).  Codes are uniform on [-8, 7]; |scale| is log-uniform on
  [1e-3, 1e-2]; the sign is negative with probability 0.5; group size 128
  along K.
* activations: N(0, sigma) with each element independently an outlier with
  probability p, multiplied by a factor, then rounded to fp16.
* vocabulary table source: bf16 values drawn from N(0, 0.02), the format the
  pages requantise to int8 group-128 ("In full" item 1).
* token ids: uniform on [0, V).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GROUP = 128
CHUNK_ROWS = 1024

# Stream ids keep the draws for different tensors of one seed independent.
_S_CODES, _S_SMAG, _S_SSIGN, _S_ACT, _S_OUTL, _S_TABLE, _S_IDS, _S_DRAFT, _S_ATTN, _S_LOGIT, _S_UNIF = range(1, 12)

_LOG_SMIN = float(np.log(1e-3))
_LOG_SMAX = float(np.log(1e-2))


def _rng(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), stream, chunk]))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_rows(rows: int, fn) -> None:
    """Call fn(chunk_index, row0, row1) for every row chunk, on a thread pool.

    numpy's generators and ufuncs release the GIL on bulk fills, so chunks
    run in parallel; results do not depend on the pool size.
    """
    chunks = [(c, c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS))
              for c in range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS)]
    if len(chunks) <= 1:
        for c in chunks:
            fn(*c)
        return
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda c: fn(*c), chunks))


def weights(N: int, K: int, seed: int):
    """int4 codes [N, K] (int8 storage, values in [-8, 7]) and signed fp16
    group scales [N, K // 128]."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    codes = np.empty((N, K), np.int8)
    scales = np.empty((N, G), np.float16)

    def fill(c, r0, r1):
        codes[r0:r1] = _rng(seed, _S_CODES, c).integers(-8, 8, size=(r1 - r0, K), dtype=np.int8)
        mag = np.exp(_rng(seed, _S_SMAG, c).uniform(_LOG_SMIN, _LOG_SMAX, size=(r1 - r0, G)))
        neg = _rng(seed, _S_SSIGN, c).random((r1 - r0, G)) < 0.5
        scales[r0:r1] = np.where(neg, -mag, mag).astype(np.float16)

    _fill_rows(N, fill)
    return codes, scales


def acts(M: int, K: int, sigma: float, p: float = 0.0, factor: float = 1.0, seed: int = 0):
    """fp16 activations [M, K]: N(0, sigma), each element an outlier (times
    ``factor``) with probability ``p``."""
    x = np.empty((M, K), np.float16)

    def fill(c, r0, r1):
        v = _rng(seed, _S_ACT, c).normal(0.0, sigma, size=(r1 - r0, K))
        if p > 0.0:
            mask = _rng(seed, _S_OUTL, c).random((r1 - r0, K)) < p
            v[mask] *= factor
        x[r0:r1] = v.astype(np.float16)

    _fill_rows(M, fill)
    return x


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def table_source(V: int, H: int, seed: int, std: float = 0.02) -> np.ndarray:
    """bf16 source values [V, H] from N(0, std), returned as uint16 bit
    patterns (numpy has no bf16 dtype)."""
    out = np.empty((V, H), np.uint16)

    def fill(c, r0, r1):
        v = _rng(seed, _S_TABLE, c).standard_normal(size=(r1 - r0, H), dtype=np.float32)
        v *= np.float32(std)
        out[r0:r1] = bf16_bits_from_f32(v)

    _fill_rows(V, fill)
    return out


def token_ids(T: int, V: int, seed: int) -> np.ndarray:
    """int32 token ids uniform on [0, V)."""
    return _rng(seed, _S_IDS, 0).integers(0, V, size=T, dtype=np.int64).astype(np.int32)


def attention_inputs(T: int, Hq: int, Hkv: int, L: int, seed: int, D: int = 256):
    """fp16 queries [T, Hq, D] and key/value caches [L, Hkv, D], all N(0, 1)."""
    rng = _rng(seed, _S_ATTN, 0)
    q = rng.standard_normal((T, Hq, D), dtype=np.float32).astype(np.float16)
    k = rng.standard_normal((L, Hkv, D), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((L, Hkv, D), dtype=np.float32).astype(np.float16)
    return q, k, v


def sampler_inputs(R: int, V: int, seed: int, sigma: float = 2.0, boosted: int = 8, boost=(6.0, 12.0),
                   grid: float = 0.0):
    """fp16 logits [R, V] and uniforms u [R] (float32, in [0, 1)) for the
    sampler.  Logits are N(0, sigma) with ``boosted`` random ids per row
    raised by U(boost) (a few likely tokens, as in a language model's
    output), rounded to fp16; with ``grid`` > 0 they are first rounded to
    multiples of ``grid``, which makes equal logits common (tie cases)."""
    x = np.empty((R, V), np.float16)

    def fill(c, r0, r1):
        rng = _rng(seed, _S_LOGIT, c)
        v = rng.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(sigma)
        for i in range(r1 - r0):
            hot = rng.choice(V, size=min(boosted, V), replace=False)
            v[i, hot] += rng.uniform(boost[0], boost[1], size=hot.size).astype(np.float32)
        if grid > 0:
            v = np.round(v / np.float32(grid)) * np.float32(grid)
        x[r0:r1] = v.astype(np.float16)

    _fill_rows(R, fill)
    u = _rng(seed, _S_UNIF, 0).random(R, dtype=np.float32)
    return x, u


def draft_ids(D: int, V: int, seed: int) -> np.ndarray:
    """A draft vocabulary: D distinct ids of [0, V), ascending, int64.  A
    stand-in of the same size for a list counted over a model's outputs."""
    return np.sort(_rng(seed, _S_DRAFT, 0).choice(V, size=D, replace=False)).astype(np.int64)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds: weights use ``seed``, activations ``seed + 100``,
# the vocabulary table ``seed + 200`` and token ids ``seed + 300``.
# ---------------------------------------------------------------------------
CONFIGS = {
    "tiny_w4a8": dict(op="w4a8", M=4, K=256, N=256, sigma=1.0, p=0.01, factor=20.0, seed=0),
    "decode_w4a8": dict(op="w4a8", M=64, K=5120, N=5120, sigma=1.0, p=0.01, factor=20.0, seed=1),
    "verify_w4a16_m8": dict(op="w4a16", M=8, K=5120, N=34816, sigma=1.0, p=0.0, factor=1.0, seed=2),
    "verify_w4a16_m16": dict(op="w4a16", M=16, K=5120, N=34816, sigma=1.0, p=0.0, factor=1.0, seed=2),
    "prefill_w4a8": dict(op="w4a8", M=4096, K=17408, N=5120, sigma=0.5, p=0.005, factor=30.0, seed=3),
    "vocab_int8": dict(op="vocab", V=248320, H=5120, T=64, M=64, sigma=1.0, p=0.0, factor=1.0,
                       table_std=0.02, seed=4),
    # lm_head variants: an int4 head (W4A16 over the 248,320 rows) and a
    # 40,960-row draft head gathered once from the int8 table of vocab_int8
    "lm_head_w4a16": dict(op="w4a16", M=64, K=5120, N=248320, sigma=1.0, p=0.0, factor=1.0, seed=5),
    "draft_head_int8": dict(op="draft", V=248320, H=5120, D=40960, M=1, sigma=1.0, p=0.0, factor=1.0,
                            table_std=0.02, seed=4),
    # the verify step's attention, one layer: 1 + 4 draft tokens, 24 query
    # heads over 4 key/value heads (the key/value head count is a reading),
    # head_dim 256, the two context lengths the pages measure
    "verify_attention": dict(op="attention", T=5, Hq=24, Hkv=4, L=(1536, 16384), seed=6),
    # the sampler after the lm_head: 248,320-wide fp16 logit rows, the
    # model's default sampling (temperature 1.0, top-p 0.95, top-k 20), for
    # one row, a 1 + 15 verify block and 64 concurrent sequences
    "sampler": dict(op="sampler", V=248320, R=(1, 16, 64), k=20, top_p=0.95, T=1.0, seed=7),
}


def gemm_inputs(cfg: dict, M: int | None = None):
    """(x fp16 [M,K], codes int8 [N,K], scales fp16 [N,K/128]) for a GEMM config."""
    M = cfg["M"] if M is None else M
    codes, scales = weights(cfg["N"], cfg["K"], cfg["seed"])
    x = acts(M, cfg["K"], cfg["sigma"], cfg["p"], cfg["factor"], cfg["seed"] + 100)
    return x, codes, scales
