"""CPU oracle for the weight-only-int4 GEMM path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU library: the two share no code.  Inputs come from
``synth`` (random draws only).

Everything here is plain numpy, written for a reader to check against the
pages by eye: float64 for floating-point results, exact integers for integer
stages.  Sources (pages from the open web, cited by title and section):

* "What this repo does that stock vLLM doesn't" (the project's
  optimisations page), "In full" item 1: lm_head and embedding tables are
  requantised to int8 group-128 with a round-trip error of about 0.6%.
* same page, "In full" item 2: a dequant-on-gather kernel serves the int8
  embedding table.
* same page, "In full" item 4: W4A8 keeps the int4 weights, quantises the
  activations to int8 per token and runs the product on int8 matrix units;
  group scales are signed (about half negative) and must be honoured.
* same page, "int8 prefill for single-user mode": prefill runs the same W4A8
  path; decode at batch 64 and speculative verify run W4A16.
* same page, "In full" item 6: the verify step's sampler takes a small top-k
  (k <= 64) by selection rather than a sort of the whole 248k-wide row, with
  a softmax spread over many workgroups.
* the project README, "What each step buys": the body is W4A16 (int4 weights,
  16-bit activations) and the lm_head/embedding tables are int8.

Readings where the pages are silent (each is also listed in the design notes):
per-token scale = fp32(absmax) / 127 with IEEE fp32 division; code =
round-half-even(fp32(x) / scale) clamped to [-127, 127]; an all-zero row gets
scale 0 and codes 0; weight groups are 128 wide along K; W4A16 dequantisation
is exact (the oracle does not round q*s to fp16); out-of-range token ids give
zero rows.

Parity pins: every function below is pinned in ``tests/test_oracle_*.py`` by
brute force with exact rationals, closed forms and invariants.  One step has
no page behind it: ``rmsnorm`` (the norm whose output the fused quantiser
takes; the pages name no norm).  Its definition is a reading (the float64
value rounded once to fp16), pinned by a 60-digit decimal evaluation,
closed forms and an exact scale invariance, and is marked "parity unpinned"
as to the pages.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

__all__ = [
    "GROUP", "quant_act", "partials", "ref_w4a8", "ref_w4a16", "quant_table",
    "ref_gather", "ref_w8a16", "fp16_bounds", "FP16_MAX_RATIO", "FP16_FROB",
    "rmsnorm", "rmsnorm_quant", "ref_verify_attention",
    "topk_topp_sample",
]

# Tolerance for fp16 outputs against the float64 reference:
# max |y - ref| <= 2^-10 * max |ref|  and  ||y - ref||_F / ||ref||_F <= 5e-4.
FP16_MAX_RATIO = 2.0 ** -10
FP16_FROB = 5e-4


def quant_act(x):
    """Per-token int8 quantisation of fp16 activations.

    "In full" item 4 of the optimisations page: activations are quantised to
    int8 per token.  Reading: for token row m,
        s[m] = fp32(max_k |x[m,k]|) / 127           (IEEE fp32 division)
        q[m,k] = clamp(rne(fp32(x[m,k]) / s[m]), -127, 127)
    and a row whose absmax is 0 gets s = 0, q = 0.

    Returns (q int8 [M,K], s float32 [M]).
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float32)
    M, K = xf.shape
    q = np.zeros((M, K), np.int8)
    s = np.zeros(M, np.float32)
    if M == 0 or K == 0:
        return q, s
    a = np.abs(xf).max(axis=1)
    nz = a > 0
    s[nz] = a[nz] / np.float32(127.0)
    if nz.any():
        quot = xf[nz] / s[nz][:, None]            # float32 / float32: IEEE
        q[nz] = np.clip(np.rint(quot), -127, 127).astype(np.int8)
    return q, s


def rmsnorm(x, w, eps):
    """RMSNorm of fp16 rows with an fp16 weight, rounded once to fp16.

    Parity unpinned as to the pages, which name no norm: this is the plain
    reading of the norm whose output a fused quantiser would take.  For row
    m of length H,
        ss[m]   = sum_h x[m, h]^2                  (exactly rounded: math.fsum)
        r[m]    = 1 / sqrt(ss[m] / H + eps)        (float64, eps as fp32; r = 0 where that is 0)
        y[m, h] = fp16(x[m, h] * r[m] * w[h])      (float64 product, one rounding to fp16)
    Every float64 step is within a few units of 2^-53 of the exact value, so
    y is the correctly rounded fp16 of x * w / sqrt(mean(x^2) + eps) except
    where that value lies within about 1e-15 (relative) of a point halfway
    between two fp16 numbers.  No summation order is part of the definition:
    any evaluation close enough to the exact value is a correct reading.
    Returns y as float16 [M, H].
    """
    import math
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    wf = np.asarray(w, dtype=np.float16).astype(np.float64)
    M, H = xf.shape
    e = float(np.float32(eps))                      # eps is an fp32 argument
    y = np.zeros((M, H), np.float64)
    for m in range(M):
        ss = math.fsum((xf[m] * xf[m]).tolist())    # squares of fp16 values are exact in float64
        t = ss / H + e
        if t > 0:
            y[m] = xf[m] * (1.0 / math.sqrt(t)) * wf
    return y.astype(np.float16)


def rmsnorm_quant(x, w, eps):
    """The fused normalise-and-quantise step: y = rmsnorm(x, w, eps), then the
    per-token int8 quantisation of y.  Returns (y fp16, q int8, s float32)."""
    y = rmsnorm(x, w, eps)
    q, s = quant_act(y)
    return y, q, s


def ref_verify_attention(q, k, v):
    """Causal multi-query attention of the speculative-verify step, float64.

    "In full" item 6 of the optimisations page: the verify step runs attention
    for several query tokens of one sequence at once (24 query heads,
    head_dim 256 there).  Reading: the T query tokens are the last T
    positions of the cache, each sees the cache up to and including its own
    position, and query heads share key/value heads in groups of
    G = Hq / Hkv (head h uses key/value head h // G):
        s[t, h, p] = q[t, h] . k[p, h // G] / sqrt(D),   p <= L - T + t
        o[t, h]    = sum_p softmax_p(s[t, h, :]) v[p, h // G]
    q: [T, Hq, D], k and v: [L, Hkv, D] (fp16 values).  Returns float64 [T, Hq, D].
    """
    qf = np.asarray(q, dtype=np.float16).astype(np.float64)
    kf = np.asarray(k, dtype=np.float16).astype(np.float64)
    vf = np.asarray(v, dtype=np.float16).astype(np.float64)
    T, Hq, D = qf.shape
    L, Hkv, _ = kf.shape
    G = Hq // Hkv
    visible = np.arange(L)[None, :] <= (L - T + np.arange(T))[:, None]      # [T, L]
    out = np.empty((T, Hq, D), np.float64)
    for h in range(Hq):
        s = qf[:, h, :] @ kf[:, h // G, :].T / np.sqrt(D)                  # [T, L]
        s = np.where(visible, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ vf[:, h // G, :]
    return out


def topk_topp_sample(logits, k, top_p, temperature, u):
    """Small-k top-k / top-p sampling of one step's logits, float64.

    "In full" item 6 of the optimisations page: with k <= 64 known up front,
    the top-k mask is a plain top-k selection instead of a sort of the whole
    248k-wide row, the softmax over the row runs on many workgroups, and the
    target and the drafts sample from the same truncated support.  Readings
    where the page is silent:
      * z = x / T with the temperature T given as fp32; the top-k are the k
        largest logits, larger value first and, among equal values, the
        lower vocabulary index first (exactly k, ties broken by index);
      * mass[j] = softmax over those k of z (j = 0 is the largest);
      * top-p keeps rank j when the mass ranked before it is below p:
        sum_{i<j} mass[i] < p (so rank 0 is always kept);
      * probs = mass renormalised over the kept ranks, 0 elsewhere;
      * the sample is the smallest kept rank j with sum_{i<=j} probs[i] > u
        for the caller's uniform u in [0, 1) (the last kept rank if none);
      * lse = log sum_v exp(z_v) over the whole row (the full softmax's
        normaliser, which needs a finite row maximum).
    logits fp16 [R, V]; u [R].  Returns a dict of float64/integer arrays:
    ids [R, k] (int64), mass and probs [R, k], kept [R], sampled [R] (the
    vocabulary id drawn), rank [R] (its rank) and lse [R].
    """
    x = np.asarray(logits, dtype=np.float16)
    R, V = x.shape
    xf = x.astype(np.float64)
    T = float(np.float32(temperature))
    uf = np.asarray(u, dtype=np.float64).reshape(R)
    ids = np.empty((R, k), np.int64)
    mass = np.empty((R, k), np.float64)
    probs = np.zeros((R, k), np.float64)
    kept = np.empty(R, np.int64)
    rank = np.empty(R, np.int64)
    lse = np.empty(R, np.float64)
    for r in range(R):
        order = np.lexsort((np.arange(V), -xf[r]))      # value descending, then index ascending
        top = order[:k]
        ids[r] = top
        z = xf[r, top] / T
        e = np.exp(z - z[0])
        mass[r] = e / e.sum()
        before = np.concatenate(([0.0], np.cumsum(mass[r])[:-1]))
        kept[r] = int(np.count_nonzero(before < top_p))
        probs[r, :kept[r]] = mass[r, :kept[r]] / mass[r, :kept[r]].sum()
        cdf = np.cumsum(probs[r, :kept[r]])
        rank[r] = min(int(np.count_nonzero(cdf <= uf[r])), kept[r] - 1)
        zr = xf[r] / T
        zmax = zr.max()
        lse[r] = zmax + np.log(np.exp(zr - zmax).sum())
    sampled = ids[np.arange(R), rank]
    return dict(ids=ids, mass=mass, probs=probs, kept=kept, rank=rank, sampled=sampled, lse=lse)


def partials(q, codes):
    """Exact per-group integer partials of the W4A8 contraction.

        P[m, n, g] = sum_{j < 128} q[m, 128 g + j] * codes[n, 128 g + j]

    ("In full" item 4: the int8 x int4 product accumulates in 32-bit integers
    per 128-wide weight group before the group scale is applied.)
    Computed as one float64 matmul per group; every product and partial sum
    is an integer below 2^53, so the result is exact.  Returns int64
    [M, N, G].
    """
    q = np.asarray(q)
    codes = np.asarray(codes)
    M, K = q.shape
    N = codes.shape[0]
    G = K // GROUP
    P = np.empty((M, N, G), np.int64)
    qf = q.astype(np.float64)
    cf = codes.astype(np.float64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        P[:, :, g] = (qf[:, sl] @ cf[:, sl].T).astype(np.int64)
    return P


def ref_w4a8(x, codes, scales, q=None, s=None):
    """float64 reference of the W4A8 GEMM.

        y[m, n] = s[m] * sum_g P[m, n, g] * scales[n, g]

    with (q, s) = quant_act(x) and P = partials(q, codes).  The group scale
    keeps its sign ("In full" item 4: about half the AutoRound group scales
    are negative and reading them as unsigned produced garbage).
    Returns float64 [M, N].
    """
    if q is None or s is None:
        q, s = quant_act(x)
    codes = np.asarray(codes)
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    M, K = q.shape
    N = codes.shape[0]
    G = K // GROUP
    acc = np.zeros((M, N), np.float64)
    qf = q.astype(np.float64)
    cf = codes.astype(np.float64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        Pg = qf[:, sl] @ cf[:, sl].T                # exact integers
        acc += Pg * sc[:, g][None, :]
    return acc * s.astype(np.float64)[:, None]


def _dequant_rows(codes, scales):
    """float64 dequantised weight rows w[n, k] = codes[n, k] * scales[n, k // 128] (exact)."""
    cf = np.asarray(codes).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    return cf * np.repeat(sc, GROUP, axis=1)


def ref_w4a16(x, codes, scales, chunk=8192):
    """float64 reference of the W4A16 GEMM (project README, "What each step
    buys": int4 body weights with 16-bit activations).

        y[m, n] = sum_k x[m, k] * codes[n, k] * scales[n, k // 128]

    The dequantised weight is kept exact; the GPU's rounding of q*s to fp16
    (if it does so) is part of the error the fp16 tolerance must absorb.
    Computed in N chunks to bound host memory.  Returns float64 [M, N].
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    codes = np.asarray(codes)
    N = codes.shape[0]
    y = np.empty((xf.shape[0], N), np.float64)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        y[:, n0:n1] = xf @ _dequant_rows(codes[n0:n1], scales[n0:n1]).T
    return y


def quant_table(src_bits):
    """Requantise a bf16 table to int8 with one fp16 scale per 128 values of a row.

    "In full" item 1 of the optimisations page: both vocabulary matrices are
    requantised offline to int8 group-128.  Reading: per row v and group g,
        a = max |fp32(src)| over the group
        S[v, g] = fp16(fp32(a) / 127)
        Q[v, h] = clamp(rne(fp32(src[v, h]) / fp32(S[v, h // 128])), -127, 127)
    dividing by the stored fp16 scale so dequantisation uses the scale that
    is kept; a group with S == 0 gets Q = 0.

    ``src_bits``: uint16 bf16 bit patterns [V, H].  Returns (Q int8 [V,H],
    S fp16 [V, H/128]).
    """
    b = np.asarray(src_bits, dtype=np.uint16)
    V, H = b.shape
    G = H // GROUP
    f = (b.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(V, G, GROUP)
    a = np.abs(f).max(axis=2)
    S = (a / np.float32(127.0)).astype(np.float16)
    Sf = S.astype(np.float32)
    Q = np.zeros((V, G, GROUP), np.int8)
    nz = Sf > 0
    if nz.any():
        Q[nz] = np.clip(np.rint(f[nz] / Sf[nz][:, None]), -127, 127).astype(np.int8)
    return Q.reshape(V, H), S


def ref_gather(ids, Q, S):
    """Dequant-on-gather embedding lookup ("In full" item 2).

        out[t, h] = fp16(fp32(Q[id_t, h]) * fp32(S[id_t, h // 128]))

    The fp32 product of an int8 code and an fp16 scale is exact, so there is
    a single rounding.  Ids outside [0, V) give a zero row.  Returns fp16
    [T, H].
    """
    ids = np.asarray(ids).astype(np.int64)
    Q = np.asarray(Q)
    V, H = Q.shape
    out = np.zeros((ids.shape[0], H), np.float16)
    ok = (ids >= 0) & (ids < V)
    if ok.any():
        rows = ids[ok]
        prod = Q[rows].astype(np.float32) * np.repeat(
            np.asarray(S, dtype=np.float16)[rows].astype(np.float32), GROUP, axis=1)
        out[ok] = prod.astype(np.float16)
    return out


def ref_w8a16(x, Q, S, rows=None, chunk=8192):
    """float64 reference of the int8-weight lm_head product over the same
    table the gather reads ("In full" items 1 and 5: a 248k-row int8 head).

        y[m, v] = sum_h x[m, h] * Q[v, h] * S[v, h // 128]

    ``rows`` optionally restricts v to a subset (in that order).  Returns
    float64 [M, len(rows) or V].
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    Q = np.asarray(Q)
    S = np.asarray(S)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        return xf @ _dequant_rows(Q[rows], S[rows]).T
    V = Q.shape[0]
    y = np.empty((xf.shape[0], V), np.float64)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        y[:, v0:v1] = xf @ _dequant_rows(Q[v0:v1], S[v0:v1]).T
    return y


def fp16_bounds(y, ref):
    """Error of fp16 outputs against a float64 reference, both bounds.

    Returns a dict with max_abs_err, max_abs_ref, max_ratio (err / max|ref|),
    frob (relative Frobenius error) and ok (both bounds hold).
    """
    y64 = np.asarray(y).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = y64 - r
    max_err = float(np.abs(err).max()) if err.size else 0.0
    max_ref = float(np.abs(r).max()) if r.size else 0.0
    nr = float(np.linalg.norm(r))
    frob = float(np.linalg.norm(err) / nr) if nr > 0 else float(np.linalg.norm(err))
    ratio = max_err / max_ref if max_ref > 0 else max_err
    ok = bool(np.isfinite(y64).all()) and ratio <= FP16_MAX_RATIO and frob <= FP16_FROB
    return dict(max_abs_err=max_err, max_abs_ref=max_ref, max_ratio=ratio, frob=frob, ok=ok)
