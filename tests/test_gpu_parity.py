"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer stages (activation codes, token scales, int32 group partials, the
gather and the table requantisation) must be bit-exact.  fp16 GEMM outputs
must satisfy max|y - ref| <= 2^-10 max|ref| and ||y - ref||_F / ||ref||_F
<= 5e-4 against the float64 oracle (oracle.fp16_bounds).  Full-size
workloads are compared on every output the oracle can afford and on sampled
rows / columns otherwise.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def qg():
    import spec_verify_amd
    return spec_verify_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32, 1: np.uint8}[a.dtype.itemsize])


def assert_bounds(y, ref, what=""):
    r = oracle.fp16_bounds(y, ref)
    assert r["ok"], f"{what}: {r}"
    return r


def packed(qg, codes, scales):
    return qg.w4_repack(dev(codes), dev(scales))


# ---------------------------------------------------------------------------
# activation quantiser
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_w4a8", "decode_w4a8", "prefill_w4a8"])
def test_act_quant_bit_exact_on_workloads(qg, name):
    cfg = synth.CONFIGS[name]
    x = synth.acts(cfg["M"], cfg["K"], cfg["sigma"], cfg["p"], cfg["factor"], cfg["seed"] + 100)
    q, s = qg.act_quant_int8(dev(x))
    oq, os_ = oracle.quant_act(x)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(bits(host(s)), bits(os_))


def test_act_quant_edge_rows_and_strided_input(qg):
    x = synth.acts(7, 640, 1.0, 0.01, 20.0, seed=9)
    x[1] = 0                                          # zero row
    x[2, :6] = [127.0, 0.5, 1.5, 2.5, -2.5, -0.5]     # ties to even with scale 1
    x[2, 6:] = 0
    x[3] = np.float16(6e-8)                           # fp16 subnormals
    x[4] = np.float16(-3.0)                           # constant row
    wide = np.zeros((7, 648), np.float16)
    wide[:, :640] = x
    wide[:, 640:] = np.float16(1000.0)               # past K: must be ignored
    xd = dev(wide)[:, :640]
    q, s = qg.act_quant_int8(xd)
    oq, os_ = oracle.quant_act(x)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(bits(host(s)), bits(os_))


def test_act_quant_values_at_rounding_boundaries(qg):
    """Every code boundary (k + 1/2) * scale, k = 0 .. 126, approached from
    both sides and hit where fp16 can: the fp16 values nearest below, at and
    above each boundary, both signs, for absmax values across the fp16
    range (normal, large, tiny).  The kernel divides by multiplying with a
    corrected reciprocal, so this is where it would differ from the IEEE
    quotient."""
    K = 1024
    rows = []
    for amax in (1.0, 3.0, 0.0107, 32752.0, 127.0, 6.103515625e-05, 1.1920929e-05):
        a = np.float16(amax)
        s = np.float32(np.float32(a) / np.float32(127.0))
        vals = [a, -a]
        for k in range(127):
            t = np.float16(np.float32(k + 0.5) * s)
            for v in (np.nextafter(t, np.float16(-np.inf)), t, np.nextafter(t, np.float16(np.inf))):
                if abs(np.float32(v)) <= np.float32(a):
                    vals += [v, -v]
        row = np.zeros(K, np.float16)
        row[:len(vals)] = np.array(vals, np.float16)[:K]
        rows.append(row)
    x = np.stack(rows)
    assert all(np.abs(r.astype(np.float32)).max() == np.float32(np.float16(a)) for r, a in
               zip(x, (1.0, 3.0, 0.0107, 32752.0, 127.0, 6.103515625e-05, 1.1920929e-05)))
    q, s = qg.act_quant_int8(dev(x))
    oq, os_ = oracle.quant_act(x)
    assert np.array_equal(bits(host(s)), bits(os_))
    assert np.array_equal(host(q), oq)


def test_quantiser_division_exhaustive(qg):
    """The quantiser divides by multiplying with a corrected reciprocal; over
    every finite positive fp16 absmax and every fp16 x with |x| <= absmax
    (1,007,713,278 pairs, on the device), rint of that quotient equals rint
    of the IEEE quotient x / (absmax / 127)."""
    pairs, bad = qg.qg_selftest_quant_division(DEV)
    assert pairs == sum(2 * a + 2 for a in range(1, 0x7C00)) == 1_007_713_278
    assert bad == 0


def test_act_quant_long_rows_take_the_reload_path(qg):
    x = synth.acts(3, 66560, 1.0, 0.01, 20.0, seed=10)   # longer than 1024 threads x 8 register-resident chunks
    q, s = qg.act_quant_int8(dev(x))
    oq, os_ = oracle.quant_act(x)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(bits(host(s)), bits(os_))
    x2 = synth.acts(1100, 20480, 1.0, 0.01, 20.0, seed=12)   # many rows: one wave per row, reloads
    q2, s2 = qg.act_quant_int8(dev(x2))
    oq2, os2 = oracle.quant_act(x2)
    assert np.array_equal(host(q2), oq2)
    assert np.array_equal(bits(host(s2)), bits(os2))
    x3 = synth.acts(1, (1 << 27) + 128, 1.0, 0.01, 20.0, seed=14)   # 2^24 + 16 chunks in one row
    q3, s3 = qg.act_quant_int8(dev(x3))
    oq3, os3 = oracle.quant_act(x3)
    assert np.array_equal(host(q3), oq3)
    assert np.array_equal(bits(host(s3)), bits(os3))


# ---------------------------------------------------------------------------
# W4A8
# ---------------------------------------------------------------------------

def _w4a8_check(qg, x, codes, scales, window=None, rows=None):
    N = codes.shape[0]
    wp, sp = packed(qg, codes, scales)
    y, q, s, P = qg.w4a8_gemm_debug(dev(x), wp, sp, N, window=window)
    oq, os_ = oracle.quant_act(x)
    assert np.array_equal(host(q), oq), "activation codes"
    assert np.array_equal(bits(host(s)), bits(os_)), "token scales"
    m0, m1, n0, n1 = window if window is not None else (0, x.shape[0], 0, N)
    if m1 > m0 and n1 > n0:
        assert np.array_equal(host(P).astype(np.int64), oracle.partials(oq[m0:m1], codes[n0:n1])), "int32 partials"
    yh = host(y)
    if rows is None:
        ref = oracle.ref_w4a8(x, codes, scales, q=oq, s=os_)
        return assert_bounds(yh, ref, "w4a8"), yh
    ref = oracle.ref_w4a8(x[rows], codes, scales, q=oq[rows], s=os_[rows])
    return assert_bounds(yh[rows], ref, "w4a8 sampled rows"), yh


def test_w4a8_tiny_workload_all_stages(qg):
    x, codes, scales = synth.gemm_inputs(synth.CONFIGS["tiny_w4a8"])
    _w4a8_check(qg, x, codes, scales)


def test_w4a8_decode_workload_full(qg):
    """The decode workload (M = 64, K = N = 5120): codes, token scales and
    the int32 partials of two windows bit-exact, every output within the
    fp16 bounds; the debug call's y is bit-identical to w4a8_gemm's, so the
    partials come from the kernel the workload runs."""
    cfg = synth.CONFIGS["decode_w4a8"]
    x, codes, scales = synth.gemm_inputs(cfg)
    _, yd = _w4a8_check(qg, x, codes, scales, window=(0, 64, 0, 512))
    _w4a8_check(qg, x, codes, scales, window=(5, 9, 4600, 5120))
    wp, sp = packed(qg, codes, scales)
    assert np.array_equal(bits(host(qg.w4a8_gemm(dev(x), wp, sp, cfg["N"]))), bits(yd))


@pytest.mark.parametrize("M,K,N", [(64, 5120, 1024), (48, 5120, 6144), (40, 2560, 144), (64, 2560, 1280),
                                   (33, 17408, 80), (17, 5120, 16), (64, 128, 96), (20, 384, 36880),
                                   # narrow outputs: one n-tile per block (the block-count floor)
                                   (64, 1024, 2048), (32, 1024, 3072)])
def test_w4a8_row_split_shapes(qg, M, K, N):
    """16 < M <= 64 runs the row-split kernel for every N (n-tiles dealt
    into balanced blocks of at most 3, at least min(N / 16, 128) of them;
    one or two m-tiles per workgroup): the production call against the
    oracle, and the debug call's partials on a window that crosses n-block
    edges, with its y bit-identical to the production call's."""
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M * 11 + K)
    codes, scales = synth.weights(N, K, seed=N * 11 + K)
    codes[: min(N, 48), :128] = -8
    wp, sp = packed(qg, codes, scales)
    y = host(qg.w4a8_gemm(dev(x), wp, sp, N))
    assert_bounds(y, oracle.ref_w4a8(x, codes, scales), f"w4a8 M={M} K={K} N={N}")
    n0, n1 = max(0, N // 2 - 72), min(N, N // 2 + 88)
    _, yd = _w4a8_check(qg, x, codes, scales, window=(M - 17, M, n0, n1))
    assert np.array_equal(bits(yd), bits(y))


@pytest.mark.parametrize("M,K,N", [(40, 44032, 96), (20, 44032, 48), (9, 66048, 48), (2, 32896, 16400),
                                   # just inside the budget: 32 KiB of scales beside the row
                                   # split's 48 KiB of partial sums at two m-tiles (80 KiB of LDS)
                                   (40, 43648, 96)])
def test_w4a8_scales_past_the_lds_budget(qg, M, K, N):
    """K long enough that a workgroup's group scales exceed the 32 KiB the
    weight-streaming kernel stages in LDS, so its stages carry them instead
    (and one shape just inside that budget):
    the row split (16 < M <= 64, three n-tiles and one or two m-tiles per
    workgroup), and two and four n-tiles per workgroup (M <= 16, N / 16 up
    to and past 1024).  The production call against the
    oracle (sampled columns on the wide case), and the debug call's partials
    on a window with its y bit-identical to the production call's."""
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M * 7 + K)
    codes, scales = synth.weights(N, K, seed=N * 7 + K)
    wp, sp = packed(qg, codes, scales)
    y = host(qg.w4a8_gemm(dev(x), wp, sp, N))
    cols = np.arange(N) if N <= 1024 else np.unique(np.concatenate([np.arange(0, N, 97), np.arange(N - 16, N)]))
    assert_bounds(y[:, cols], oracle.ref_w4a8(x, codes[cols], scales[cols]), f"w4a8 M={M} K={K} N={N}")
    n0, n1 = max(0, N // 2 - 40), min(N, N // 2 + 56)
    yd, _, _, P = qg.w4a8_gemm_debug(dev(x), wp, sp, N, window=(0, M, n0, n1))
    oq, _ = oracle.quant_act(x)
    assert np.array_equal(host(P).astype(np.int64), oracle.partials(oq, codes[n0:n1])), "int32 partials"
    assert np.array_equal(bits(host(yd)), bits(y))


@pytest.mark.parametrize("M,N", [(3, 32), (40, 80), (65, 128)])
def test_w4a8_at_the_longest_k(qg, M, N):
    """K = 2^22, the longest w4a8_gemm accepts, in each M regime (two n-tiles
    per workgroup with the scales carried by the stages, the row split, the
    128 x 128 tile kernel): codes and token scales bit-exact, the int32
    partials of a window bit-exact, every output within the fp16 bounds, and
    the debug call's y bit-identical to the production call's."""
    K = 1 << 22
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M + 7)
    codes, scales = synth.weights(N, K, seed=N + 7)
    _, yd = _w4a8_check(qg, x, codes, scales, window=(0, 3, N - 16, N))
    wp, sp = packed(qg, codes, scales)
    assert np.array_equal(bits(host(qg.w4a8_gemm(dev(x), wp, sp, N))), bits(yd))


@pytest.mark.slow
def test_w4a8_prefill_workload_sampled(qg):
    cfg = synth.CONFIGS["prefill_w4a8"]
    x, codes, scales = synth.gemm_inputs(cfg)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(4090, 4096),
                                     rng.choice(4096, 40, replace=False)]))
    _w4a8_check(qg, x, codes, scales, window=(120, 136, 4990, 5120), rows=rows)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (17, 256, 80), (33, 384, 144), (64, 1024, 48),
                                   (65, 256, 144), (100, 512, 272), (129, 384, 128), (200, 128, 16),
                                   # odd group counts per wave, ragged n-blocks, long K, wide N
                                   (7, 2560, 176), (64, 4992, 400), (40, 17408, 96),
                                   (5, 33024, 32), (4, 256, 16400),
                                   # M <= 16: 254 n-tiles, one per workgroup; 257, blocks of two
                                   (9, 256, 4064), (9, 256, 4112)])
def test_w4a8_ragged_shapes(qg, M, K, N):
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M + K)
    codes, scales = synth.weights(N, K, seed=N + K)
    _w4a8_check(qg, x, codes, scales, window=(0, M, 0, N))


@pytest.mark.parametrize("M,K,N", [(130, 640, 272), (257, 1152, 400), (192, 1664, 160)])
def test_w4a8_large_kernel_back_to_back_bias_windows(qg, M, K, N):
    """M > 64 runs the large-M kernel, which takes the accumulated bias off
    every 4 groups and after the last one.  With G = 1 (mod 4) groups two
    windows end in consecutive groups; their column sums sit in alternating
    LDS buffers.  The production call against the oracle, the debug call's
    partials, and the two calls' outputs bit-identical."""
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M * 7 + K)
    codes, scales = synth.weights(N, K, seed=N * 7 + K)
    wp, sp = packed(qg, codes, scales)
    y = host(qg.w4a8_gemm(dev(x), wp, sp, N))
    assert_bounds(y, oracle.ref_w4a8(x, codes, scales), f"w4a8 M={M} K={K} N={N}")
    _, yd = _w4a8_check(qg, x, codes, scales, window=(M - 40, M, 0, N))
    assert np.array_equal(bits(yd), bits(y))


def test_w4a8_all_minus_8_with_negative_scales_and_zero_rows(qg):
    """The pages' failure: signed scales read as unsigned.  Every code -8 and
    every scale negative, plus an all-zero token row."""
    M, K, N = 5, 256, 32
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=77)
    x[2] = 0
    codes = np.full((N, K), -8, np.int8)
    scales = -np.abs(synth.weights(N, K, seed=78)[1])
    r, yh = _w4a8_check(qg, x, codes, scales)
    assert not yh[2].astype(np.float32).any()


def test_w4a8_strided_activations(qg):
    M, K, N = 10, 512, 64
    wide = synth.acts(M, K + 64, 1.0, 0.01, 20.0, seed=5)
    x = np.ascontiguousarray(wide[:, :K])
    codes, scales = synth.weights(N, K, seed=6)
    wp, sp = packed(qg, codes, scales)
    y = qg.w4a8_gemm(dev(wide)[:, :K], wp, sp, N)
    assert_bounds(host(y), oracle.ref_w4a8(x, codes, scales))


@pytest.mark.parametrize("op,M,K,N", [("w4a8", 40, 640, 160), ("w4a8", 100, 384, 144),
                                      ("w4a16", 8, 640, 160), ("w4a16", 100, 384, 96), ("w4a16", 40, 256, 32784),
                                      ("w8a16", 8, 640, 160), ("w8a16", 100, 384, 96)])
def test_strided_activations_in_every_regime(qg, op, M, K, N):
    """Activation rows 64 elements apart beyond K (ldx = K + 64): the row
    split and the 128 x 128 tile kernel for W4A8; the streaming kernel, its
    64-row chunks past M = 64 and the wide kernel for W4A16; W8A16."""
    wide = synth.acts(M, K + 64, 1.0, 0.01, 20.0, seed=M + K + N)
    wide[:, K:] = 30000.0                 # the columns past K must not be read
    x = np.ascontiguousarray(wide[:, :K])
    xs = dev(wide)[:, :K]
    if op == "w8a16":
        Q, S = oracle.quant_table(synth.table_source(N, K, seed=N + 3))
        y = qg.w8a16_gemm(xs, dev(Q), dev(S))
        ref = oracle.ref_w8a16(x, Q, S)
    else:
        codes, scales = synth.weights(N, K, seed=N + K)
        wp, sp = packed(qg, codes, scales)
        if op == "w4a8":
            y = qg.w4a8_gemm(xs, wp, sp, N)
            ref = oracle.ref_w4a8(x, codes, scales)
        else:
            y = qg.w4a16_gemm(xs, wp, sp, N)
            ref = oracle.ref_w4a16(x, codes, scales)
    assert_bounds(host(y), ref, f"{op} strided M={M} K={K} N={N}")


# ---------------------------------------------------------------------------
# RMSNorm fused with the quantiser
# ---------------------------------------------------------------------------

def _fp16_ulps(a, b):
    """Distance of two fp16 arrays in units in the last place (+0 and -0 equal)."""
    def ordered(v):
        u = np.ascontiguousarray(v).view(np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(ordered(a) - ordered(b))


def _unpack_prepared(buf, M, K):
    """Row-major codes [M, K] and token scales [M] from a prepared buffer, as
    the library lays it out: M <= 64 in fragment order (tiles of 16 rows; for
    tile t, group g, half h a 1 KiB block in which lane col + 16 quad holds
    the 16 codes of row 16 t + col at k = 128 g + 64 h + 16 quad + [0, 16)),
    M > 64 row-major; the fp32 scales follow at the next 256-byte boundary."""
    rows = (M + 15) // 16 * 16 if M <= 64 else M
    codes = buf[: rows * K].view(np.int8)
    if M <= 64:
        G = K // 128
        codes = codes.reshape(rows // 16, G, 2, 4, 16, 16).transpose(0, 4, 1, 2, 3, 5).reshape(rows, K)
    else:
        codes = codes.reshape(M, K)
    s_off = (rows * K + 255) // 256 * 256
    return codes[:M], buf[s_off: s_off + 4 * M].view(np.float32)


@pytest.mark.parametrize("M,H,pad,eps", [(1, 128, 0, 1e-6), (7, 640, 8, 1e-5), (64, 5120, 0, 1e-6),
                                         (70, 1280, 0, 0.0), (3, 17408, 0, 1e-6), (2, 65536, 128, 1e-6),
                                         (16, 2048, 0, 0.5)])
def test_rmsnorm_prepare_against_the_exact_norm(qg, M, H, pad, eps):
    """y within one fp16 unit in the last place of the oracle's norm (the
    float64 value rounded once; the kernel evaluates it in fp32, so it may
    round the other way where the exact value is within a few fp32 ulps of
    a tie, a few times in 10^4), and the prepared buffer holding exactly the
    oracle quantiser's codes and token scales of the kernel's own y, and the
    same bytes as w4a8_prepare of that y.  Covers one wave through 1024
    threads x 8 chunks, a strided input, M > 64 (row-major codes), eps = 0
    with a zero row, a row of outliers and a negative zero."""
    x = synth.acts(M, H + pad, 1.0, 0.01, 20.0, seed=M * 7 + H)
    x[0, 3] = -0.0                                    # signed zero keeps its sign through the norm
    if M > 2:
        x[1] = 0
        x[2, ::97] = 3000.0
    w = (1.0 + 0.25 * synth.acts(1, H, 1.0, 0.0, 1.0, seed=H + 1)[0].astype(np.float32)).astype(np.float16)
    xd = dev(x)[:, :H]
    need = qg.w4a8_prepared_bytes(M, H)
    got = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    y, _ = qg.rmsnorm_w4a8_prepare(xd, dev(w), eps, prepared=got)
    yk = host(y)
    want_y = oracle.rmsnorm(x[:, :H], w, eps)
    d = _fp16_ulps(yk, want_y)
    assert d.max() <= 1 and (d > 0).mean() <= 2e-3, (d.max(), (d > 0).mean())
    assert np.signbit(yk[0, 3])
    q, s = _unpack_prepared(host(got), M, H)
    oq, os_ = oracle.quant_act(yk)
    assert np.array_equal(q, oq)
    assert np.array_equal(bits(s), bits(os_))
    want = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    qg.w4a8_prepare(y, prepared=want)
    assert torch.equal(got, want)
    # without the fp16 output the prepared buffer is the same
    again = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    none, _ = qg.rmsnorm_w4a8_prepare(xd, dev(w), eps, prepared=again, want_y=False)
    assert none is None and torch.equal(again, want)


def test_rmsnorm_prepare_feeds_the_w4a8_gemm(qg):
    """The fused buffer drives w4a8_gemm_prepared to exactly w4a8_gemm's
    output on the normalised rows (decode shape)."""
    cfg = synth.CONFIGS["decode_w4a8"]
    x, codes, scales = synth.gemm_inputs(cfg)
    wp, sp = packed(qg, codes, scales)
    w = (1.0 + 0.25 * synth.acts(1, cfg["K"], 1.0, 0.0, 1.0, seed=77)[0].astype(np.float32)).astype(np.float16)
    y, prep = qg.rmsnorm_w4a8_prepare(dev(x), dev(w), 1e-6)
    a = host(qg.w4a8_gemm_prepared(prep, cfg["M"], cfg["K"], wp, sp, cfg["N"]))
    b = host(qg.w4a8_gemm(y, wp, sp, cfg["N"]))
    assert np.array_equal(bits(a), bits(b))
    assert_bounds(a, oracle.ref_w4a8(host(y), codes, scales))


# ---------------------------------------------------------------------------
# split-KV verify attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,Hq,Hkv,L", [(1, 8, 8, 1), (1, 4, 1, 300), (5, 24, 4, 37), (5, 24, 4, 1536),
                                        (8, 16, 2, 300), (16, 16, 2, 2000), (16, 24, 4, 16384),
                                        (3, 6, 3, 8193), (7, 2, 1, 7), (6, 12, 2, 500), (2, 4, 1, 9000),
                                        (16, 4096, 4096, 40), (1, 4096, 32, 300), (16, 8, 1, (1 << 20) + 7)])
def test_verify_attention_within_bounds(qg, T, Hq, Hkv, L):
    """Against the float64 oracle, element by element, within the fp16 output
    bounds.  Covers one position, GQA groups of 1 to 8 heads, 16 queries x 8
    heads (128 rows: two row tiles per wave), three row tiles (one per wave),
    up to two row tiles (the block's positions split between wave pairs), a
    16k cache (64 splits), 86 and 141 splits (pass 2 loads 64 at a time), a
    ragged last block and split, a cache that is only the verify block, the
    most query heads (4096: one split per KV head, 4096 KV heads), 128 query
    heads per KV head, and a cache of 2^20 + 7 positions (255 splits of 129
    blocks)."""
    rng = np.random.default_rng(T * 1000 + L)
    q = rng.standard_normal((T, Hq, 256)).astype(np.float16)
    k = rng.standard_normal((L, Hkv, 256)).astype(np.float16)
    v = rng.standard_normal((L, Hkv, 256)).astype(np.float16)
    o = qg.verify_attention_f16(dev(q), dev(k), dev(v))
    assert_bounds(host(o).reshape(T, -1), oracle.ref_verify_attention(q, k, v).reshape(T, -1),
                  f"attention T={T} Hq={Hq} Hkv={Hkv} L={L}")


@pytest.mark.parametrize("T,Hq,Hkv,L,kind", [(5, 24, 4, 16384, "rising"), (8, 16, 16, 4096, "blocks"),
                                             (1, 8, 8, 3000, "rising"), (16, 16, 2, 5000, "blocks")])
def test_verify_attention_online_rescale(qg, T, Hq, Hkv, L, kind):
    """Keys whose size changes along the positions, so that a row's visible
    scores move by many log2 units from one 32-position block to the next:
    "rising" scales key p by 64^(p / L) (later blocks top earlier ones, by
    more than 8 log2 units within a split near the end), "blocks" gives each
    32-position block its own scale, log-uniform on [0.125, 16].  The running
    maximum then moves past the 8 log2 units the kernel lets it lag, the
    partial output is rescaled by factors far from 1, and the splits' maxima
    differ widely in the combine.  Element by element within the fp16
    bounds."""
    rng = np.random.default_rng(L + T)
    q = rng.standard_normal((T, Hq, 256)).astype(np.float16)
    pos = np.arange(L)
    if kind == "rising":
        scale = 64.0 ** (pos / L)
    else:
        scale = np.exp(rng.uniform(np.log(0.125), np.log(16.0), (L + 31) // 32))[pos // 32]
    k = (rng.standard_normal((L, Hkv, 256)) * scale[:, None, None]).astype(np.float16)
    v = rng.standard_normal((L, Hkv, 256)).astype(np.float16)
    # the inputs do move a lagging maximum many times: query 0, head 0, block
    # maxima in log2 units, the reference moved whenever a block tops it by 8
    s0 = (q[0, 0].astype(np.float64) @ k[: L - T + 1, 0].astype(np.float64).T) / 16.0 * np.log2(np.e)
    bmax = np.array([blk.max() for blk in np.array_split(s0, np.arange(32, len(s0), 32))])
    ref, moves = -np.inf, 0
    for b in bmax:
        if b > ref + 8:
            ref, moves = b, moves + 1
    assert moves >= 3 and np.ptp(bmax) > 16, (moves, np.ptp(bmax))
    o = qg.verify_attention_f16(dev(q), dev(k), dev(v))
    assert_bounds(host(o).reshape(T, -1), oracle.ref_verify_attention(q, k, v).reshape(T, -1),
                  f"attention rescale {kind} T={T} Hq={Hq} Hkv={Hkv} L={L}")


def test_verify_attention_is_causal_and_deterministic(qg):
    """Changing the cache after query 0's position leaves query 0's output
    unchanged bit for bit; repeated calls agree bit for bit."""
    T, Hq, Hkv, L = 5, 24, 4, 700
    rng = np.random.default_rng(3)
    q = rng.standard_normal((T, Hq, 256)).astype(np.float16)
    k = rng.standard_normal((L, Hkv, 256)).astype(np.float16)
    v = rng.standard_normal((L, Hkv, 256)).astype(np.float16)
    a = host(qg.verify_attention_f16(dev(q), dev(k), dev(v)))
    b = host(qg.verify_attention_f16(dev(q), dev(k), dev(v)))
    assert np.array_equal(bits(a), bits(b))
    k[L - T + 1:] = 9.0
    v[L - T + 1:] = -4.0
    c = host(qg.verify_attention_f16(dev(q), dev(k), dev(v)))
    assert np.array_equal(bits(c[0]), bits(a[0]))


# ---------------------------------------------------------------------------
# W4A16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["verify_w4a16_m8", "verify_w4a16_m16"])
def test_w4a16_verify_workload_full(qg, name):
    cfg = synth.CONFIGS[name]
    x, codes, scales = synth.gemm_inputs(cfg)
    wp, sp = packed(qg, codes, scales)
    y = qg.w4a16_gemm(dev(x), wp, sp, cfg["N"])
    assert_bounds(host(y), oracle.ref_w4a16(x, codes, scales), name)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (8, 5120, 80), (16, 384, 144), (64, 256, 48),
                                   (65, 256, 32), (150, 384, 96),
                                   # wide outputs (M > 32: waves split N, LDS-shared activations,
                                   # 4 or 8 waves of 2 n-tiles, or 8 waves of 4 n-tiles from 12288
                                   # n-tiles on, a last workgroup with one valid n-tile; M <= 32:
                                   # the K-split kernel on many workgroups)
                                   (5, 384, 32784), (33, 256, 32784), (64, 128, 131088), (3, 256, 131072),
                                   (64, 128, 196624), (40, 256, 196608),
                                   # 1025 and 2560 n-tiles: the 512 balanced blocks, split unevenly
                                   # between the first and second 256 and evenly at the top
                                   (2, 256, 16400), (16, 128, 40960),
                                   # 1020 n-tiles: 255 four-tile blocks become 256 blocks of up to four
                                   (8, 256, 16320)])
def test_w4a16_ragged_shapes(qg, M, K, N):
    x = synth.acts(M, K, 1.0, 0.0, 1.0, seed=M * 3 + K)
    codes, scales = synth.weights(N, K, seed=N * 3 + K)
    codes[:, :128] = -8
    wp, sp = packed(qg, codes, scales)
    y = qg.w4a16_gemm(dev(x), wp, sp, N)
    assert_bounds(host(y), oracle.ref_w4a16(x, codes, scales))


@pytest.mark.parametrize("M", [1, 8, 16])
def test_w4a16_biased_operands_with_extreme_activations(qg, M):
    """The K-split W4A16 kernel multiplies biased codes (1032 + q, or
    1152 + 16 q against x / 16) and starts each product from minus the
    activations' bias.  Activations near the fp16 limit, subnormal ones and
    zero rows, codes -8 and 7, and weight columns of all-zero codes (whose
    outputs must stay at rounding level) all stay within the fp16 bounds."""
    K, N = 1024, 160
    rng = np.random.default_rng(M + 5)
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=M + 70)
    x[0, ::97] = np.float16(60000.0)
    x[0, 5::131] = np.float16(-60000.0)
    x[-1, ::3] = np.float16(2.0 ** -20)        # subnormal, and subnormal again once divided by 16
    if M > 2:
        x[1] = 0
    codes, scales = synth.weights(N, K, seed=M + 71)
    codes[:16] = -8
    codes[16:32] = 7
    codes[32:48] = 0
    codes[48:64] = rng.choice(np.array([-8, 7], np.int8), size=(16, K))
    wp, sp = packed(qg, codes, scales)
    y = host(qg.w4a16_gemm(dev(x), wp, sp, N))
    ref = oracle.ref_w4a16(x, codes, scales)
    # row 0 (outputs up to about 2e4) on its own, so that it does not set
    # the tolerance of the ordinary rows
    assert_bounds(y[:1], ref[:1], f"w4a16 extreme M={M} row 0")
    if M > 1:
        assert_bounds(y[1:], ref[1:], f"w4a16 extreme M={M} rows 1+")


# ---------------------------------------------------------------------------
# int8 vocabulary table: requantisation, gather, lm_head
# ---------------------------------------------------------------------------

def test_quant_table_bit_exact(qg):
    src = synth.table_source(3000, 640, seed=21)
    src[7, :128] = 0
    Q, S = qg.quant_table_int8(dev(src.view(np.int16)))
    oQ, oS = oracle.quant_table(src)
    assert np.array_equal(host(Q), oQ)
    assert np.array_equal(bits(host(S)), bits(oS))


def test_gather_bit_exact_with_out_of_range_ids(qg):
    src = synth.table_source(1000, 384, seed=22)
    oQ, oS = oracle.quant_table(src)
    ids = np.array([0, 999, -1, 1000, 5, 5, 2 ** 31 - 1, 123], np.int32)
    out = qg.embed_gather_dequant_int8(dev(ids), dev(oQ), dev(oS))
    assert np.array_equal(bits(host(out)), bits(oracle.ref_gather(ids, oQ, oS)))


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (64, 640, 400), (8, 256, 1040), (70, 256, 64), (8, 256, 16400),
                                   # wide outputs (see the W4A16 cases)
                                   (40, 384, 32784), (9, 128, 131088), (64, 256, 32768), (48, 128, 131088),
                                   (33, 256, 196624), (64, 128, 196624)])
def test_w8a16_ragged_shapes(qg, M, K, N):
    src = synth.table_source(N, K, seed=N + 1)
    Q, S = oracle.quant_table(src)
    x = synth.acts(M, K, 1.0, 0.0, 1.0, seed=M + 2)
    y = qg.w8a16_gemm(dev(x), dev(Q), dev(S))
    assert_bounds(host(y), oracle.ref_w8a16(x, Q, S))


@pytest.mark.parametrize("mode,M,N", [("w4a16", 8, 48), ("w4a16", 40, 48), ("w8a16", 8, 48), ("w8a16", 64, 80)])
def test_fp16_modes_at_the_longest_k(qg, mode, M, N):
    """K = 65536, the longest w4a16_gemm and w8a16_gemm accept: a workgroup
    of four n-tiles holds 48-64 KiB of group scales in LDS (beside 64 KiB of
    partial sums at M > 32), most of them stored by the passes past the
    four register-staged ones."""
    K = 65536
    x = synth.acts(M, K, 1.0, 0.0, 1.0, seed=M * 5 + N)
    if mode == "w4a16":
        codes, scales = synth.weights(N, K, seed=N * 5 + M)
        codes[:, :128] = -8
        wp, sp = packed(qg, codes, scales)
        y = qg.w4a16_gemm(dev(x), wp, sp, N)
        ref = oracle.ref_w4a16(x, codes, scales)
    else:
        Q, S = oracle.quant_table(synth.table_source(N, K, seed=N * 5 + M))
        y = qg.w8a16_gemm(dev(x), dev(Q), dev(S))
        ref = oracle.ref_w8a16(x, Q, S)
    assert_bounds(host(y), ref, f"{mode} M={M} K={K} N={N}")


@pytest.mark.parametrize("N,Ms", [(16400, (2, 64)), (32784, (40,))])
def test_w4a16_longest_k_on_wide_outputs(qg, N, Ms):
    """K = 65536 on wide outputs: 1025 n-tiles make the 512 balanced blocks
    of up to five tiles (80 KiB of scales per workgroup; 144 KiB of LDS with
    the partial sums at M = 64), and 2049 n-tiles at M > 32 take the wide
    kernel, which streams its scales group by group.  Sampled columns (every
    97th, the edges of the two halves' blocks, the last tile) against the
    oracle."""
    K = 65536
    codes, scales = synth.weights(N, K, seed=N + 65)
    wp, sp = packed(qg, codes, scales)
    t1 = min(N // 16 * 10 // 17, 5 * 256) * 16
    cols = np.unique(np.concatenate([np.arange(0, N, 97), np.arange(t1 - 16, t1 + 16), np.arange(N - 16, N)]))
    for M in Ms:
        x = synth.acts(M, K, 1.0, 0.0, 1.0, seed=M + N)
        y = host(qg.w4a16_gemm(dev(x), wp, sp, N))
        assert_bounds(y[:, cols], oracle.ref_w4a16(x, codes[cols], scales[cols]), f"w4a16 M={M} K={K} N={N}")


@pytest.mark.slow
def test_vocab_workload_full_table(qg):
    """248,320 x 5,120 table: requantised on the device, then the 64-id
    gather (bit-exact) and the M=64 lm_head (sampled columns)."""
    cfg = synth.CONFIGS["vocab_int8"]
    V, H, seed = cfg["V"], cfg["H"], cfg["seed"]
    src = synth.table_source(V, H, seed + 200)
    Qd, Sd = qg.quant_table_int8(dev(src.view(np.int16)))
    rng = np.random.default_rng(1)
    check_rows = np.unique(np.concatenate([rng.choice(V, 2048, replace=False), [0, V - 1]]))
    oQ, oS = oracle.quant_table(src[check_rows])
    assert np.array_equal(host(Qd[torch.from_numpy(check_rows).to(DEV)]), oQ)
    assert np.array_equal(bits(host(Sd[torch.from_numpy(check_rows).to(DEV)])), bits(oS))

    ids = synth.token_ids(cfg["T"], V, seed + 300)
    out = qg.embed_gather_dequant_int8(dev(ids), Qd, Sd)
    gQ, gS = oracle.quant_table(src[ids])
    want = oracle.ref_gather(np.arange(len(ids), dtype=np.int32), gQ, gS)
    assert np.array_equal(bits(host(out)), bits(want))

    x = synth.acts(cfg["M"], H, cfg["sigma"], cfg["p"], cfg["factor"], seed + 100)
    y = qg.w8a16_gemm(dev(x), Qd, Sd)
    cols = np.unique(np.concatenate([rng.choice(V, 4096, replace=False), np.arange(V - 16, V)]))
    cQ, cS = oracle.quant_table(src[cols])
    assert_bounds(host(y)[:, cols], oracle.ref_w8a16(x, cQ, cS), "lm_head sampled columns")

    # the 40,960-row draft head: its rows gathered once from the table, then
    # the same int8 lm_head product at M = 1 (sampled columns)
    dcfg = synth.CONFIGS["draft_head_int8"]
    dids = synth.draft_ids(dcfg["D"], V, dcfg["seed"])
    dt = torch.from_numpy(dids).to(DEV)
    DQ, DS = Qd.index_select(0, dt).contiguous(), Sd.index_select(0, dt).contiguous()
    xd = synth.acts(dcfg["M"], H, dcfg["sigma"], dcfg["p"], dcfg["factor"], dcfg["seed"] + 100)
    yd = qg.w8a16_gemm(dev(xd), DQ, DS)
    dcols = np.unique(np.concatenate([rng.choice(dcfg["D"], 2048, replace=False), np.arange(dcfg["D"] - 8, dcfg["D"])]))
    dQ, dS = oracle.quant_table(src[dids[dcols]])
    assert_bounds(host(yd)[:, dcols], oracle.ref_w8a16(xd, dQ, dS), "draft head sampled columns")
    del Qd, Sd, DQ, DS, src


@pytest.mark.parametrize("M", [1, 8])
def test_draft_head_is_the_lm_head_over_a_row_subset(qg, M):
    """A draft head of 40,960 distinct rows gathered from a requantised table:
    the gathered rows are the table's rows bit for bit, and the product over
    them matches the oracle's over the same rows (every column)."""
    V, H = 60000, 1280
    src = synth.table_source(V, H, seed=41)
    Qd, Sd = qg.quant_table_int8(dev(src.view(np.int16)))
    oQ, oS = oracle.quant_table(src)
    ids = synth.draft_ids(40960, V, seed=41)
    dt = torch.from_numpy(ids).to(DEV)
    DQ, DS = Qd.index_select(0, dt).contiguous(), Sd.index_select(0, dt).contiguous()
    assert np.array_equal(host(DQ), oQ[ids])
    assert np.array_equal(bits(host(DS)), bits(oS[ids]))
    x = synth.acts(M, H, 1.0, 0.0, 1.0, seed=M + 42)
    y = qg.w8a16_gemm(dev(x), DQ, DS)
    assert_bounds(host(y), oracle.ref_w8a16(x, oQ[ids], oS[ids]), "draft head")


@pytest.mark.slow
@pytest.mark.parametrize("M", [16, 64])
def test_int4_lm_head_full_size(qg, M):
    """An int4 lm_head over all 248,320 rows (W4A16, group-128 signed scales):
    M = 16 takes the K-split kernel, M = 64 the wide-output one (sampled
    columns, the last tiles included)."""
    cfg = synth.CONFIGS["lm_head_w4a16"]
    K, N = cfg["K"], cfg["N"]
    codes, scales = synth.weights(N, K, cfg["seed"])
    wp, sp = packed(qg, codes, scales)
    x = synth.acts(M, K, cfg["sigma"], cfg["p"], cfg["factor"], cfg["seed"] + 100)
    y = host(qg.w4a16_gemm(dev(x), wp, sp, N))
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([rng.choice(N, 4096, replace=False), np.arange(N - 16, N)]))
    assert_bounds(y[:, cols], oracle.ref_w4a16(x, codes[cols], scales[cols]), f"int4 lm_head M={M}")
    del wp, sp


# ---------------------------------------------------------------------------
# properties: empty input, batch invariance, determinism, no stray writes
# ---------------------------------------------------------------------------

def test_empty_batch_is_a_no_op(qg):
    codes, scales = synth.weights(32, 256, seed=1)
    wp, sp = packed(qg, codes, scales)
    x = torch.empty((0, 256), dtype=torch.float16, device=DEV)
    for fn in (qg.w4a8_gemm, qg.w4a16_gemm):
        y = fn(x, wp, sp, 32)
        assert y.shape == (0, 32)
    out = qg.embed_gather_dequant_int8(torch.empty((0,), dtype=torch.int32, device=DEV),
                                       dev(np.zeros((4, 128), np.int8)), dev(np.zeros((4, 1), np.float16)))
    assert out.shape == (0, 128)


@pytest.mark.parametrize("op", ["w4a8", "w4a16"])
def test_rows_do_not_depend_on_the_batch(qg, op):
    """A token's output does not change with the other tokens in the batch,
    bit for bit, within each kernel regime: W4A16 takes the weight-streaming
    kernel at M = 1 .. 64 here; W4A8 takes it at M <= 16 and its row-split
    form at 16 < M <= 64 (one 16-row m-tile per workgroup up to M = 32, two
    above, over the same n-blocks, with the same group order for every
    m-tile), which adds the groups in another order than the M <= 16 form."""
    cfg = synth.CONFIGS["decode_w4a8"]
    x, codes, scales = synth.gemm_inputs(cfg)
    wp, sp = packed(qg, codes, scales)
    fn = qg.w4a8_gemm if op == "w4a8" else qg.w4a16_gemm
    full = host(fn(dev(x), wp, sp, cfg["N"]))
    small = host(fn(dev(x[:16]), wp, sp, cfg["N"]))
    for M in (1, 8):
        part = host(fn(dev(x[:M]), wp, sp, cfg["N"]))
        assert np.array_equal(bits(part), bits(small[:M])), M
    if op == "w4a16":
        assert np.array_equal(bits(small), bits(full[:16]))
    for M in (17, 33, 48):
        part = host(fn(dev(x[:M]), wp, sp, cfg["N"]))
        assert np.array_equal(bits(part), bits(full[:M])), M


@pytest.mark.parametrize("name", ["decode_w4a8", "verify_w4a16_m16"])
def test_repeat_runs_are_bit_identical(qg, name):
    cfg = synth.CONFIGS[name]
    x, codes, scales = synth.gemm_inputs(cfg)
    wp, sp = packed(qg, codes, scales)
    fn = qg.w4a8_gemm if cfg["op"] == "w4a8" else qg.w4a16_gemm
    xd = dev(x)
    a = host(fn(xd, wp, sp, cfg["N"]))
    b = host(fn(xd, wp, sp, cfg["N"]))
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("M,K,N", [(64, 5120, 5120), (3, 256, 48), (130, 384, 144)])
def test_prepared_activations_are_reusable_and_match_the_one_call_path(qg, M, K, N):
    """One w4a8_prepare feeding two GEMMs (different weights) gives exactly
    w4a8_gemm's outputs for each."""
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=21)
    xd = dev(x)
    prep = qg.w4a8_prepare(xd)
    for seed in (22, 23):
        codes, scales = synth.weights(N, K, seed=seed)
        wp, sp = packed(qg, codes, scales)
        a = host(qg.w4a8_gemm_prepared(prep, M, K, wp, sp, N))
        b = host(qg.w4a8_gemm(xd, wp, sp, N))
        assert np.array_equal(bits(a), bits(b))
        assert_bounds(a, oracle.ref_w4a8(x, codes, scales))


@pytest.mark.parametrize("M,K,N", [(64, 5120, 5120), (5, 5120, 144), (100, 512, 272)])
def test_w4a8_workspace_reuse_across_weight_sets(qg, M, K, N):
    """One workspace reused for different inputs and weights gives each
    call's own result (nothing stale carries over between calls)."""
    ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=DEV)
    for seed in (11, 12, 11):
        x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=seed)
        codes, scales = synth.weights(N, K, seed=seed + 1)
        wp, sp = packed(qg, codes, scales)
        y = qg.w4a8_gemm(dev(x), wp, sp, N, workspace=ws)
        assert_bounds(host(y), oracle.ref_w4a8(x, codes, scales), f"seed {seed}")


@pytest.mark.parametrize("M,N", [(3, 48), (64, 80), (130, 144)])
def test_outputs_stay_inside_their_buffer(qg, M, N):
    """Canary-filled padding around y is untouched after the call."""
    K = 256
    x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=3)
    codes, scales = synth.weights(N, K, seed=4)
    wp, sp = packed(qg, codes, scales)
    pad = 4096
    for fn in (qg.w4a8_gemm, qg.w4a16_gemm):
        buf = torch.full((M * N + 2 * pad,), 0x7bcd, dtype=torch.int16, device=DEV)
        y = buf[pad:pad + M * N].view(torch.float16).view(M, N)
        fn(dev(x), wp, sp, N, y=y)
        hb = host(buf)
        assert (hb[:pad] == 0x7bcd).all() and (hb[pad + M * N:] == 0x7bcd).all()
