"""Entry points captured in a HIP graph and replayed.

Each case captures one or more library calls in a torch.cuda.CUDAGraph
(outputs, workspaces and inputs allocated before the capture), then replays
the graph three times.  Between replays the host poisons every output and
workspace with an eager fill on the same stream and synchronises, so each
replay must recompute everything from its inputs.  Every replay's outputs
must be bit-identical to the eager call's.  The library allocates nothing
and enqueues no memset, so its calls are capturable as they are.
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


def raw(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def replay_matches_eager(run, outs, scratch=()):
    """run() issues the calls into the tensors of `outs` (and may use those of
    `scratch`).  Eager result first, then capture, then three poisoned
    replays, each compared byte for byte."""
    run()
    torch.cuda.synchronize()
    want = [raw(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                   # warm on a side stream, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in list(outs) + list(scratch):
            t.view(torch.uint8).fill_(0xA5 ^ rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(raw(o), w), f"replay {rep}, output {i}"


def _packed(qg, N, K, seed):
    codes, scales = synth.weights(N, K, seed=seed)
    return qg.w4_repack(dev(codes), dev(scales))


@pytest.mark.parametrize("M,K,N", [(64, 1280, 1280), (8, 640, 160), (200, 512, 256)])
def test_w4a8_gemm_in_a_graph(qg, M, K, N):
    """The row split, two n-tiles per workgroup and the 128 x 128 kernel, each
    behind the quantiser, with the workspace poisoned between replays."""
    x = dev(synth.acts(M, K, 1.0, 0.01, 20.0, seed=M + K))
    wp, sp = _packed(qg, N, K, seed=N + 1)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=DEV)
    replay_matches_eager(lambda: qg.w4a8_gemm(x, wp, sp, N, y=y, workspace=ws), [y], [ws])


def test_w4a8_noalloc_in_a_graph(qg):
    M, K, N = 64, 1280, 1280
    x = dev(synth.acts(M, K, 1.0, 0.01, 20.0, seed=5))
    wp, sp = _packed(qg, N, K, seed=6)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    replay_matches_eager(lambda: qg.w4a8_gemm_noalloc(x, wp, sp, N, y), [y])


def test_norm_prepare_and_prepared_gemms_in_one_graph(qg):
    """The fused norm + quantiser feeding two GEMMs on one prepared buffer."""
    M, H, N1, N2 = 64, 1280, 1280, 640
    x = dev(synth.acts(M, H, 1.0, 0.01, 20.0, seed=7))
    w = dev((1.0 + 0.25 * synth.acts(1, H, 1.0, 0.0, 1.0, seed=8)[0].astype(np.float32)).astype(np.float16))
    wp1, sp1 = _packed(qg, N1, H, seed=9)
    wp2, sp2 = _packed(qg, N2, H, seed=10)
    prep = torch.empty((qg.w4a8_prepared_bytes(M, H),), dtype=torch.uint8, device=DEV)
    yn = torch.empty((M, H), dtype=torch.float16, device=DEV)
    y1 = torch.empty((M, N1), dtype=torch.float16, device=DEV)
    y2 = torch.empty((M, N2), dtype=torch.float16, device=DEV)

    def run():
        qg.rmsnorm_w4a8_prepare(x, w, 1e-6, prepared=prep, y=yn)
        qg.w4a8_gemm_prepared(prep, M, H, wp1, sp1, N1, y=y1)
        qg.w4a8_gemm_prepared(prep, M, H, wp2, sp2, N2, y=y2)

    replay_matches_eager(run, [yn, prep, y1, y2])


@pytest.mark.parametrize("M,K,N", [(8, 512, 16400), (16, 640, 160), (40, 256, 32784), (100, 384, 96)])
def test_w4a16_gemm_in_a_graph(qg, M, K, N):
    """The balanced blocks, the streaming kernel, the wide kernel and the
    64-row chunks past M = 64."""
    x = dev(synth.acts(M, K, 1.0, 0.0, 1.0, seed=M + N))
    wp, sp = _packed(qg, N, K, seed=K + 3)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    replay_matches_eager(lambda: qg.w4a16_gemm(x, wp, sp, N, y=y), [y])


def test_quantiser_table_gather_and_lm_head_in_one_graph(qg):
    """Per-token quantiser, table requantisation, gather and the int8-table
    lm_head, captured together."""
    V, H, T, M = 1040, 512, 64, 8
    src = dev(synth.table_source(V, H, seed=11).view(np.int16))
    Q = torch.empty((V, H), dtype=torch.int8, device=DEV)
    S = torch.empty((V, H // 128), dtype=torch.float16, device=DEV)
    ids = dev(np.random.default_rng(12).integers(-3, V + 3, T).astype(np.int32))
    emb = torch.empty((T, H), dtype=torch.float16, device=DEV)
    xa = dev(synth.acts(M, H, 1.0, 0.01, 20.0, seed=13))
    q = torch.empty((M, H), dtype=torch.int8, device=DEV)
    sc = torch.empty((M,), dtype=torch.float32, device=DEV)
    logits = torch.empty((M, V), dtype=torch.float16, device=DEV)

    def run():
        qg.quant_table_int8(src, Q=Q, S=S)
        qg.embed_gather_dequant_int8(ids, Q, S, out=emb)
        qg.act_quant_int8(xa, q=q, scale=sc)
        qg.w8a16_gemm(xa, Q, S, y=logits)

    replay_matches_eager(run, [Q, S, emb, q, sc, logits])


def test_attention_and_sampler_in_one_graph(qg):
    """Verify attention over a 1.5k cache and the sampler over 16 rows of
    248,320 logits, workspaces poisoned between replays."""
    T, Hq, Hkv, L = 5, 24, 4, 1536
    qa, ka, va = synth.attention_inputs(T, Hq, Hkv, L, seed=14)
    qd, kd, vd = dev(qa), dev(ka), dev(va)
    o = torch.empty((T, Hq, 256), dtype=torch.float16, device=DEV)
    aws = torch.empty((qg.verify_attention_workspace_bytes(T, Hq, Hkv, L),), dtype=torch.uint8, device=DEV)
    R, V, k = 16, 248320, 20
    lx, lu = synth.sampler_inputs(R, V, seed=15)
    ld, ud = dev(lx), dev(lu.astype(np.float32))
    outs = (torch.empty((R, k), dtype=torch.int32, device=DEV), torch.empty((R, k), dtype=torch.float32, device=DEV),
            torch.empty((R,), dtype=torch.int32, device=DEV), torch.empty((R,), dtype=torch.int32, device=DEV),
            torch.empty((R,), dtype=torch.float32, device=DEV))
    sws = torch.empty((qg.sampler_workspace_bytes(R, V, k),), dtype=torch.uint8, device=DEV)

    def run():
        qg.verify_attention_f16(qd, kd, vd, o=o, workspace=aws)
        qg.sample_topk_topp(ld, ud, k, 0.95, 1.0, out=outs, workspace=sws)

    replay_matches_eager(run, [o, *outs], [aws, sws])
    # and the replayed top-k ids are the oracle's
    want = oracle.topk_topp_sample(lx, k, 0.95, 1.0, lu)
    assert np.array_equal(outs[0].cpu().numpy().astype(np.int64), want["ids"])
