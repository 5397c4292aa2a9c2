"""Calls on several streams at once, and from several host threads.

The library keeps no mutable global state on the host or the device (the
allocation-free entry point's scratch array aside, which is not used here):
each call works only on the caller's buffers and the stream it is given.
Independent calls issued on separate streams, and from separate host threads
each with its own stream, must give the same bytes as the same calls made
one after another.  Streams keep the default priority.
"""
import threading

import numpy as np
import pytest
import torch

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


def _jobs(qg):
    """Independent jobs, each a (run, outputs) pair with its own buffers."""
    jobs = []
    for j, (M, K, N) in enumerate([(64, 1280, 1280), (8, 1024, 16400), (200, 512, 256), (40, 640, 400)]):
        x = dev(synth.acts(M, K, 1.0, 0.01, 20.0, seed=30 + j))
        codes, scales = synth.weights(N, K, seed=40 + j)
        wp, sp = qg.w4_repack(dev(codes), dev(scales))
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        if j % 2 == 0:
            ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=DEV)
            run = (lambda x=x, wp=wp, sp=sp, N=N, y=y, ws=ws: qg.w4a8_gemm(x, wp, sp, N, y=y, workspace=ws))
        else:
            run = (lambda x=x, wp=wp, sp=sp, N=N, y=y: qg.w4a16_gemm(x, wp, sp, N, y=y))
        jobs.append((run, [y]))
    T, Hq, Hkv, L = 5, 24, 4, 4096
    qa, ka, va = synth.attention_inputs(T, Hq, Hkv, L, seed=50)
    qd, kd, vd = dev(qa), dev(ka), dev(va)
    o = torch.empty((T, Hq, 256), dtype=torch.float16, device=DEV)
    aws = torch.empty((qg.verify_attention_workspace_bytes(T, Hq, Hkv, L),), dtype=torch.uint8, device=DEV)
    jobs.append((lambda: qg.verify_attention_f16(qd, kd, vd, o=o, workspace=aws), [o]))
    R, V, k = 8, 248320, 20
    lx, lu = synth.sampler_inputs(R, V, seed=51)
    ld, ud = dev(lx), dev(lu.astype(np.float32))
    outs = (torch.empty((R, k), dtype=torch.int32, device=DEV), torch.empty((R, k), dtype=torch.float32, device=DEV),
            torch.empty((R,), dtype=torch.int32, device=DEV), torch.empty((R,), dtype=torch.int32, device=DEV),
            torch.empty((R,), dtype=torch.float32, device=DEV))
    sws = torch.empty((qg.sampler_workspace_bytes(R, V, k),), dtype=torch.uint8, device=DEV)
    jobs.append((lambda: qg.sample_topk_topp(ld, ud, k, 0.95, 1.0, out=outs, workspace=sws), list(outs)))
    return jobs


def _sequential(jobs):
    want = []
    for run, outs in jobs:
        run()
        torch.cuda.synchronize()
        want.append([raw(o) for o in outs])
        for o in outs:
            o.view(torch.uint8).fill_(0x5A)
    torch.cuda.synchronize()
    return want


def test_independent_calls_on_separate_streams(qg):
    jobs = _jobs(qg)
    want = _sequential(jobs)
    streams = [torch.cuda.Stream() for _ in jobs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for (run, _), s in zip(jobs, streams):
            with torch.cuda.stream(s):
                run()
        torch.cuda.synchronize()
        for i, ((_, outs), w) in enumerate(zip(jobs, want)):
            for o, wo in zip(outs, w):
                assert np.array_equal(raw(o), wo), f"rep {rep}, job {i}"
            for o in outs:
                o.view(torch.uint8).fill_(0x5A ^ rep)
        torch.cuda.synchronize()


def test_calls_from_several_host_threads(qg):
    """One host thread per job, each on its own stream, all started together
    and each calling its job several times."""
    jobs = _jobs(qg)
    want = _sequential(jobs)
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(i):
        try:
            s = torch.cuda.Stream()
            run, outs = jobs[i]
            start.wait()
            for _ in range(5):
                with torch.cuda.stream(s):
                    run()
            s.synchronize()
        except Exception as e:          # reported below, on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i, ((_, outs), w) in enumerate(zip(jobs, want)):
        for o, wo in zip(outs, w):
            assert np.array_equal(raw(o), wo), f"job {i}"
