"""The diagnostic read (qg_probe_read) reads exactly the slices its contract
assigns: its per-wave checksums equal those formed on the host from the
same slice and thread assignment."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import spec_verify_amd
    return spec_verify_amd


def expected_sink(a, c, share, wgs, threads):
    """Host model: workgroup b -> lin (the row split's XCD walk), slice
    lin // share of a and lin % share of c; thread t XORs the four words of
    its 16-byte chunks t, t + threads, ...; a wave's word is the XOR of its
    threads'."""
    per = wgs // 8
    out = np.zeros(wgs * threads // 64, np.uint32)
    na = wgs // share
    for b in range(wgs):
        lin = (b % 8) * per + b // 8 if wgs % 8 == 0 and per % share == 0 else b
        sa, sc = lin // share, lin % share
        acc = np.zeros(threads, np.uint32)
        for buf, nslices, s in ((a, na, sa), (c, share, sc)):
            if buf is None:
                continue
            n = buf.size
            lo, hi = n * s // nslices, n * (s + 1) // nslices
            words = buf[lo:hi].view(np.uint32).reshape(-1, 4)
            chunk_x = np.bitwise_xor.reduce(words, axis=1)
            for k in range(chunk_x.size):
                acc[k % threads] ^= chunk_x[k]
        for w in range(threads // 64):
            out[b * (threads // 64) + w] = np.bitwise_xor.reduce(acc[64 * w:64 * (w + 1)])
    return out


@pytest.mark.parametrize("share,wgs,threads,with_c", [(1, 32, 128, False), (2, 32, 512, True), (4, 32, 256, True),
                                                    (4, 24, 192, True)])
def test_probe_reads_its_slices(qg, share, wgs, threads, with_c):
    rng = np.random.default_rng(wgs * 7 + share)
    a = rng.integers(0, 256, size=wgs // share * 16 * 37, dtype=np.uint8)   # slices of 37 chunks
    c = rng.integers(0, 256, size=share * 16 * 11, dtype=np.uint8) if with_c else None
    dev = torch.device("cuda:0")
    ad = torch.from_numpy(a).to(dev)
    cd = torch.from_numpy(c).to(dev) if with_c else None
    sink = qg.qg_probe_read(ad, cd, share, wgs, threads, True)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_sink(a, c, share, wgs, threads))
