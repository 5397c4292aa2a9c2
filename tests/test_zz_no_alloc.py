"""w4a8_gemm_noalloc, the W4A8 entry point that takes no workspace (its
codes and token scales live in a device array inside the library), against
w4a8_gemm through the C ABI: two calls in a row, the second smaller, each
bit-identical to w4a8_gemm on the same inputs and within the fp16 bounds of
the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _bits(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def test_noalloc_matches_w4a8_gemm_on_two_calls_in_a_row():
    import spec_verify_amd as qg
    cases = [(64, 5120, 5120, 1), (5, 2560, 1040, 7)]      # the second call is smaller
    for M, K, N, seed in cases:
        x = synth.acts(M, K, 1.0, 0.01, 20.0, seed=seed + 100)
        codes, scales = synth.weights(N, K, seed=seed)
        wp, sp = qg.w4_repack(_dev(codes), _dev(scales))
        xd = _dev(x)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        qg.w4a8_gemm_noalloc(xd, wp, sp, N, y)
        want = qg.w4a8_gemm(xd, wp, sp, N)
        assert np.array_equal(_bits(y), _bits(want)), (M, K, N)
        r = oracle.fp16_bounds(y.cpu().numpy(), oracle.ref_w4a8(x, codes, scales))
        assert r["ok"], (M, K, N, r)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    import spec_verify_amd as qg
    x = torch.zeros((64, 131072), dtype=torch.float16, device=DEV)
    y = torch.zeros((64, 16), dtype=torch.float16, device=DEV)
    w = torch.zeros((16 * 131072 // 2,), dtype=torch.uint8, device=DEV)
    s = torch.zeros((16, 1024), dtype=torch.float16, device=DEV)
    with pytest.raises(qg.QGemmError):
        qg.w4a8_gemm_noalloc(x, w, s, 16, y)
