"""The C ABI on the host: the library loads, exports every entry point the
header declares, sizes buffers as documented and rejects bad arguments with
the documented status before launching anything (CPU only: every call here
fails validation, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

import spec_verify_amd as qg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qgemm.h")

FAKE = ctypes.c_void_p(1 << 20)           # aligned, never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 8)      # 8-byte aligned only


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", src, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(qg.lib, n), n
    assert set(names) == set(qg.EXPORTS)


def test_status_strings():
    assert qg.qg_status_string(0) == "ok"
    for s in range(1, 5):
        assert qg.qg_status_string(s) and qg.qg_status_string(s) != "unknown status"
    assert qg.qg_status_string(99) == "unknown status"


def test_size_helpers():
    assert qg.w4_packed_bytes(5120, 5120) == 5120 * 5120 // 2
    assert qg.w4_scales_bytes(5120, 5120) == 5120 * 40 * 2
    assert qg.w4_packed_bytes(5120, 100) == 0 and qg.w4_packed_bytes(17, 128) == 0
    big = qg.qg_workspace_bytes(qg.QG_OP_W4A8, 4096, 17408, 5120)
    assert big >= 4096 * 17408 + 4096 * 4
    dec = qg.qg_workspace_bytes(qg.QG_OP_W4A8, 64, 5120, 5120)
    assert dec >= 64 * 5120 + 64 * 4
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 0, 5120, 5120) == 0
    assert qg.qg_workspace_bytes(7, 1, 128, 16) == 2 ** 64 - 1
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 1, 100, 16) == 2 ** 64 - 1
    # small batches keep their codes in 16-row tiles, so the workspace rounds M up to 16
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 1, 5120, 5120) >= 16 * 5120 + 4


GEMMS = ["w4a16_gemm", "w4a8_gemm", "w8a16_gemm"]


def call_gemm(name, M=4, K=256, N=32, ldx=None, x=FAKE, w=FAKE, s=FAKE, y=FAKE, ws=None, wsb=0):
    f = getattr(qg.lib, name)
    return f(x, M, K, N, K if ldx is None else ldx, w, s, y, ws, wsb, None)


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_shape_errors(name):
    assert call_gemm(name, K=200) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call_gemm(name, N=40) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call_gemm(name, M=-1) == qg.QG_ERR_INVALID_ARG
    assert call_gemm(name, K=0) == qg.QG_ERR_INVALID_ARG
    assert call_gemm(name, ldx=128) == qg.QG_ERR_INVALID_ARG       # ldx < K
    assert call_gemm(name, ldx=260) == qg.QG_ERR_INVALID_ARG       # rows not 16-byte aligned
    assert call_gemm(name, M=2 ** 31) == qg.QG_ERR_UNSUPPORTED_SHAPE


@pytest.mark.parametrize("name", GEMMS)
def test_gemm_pointer_errors(name):
    assert call_gemm(name, x=None) == qg.QG_ERR_INVALID_ARG
    assert call_gemm(name, w=None) == qg.QG_ERR_INVALID_ARG
    assert call_gemm(name, y=MIS) == qg.QG_ERR_INVALID_ARG
    assert call_gemm(name, s=MIS) == qg.QG_ERR_INVALID_ARG
    # an empty batch needs no pointers at all
    assert call_gemm(name, M=0, x=None, w=None, s=None, y=None) == qg.QG_OK


def test_fp16_activation_gemms_limit_k():
    """w4a16_gemm / w8a16_gemm keep a workgroup's group scales in LDS, so K is
    capped at 65536; W4A8 is not."""
    K = 65536 + 128
    assert call_gemm("w4a16_gemm", M=4, K=K, N=32) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call_gemm("w8a16_gemm", M=4, K=K, N=32) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 4, K, 32) == 2 ** 64 - 1
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 4, 65536, 32) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 4, K, 32) > 0


def test_w4a8_limits_k():
    """w4a8_gemm addresses a workgroup's operand block with 32-bit buffer
    offsets, so K is capped at 2^22."""
    K = (1 << 22) + 128
    assert call_gemm("w4a8_gemm", M=4, K=K, N=32, ws=FAKE, wsb=1 << 40) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 4, K, 32) == 2 ** 64 - 1
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A8, 4, 1 << 22, 32) > 0


def test_workspace_errors():
    need = qg.qg_workspace_bytes(qg.QG_OP_W4A8, 64, 5120, 5120)
    assert call_gemm("w4a8_gemm", M=64, K=5120, N=5120, ws=None, wsb=0) == qg.QG_ERR_WORKSPACE
    assert call_gemm("w4a8_gemm", M=64, K=5120, N=5120, ws=FAKE, wsb=need - 1) == qg.QG_ERR_WORKSPACE
    assert call_gemm("w4a8_gemm", M=64, K=5120, N=5120, ws=MIS, wsb=need) == qg.QG_ERR_INVALID_ARG
    # the weight-streaming W4A16 / W8A16 GEMMs need no workspace
    assert qg.qg_workspace_bytes(qg.QG_OP_W4A16, 16, 5120, 5120) == 0
    assert qg.qg_workspace_bytes(qg.QG_OP_W8A16, 64, 5120, 248320) == 0


def test_debug_window_errors():
    f = qg.lib.w4a8_gemm_debug
    need = qg.qg_workspace_bytes(qg.QG_OP_W4A8, 4, 256, 32)
    args = [FAKE, 4, 256, 32, 256, FAKE, FAKE, FAKE, FAKE, need, None, None, None, FAKE]
    assert f(*args, 0, 5, 0, 32) == qg.QG_ERR_INVALID_ARG
    assert f(*args, 2, 1, 0, 32) == qg.QG_ERR_INVALID_ARG
    assert f(*args, 0, 4, 0, 33) == qg.QG_ERR_INVALID_ARG
    assert f(*args, -1, 4, 0, 32) == qg.QG_ERR_INVALID_ARG


def test_quantiser_repack_gather_table_errors():
    L = qg.lib
    assert L.act_quant_int8(FAKE, 4, 200, 200, FAKE, FAKE, None) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert L.act_quant_int8(FAKE, 4, 256, 128, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.act_quant_int8(None, 4, 256, 256, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.act_quant_int8(None, 0, 256, 256, None, None, None) == qg.QG_OK
    assert L.w4_repack(FAKE, FAKE, 24, 256, FAKE, FAKE, None) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert L.w4_repack(FAKE, FAKE, 32, 256, None, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.w4_repack(FAKE, FAKE, 0, 256, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.embed_gather_dequant_int8(FAKE, 4, FAKE, FAKE, 10, 100, FAKE, None) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert L.embed_gather_dequant_int8(FAKE, -1, FAKE, FAKE, 10, 128, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.embed_gather_dequant_int8(FAKE, 4, FAKE, FAKE, 0, 128, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.embed_gather_dequant_int8(None, 4, FAKE, FAKE, 10, 128, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert L.embed_gather_dequant_int8(None, 0, None, None, 10, 128, None, None) == qg.QG_OK
    assert L.quant_table_int8(FAKE, 10, 100, FAKE, FAKE, None) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert L.quant_table_int8(FAKE, 10, 128, MIS, FAKE, None) == qg.QG_ERR_INVALID_ARG


def test_rmsnorm_prepare_errors():
    """Shape, eps, pointer and buffer-size checks of the fused norm+quantiser,
    all on the host before any launch."""
    f = qg.lib.rmsnorm_w4a8_prepare
    need = qg.w4a8_prepared_bytes(4, 256)

    def call(M=4, H=256, ldx=None, eps=1e-6, x=FAKE, w=FAKE, y=FAKE, p=FAKE, pb=need):
        return f(x, w, M, H, H if ldx is None else ldx, eps, y, p, pb, None)

    assert call(H=200) == qg.QG_ERR_UNSUPPORTED_SHAPE             # H % 128
    assert call(H=65536 + 128, pb=2 ** 40) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call(M=-1) == qg.QG_ERR_INVALID_ARG
    assert call(ldx=128) == qg.QG_ERR_INVALID_ARG
    assert call(eps=-1e-6) == qg.QG_ERR_INVALID_ARG
    assert call(eps=float("nan")) == qg.QG_ERR_INVALID_ARG
    assert call(eps=float("inf")) == qg.QG_ERR_INVALID_ARG
    assert call(w=None) == qg.QG_ERR_INVALID_ARG
    assert call(y=MIS) == qg.QG_ERR_INVALID_ARG
    assert call(pb=need - 1) == qg.QG_ERR_WORKSPACE
    assert call(M=0, x=None, w=None, y=None, p=None, pb=0) == qg.QG_OK


def test_verify_attention_errors():
    f = qg.lib.verify_attention_f16
    need = qg.verify_attention_workspace_bytes(5, 24, 4, 1536)
    assert 0 < need < 2 ** 40

    def call(T=5, Hq=24, Hkv=4, L=1536, q=FAKE, k=FAKE, v=FAKE, o=FAKE, ws=FAKE, wsb=need):
        return f(q, k, v, T, Hq, Hkv, L, o, ws, wsb, None)

    assert call(T=0) == qg.QG_ERR_INVALID_ARG
    assert call(Hkv=5) == qg.QG_ERR_UNSUPPORTED_SHAPE              # Hq % Hkv
    assert call(T=17) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call(T=16, Hq=24, Hkv=2) == qg.QG_ERR_UNSUPPORTED_SHAPE  # 12 heads per group x 16 queries > 128 rows
    assert call(L=4) == qg.QG_ERR_UNSUPPORTED_SHAPE                 # L < T
    assert call(q=None) == qg.QG_ERR_INVALID_ARG
    assert call(o=MIS) == qg.QG_ERR_INVALID_ARG
    assert call(wsb=need - 1) == qg.QG_ERR_WORKSPACE
    assert call(ws=None) == qg.QG_ERR_WORKSPACE
    assert call(ws=MIS) == qg.QG_ERR_INVALID_ARG
    assert qg.verify_attention_workspace_bytes(17, 24, 4, 100) == 2 ** 64 - 1


def call_sampler(R=2, V=1000, ld=None, k=20, p=0.95, T=1.0, x=FAKE, u=FAKE, out=FAKE, ws=FAKE, wsb=None):
    wsb = qg.sampler_workspace_bytes(max(R, 1), V, k) if wsb is None else wsb
    return qg.lib.sample_topk_topp(x, R, V, V if ld is None else ld, k, p, T, u, out, out, out, out, out, ws, wsb,
                                   None)


def test_sampler_sizes():
    assert qg.sampler_workspace_bytes(64, 248320, 20) > 64 * 20 * 8
    assert qg.sampler_workspace_bytes(1, 100, 65) == 2 ** 64 - 1         # k > 64
    assert qg.sampler_workspace_bytes(1, 10, 11) == 2 ** 64 - 1          # k > V
    assert qg.sampler_workspace_bytes(1, 2 ** 24, 8) == 2 ** 64 - 1      # ids beyond 24 bits
    assert qg.sampler_workspace_bytes(1, 8192 * 257, 64) == 2 ** 64 - 1  # more candidates than pass 2 holds
    assert qg.sampler_workspace_bytes(1, 8192 * 256, 64) != 2 ** 64 - 1


def test_sampler_argument_errors():
    assert call_sampler(k=0) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(k=65) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert call_sampler(R=-1) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(p=0.0) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(p=1.5) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(p=float("nan")) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(T=0.0) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(T=float("inf")) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(ld=1004) == qg.QG_ERR_INVALID_ARG                # rows not 16-byte aligned
    assert call_sampler(ld=992) == qg.QG_ERR_INVALID_ARG                 # ld < V
    assert call_sampler(x=None) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(x=MIS) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(u=None) == qg.QG_ERR_INVALID_ARG
    assert call_sampler(ws=None) == qg.QG_ERR_WORKSPACE
    assert call_sampler(wsb=16) == qg.QG_ERR_WORKSPACE
    assert call_sampler(ws=MIS) == qg.QG_ERR_INVALID_ARG
    # no rows: nothing to do, no pointers needed
    assert call_sampler(R=0, x=None, u=None, out=None, ws=None, wsb=0) == qg.QG_OK


def test_probe_read_argument_errors():
    """The diagnostic read rejects its bad arguments on the host, before any
    device call."""
    f = qg.lib.qg_probe_read
    ok = dict(a=FAKE, ab=1 << 20, c=None, cb=0, share=4, wgs=256, threads=512, nt=1, sink=FAKE)

    def call(**kw):
        v = dict(ok, **kw)
        return f(v["a"], v["ab"], v["c"], v["cb"], v["share"], v["wgs"], v["threads"], v["nt"], v["sink"], None)
    assert call(a=None) == qg.QG_ERR_INVALID_ARG             # bytes without a pointer
    assert call(c=None, cb=64) == qg.QG_ERR_INVALID_ARG
    assert call(ab=-1) == qg.QG_ERR_INVALID_ARG
    assert call(sink=None) == qg.QG_ERR_INVALID_ARG
    assert call(share=0) == qg.QG_ERR_INVALID_ARG
    assert call(wgs=258) == qg.QG_ERR_INVALID_ARG            # not a multiple of share
    assert call(wgs=2, share=4) == qg.QG_ERR_INVALID_ARG
    assert call(threads=100) == qg.QG_ERR_INVALID_ARG        # not a multiple of 64
    assert call(threads=1088) == qg.QG_ERR_INVALID_ARG
    assert call(wgs=4, share=4, ab=1 << 31) == qg.QG_ERR_UNSUPPORTED_SHAPE   # a 2 GiB slice


def test_selftest_rejects_bad_counters():
    assert qg.lib.qg_selftest_quant_division(None, None) == qg.QG_ERR_INVALID_ARG
    assert qg.lib.qg_selftest_quant_division(ctypes.c_void_p((1 << 20) + 4), None) == qg.QG_ERR_INVALID_ARG


def test_noalloc_gemm_rejects_shapes_beyond_its_scratch():
    limit = qg.lib.w4a8_noalloc_scratch_bytes()
    assert limit == 8 << 20
    assert qg.lib.w4a8_prepared_bytes(64, 130944) <= limit < qg.lib.w4a8_prepared_bytes(64, 131072)
    f = qg.lib.w4a8_gemm_noalloc
    assert f(FAKE, 64, 131072, 16, 131072, FAKE, FAKE, FAKE, None) == qg.QG_ERR_WORKSPACE
    assert f(FAKE, 4096, 2048, 16, 2048, FAKE, FAKE, FAKE, None) == qg.QG_ERR_WORKSPACE
    assert f(FAKE, 0, 256, 16, 256, FAKE, FAKE, FAKE, None) == qg.QG_OK
    assert f(FAKE, 4, 200, 16, 200, FAKE, FAKE, FAKE, None) == qg.QG_ERR_UNSUPPORTED_SHAPE
    assert f(MIS, 4, 256, 16, 256, FAKE, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG
    assert f(None, 4, 256, 16, 256, FAKE, FAKE, FAKE, None) == qg.QG_ERR_INVALID_ARG


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With no built library the package import raises; there is no fallback
    path that could compute anything elsewhere."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "spec_verify_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "spec_verify_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import spec_verify_amd"], cwd=str(tmp_path), capture_output=True,
                       text=True, env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is missing" in r.stderr, r.stderr[-2000:]


def test_product_sources_never_reference_the_oracle():
    """The kernels, the C ABI and the binding neither import nor mention the
    CPU oracle: it is test infrastructure only."""
    seen = 0
    for d in ("spec_verify_amd", "include"):
        for base, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith((".py", ".hip", ".cpp", ".h", ".c")):
                    seen += 1
                    assert "oracle" not in open(os.path.join(base, f), errors="replace").read().lower(), f
    assert seen >= 10
