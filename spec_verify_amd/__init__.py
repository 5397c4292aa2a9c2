"""Python binding of libqgemm, the MI355X (gfx950) weight-only-int4 GEMM library.

Argument marshalling only: every function here checks nothing the C ABI does
not check itself, allocates outputs with torch when the caller passes none,
and calls the entry point of the same name in ``libqgemm.so`` on the current
torch stream.  All arithmetic runs in the library's HIP kernels.  If the
library has not been built the import fails; there is no fallback.

Entry points (see ``include/qgemm.h`` for the contract of each):
act_quant_int8, w4_repack, w4a16_gemm, w4a8_gemm, w4a8_prepare, rmsnorm_w4a8_prepare,
verify_attention_f16, sample_topk_topp,
w4a8_gemm_prepared, w4a8_gemm_debug,
w8a16_gemm, embed_gather_dequant_int8, quant_table_int8, the self-test
qg_selftest_quant_division, the diagnostic read qg_probe_read, plus the size helpers w4_packed_bytes,
w4_scales_bytes, qg_workspace_bytes and qg_status_string.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")

QG_OK, QG_ERR_INVALID_ARG, QG_ERR_UNSUPPORTED_SHAPE, QG_ERR_WORKSPACE, QG_ERR_LAUNCH = range(5)
QG_OP_W4A16, QG_OP_W4A8, QG_OP_W8A16 = 1, 2, 3

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(python spec_verify_amd/build.py)")

# torch ships its own HIP runtime (soname libamdhip64.so.7) and loads it by
# file name.  Importing torch first makes libqgemm's libamdhip64.so.7
# dependency resolve to that already-loaded runtime; loading libqgemm first
# would put a second HIP runtime in the process, one that does not see the
# device memory and streams torch hands us.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_SIGS = {
    "qg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qg_last_hip_error": (ctypes.c_char_p, []),
    "w4_packed_bytes": (_sz, [_i64, _i64]),
    "w4_scales_bytes": (_sz, [_i64, _i64]),
    "qg_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64]),
    "act_quant_int8": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "w4_repack": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _p]),
    "w4a16_gemm": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "w4a8_gemm": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "w4a8_prepared_bytes": (_sz, [_i64, _i64]),
    "w4a8_prepare": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _sz, _p]),
    "rmsnorm_w4a8_prepare": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, ctypes.c_float, _p, _p, _sz, _p]),
    "verify_attention_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "verify_attention_f16": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "sampler_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "sample_topk_topp": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float, _p, _p, _p, _p,
                                        _p, _p, _p, _sz, _p]),
    "w4a8_gemm_prepared": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "w4a8_gemm_debug": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p,
                                       _p, _p, _p, _i64, _i64, _i64, _i64]),
    "w8a16_gemm": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "embed_gather_dequant_int8": (ctypes.c_int, [_p, _i64, _p, _p, _i64, _i64, _p, _p]),
    "quant_table_int8": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "qg_selftest_quant_division": (ctypes.c_int, [_p, _p]),
    "qg_probe_read": (ctypes.c_int, [_p, _i64, _p, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p]),
    "w4a8_noalloc_scratch_bytes": (_sz, []),
    "w4a8_gemm_noalloc": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_SIGS)


class QGemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn}: status {status} ({qg_status_string(status)})"
        if status == QG_ERR_LAUNCH:
            msg += f": {lib.qg_last_hip_error().decode()}"
        super().__init__(msg)
        self.status = status


def qg_status_string(status: int) -> str:
    return lib.qg_status_string(int(status)).decode()


def w4_packed_bytes(N: int, K: int) -> int:
    return int(lib.w4_packed_bytes(N, K))


def w4_scales_bytes(N: int, K: int) -> int:
    return int(lib.w4_scales_bytes(N, K))


def qg_workspace_bytes(op: int, M: int, K: int, N: int) -> int:
    return int(lib.qg_workspace_bytes(op, M, K, N))


def _check(fn: str, status: int) -> None:
    if status != QG_OK:
        raise QGemmError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


def _ldx(x) -> int:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    return x.stride(0)


def act_quant_int8(x, q=None, scale=None):
    """Per-token int8 codes [M, K] and fp32 scales [M] of fp16 x [M, K]."""
    import torch
    M, K = x.shape
    q = _empty((M, K), torch.int8, x) if q is None else q
    scale = _empty((M,), torch.float32, x) if scale is None else scale
    _check("act_quant_int8", lib.act_quant_int8(_ptr(x), M, K, _ldx(x), _ptr(q), _ptr(scale), _stream(x.device)))
    return q, scale


def w4_repack(codes, scales):
    """Packed weights (uint8 [N*K/2]) and packed scales (fp16 [N, K/128])."""
    import torch
    N, K = codes.shape
    wp = _empty((max(1, w4_packed_bytes(N, K)),), torch.uint8, codes)
    sp = _empty((N, K // 128), torch.float16, codes)
    _check("w4_repack", lib.w4_repack(_ptr(codes), _ptr(scales), N, K, _ptr(wp), _ptr(sp), _stream(codes.device)))
    return wp, sp


def _workspace(op, M, K, N, like, workspace):
    import torch
    need = qg_workspace_bytes(op, M, K, N)
    if workspace is None and need > 0:
        workspace = _empty((need,), torch.uint8, like)
    size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, size


def w4a16_gemm(x, w_packed, s_packed, N, y=None, workspace=None):
    """fp16 y [M, N] = x [M, K] times the packed int4 weights (transposed)."""
    import torch
    M, K = x.shape
    y = _empty((M, N), torch.float16, x) if y is None else y
    ws, wsz = _workspace(QG_OP_W4A16, M, K, N, x, workspace)
    _check("w4a16_gemm", lib.w4a16_gemm(_ptr(x), M, K, N, _ldx(x), _ptr(w_packed), _ptr(s_packed), _ptr(y),
                                        _ptr(ws), wsz, _stream(x.device)))
    return y


def w4a8_gemm(x, w_packed, s_packed, N, y=None, workspace=None):
    """fp16 y [M, N]: x quantised per token to int8 inside the call, int8 x int4."""
    import torch
    M, K = x.shape
    y = _empty((M, N), torch.float16, x) if y is None else y
    ws, wsz = _workspace(QG_OP_W4A8, M, K, N, x, workspace)
    _check("w4a8_gemm", lib.w4a8_gemm(_ptr(x), M, K, N, _ldx(x), _ptr(w_packed), _ptr(s_packed), _ptr(y),
                                      _ptr(ws), wsz, _stream(x.device)))
    return y


def w4a8_gemm_noalloc(x, w_packed, s_packed, N, y):
    """y = the W4A8 product of fp16 x [M, K] with packed weights, through the
    entry point that takes no workspace (its scratch is a device array inside
    the library).  The caller passes y (fp16 [M, N]); nothing is allocated."""
    M, K = x.shape
    _check("w4a8_gemm_noalloc", lib.w4a8_gemm_noalloc(_ptr(x), M, K, N, _ldx(x), _ptr(w_packed), _ptr(s_packed),
                                                      _ptr(y), _stream(x.device)))
    return y


def w4a8_prepared_bytes(M: int, K: int) -> int:
    return int(lib.w4a8_prepared_bytes(M, K))


def w4a8_prepare(x, prepared=None):
    """Quantise x [M, K] per token into an opaque prepared buffer (uint8) for
    w4a8_gemm_prepared."""
    import torch
    M, K = x.shape
    need = w4a8_prepared_bytes(M, K)
    prepared = _empty((max(1, need),), torch.uint8, x) if prepared is None else prepared
    _check("w4a8_prepare", lib.w4a8_prepare(_ptr(x), M, K, _ldx(x), _ptr(prepared),
                                            prepared.numel() * prepared.element_size(), _stream(x.device)))
    return prepared


def rmsnorm_w4a8_prepare(x, w, eps, prepared=None, y=None, want_y=True):
    """RMSNorm of x [M, H] with weight w [H], fused with the W4A8 quantiser:
    returns (y fp16 [M, H] or None, prepared) where prepared is what
    w4a8_prepare(y) would write."""
    import torch
    M, H = x.shape
    need = w4a8_prepared_bytes(M, H)
    prepared = _empty((max(1, need),), torch.uint8, x) if prepared is None else prepared
    if want_y and y is None:
        y = _empty((M, H), torch.float16, x)
    _check("rmsnorm_w4a8_prepare",
           lib.rmsnorm_w4a8_prepare(_ptr(x), _ptr(w), M, H, _ldx(x), float(eps), _ptr(y) if want_y else None,
                                    _ptr(prepared), prepared.numel() * prepared.element_size(), _stream(x.device)))
    return (y if want_y else None), prepared


def verify_attention_workspace_bytes(T: int, Hq: int, Hkv: int, L: int) -> int:
    return int(lib.verify_attention_workspace_bytes(T, Hq, Hkv, L))


def verify_attention_f16(q, k_cache, v_cache, o=None, workspace=None):
    """Split-KV attention of q [T, Hq, 256] over the cache k, v [L, Hkv, 256]
    (the T query tokens are its last T positions, causal among themselves);
    returns o [T, Hq, 256] fp16."""
    import torch
    T, Hq, _ = q.shape
    L, Hkv, _ = k_cache.shape
    o = _empty((T, Hq, 256), torch.float16, q) if o is None else o
    need = verify_attention_workspace_bytes(T, Hq, Hkv, L)
    if workspace is None:
        workspace = _empty((max(16, need if need != 2 ** 64 - 1 else 16),), torch.uint8, q)
    _check("verify_attention_f16",
           lib.verify_attention_f16(_ptr(q), _ptr(k_cache), _ptr(v_cache), T, Hq, Hkv, L, _ptr(o), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(q.device)))
    return o


def sampler_workspace_bytes(R: int, V: int, k: int) -> int:
    return int(lib.sampler_workspace_bytes(R, V, k))


def sample_topk_topp(logits, u, k, top_p, temperature, V=None, out=None, workspace=None):
    """Top-k / top-p sampling of fp16 logits [R, >= V] with uniforms u [R]
    (fp32).  Returns (ids int32 [R, k], probs fp32 [R, k], kept int32 [R],
    sampled int32 [R], lse fp32 [R])."""
    import torch
    R = logits.shape[0]
    V = logits.shape[1] if V is None else V
    if out is None:
        out = (_empty((R, k), torch.int32, logits), _empty((R, k), torch.float32, logits),
               _empty((R,), torch.int32, logits), _empty((R,), torch.int32, logits),
               _empty((R,), torch.float32, logits))
    ids, probs, kept, sampled, lse = out
    need = sampler_workspace_bytes(R, V, k)
    if workspace is None:
        workspace = _empty((max(16, need if need != 2 ** 64 - 1 else 16),), torch.uint8, logits)
    _check("sample_topk_topp",
           lib.sample_topk_topp(_ptr(logits), R, V, _ldx(logits) if R > 0 else V, k, float(top_p), float(temperature),
                                _ptr(u), _ptr(ids), _ptr(probs), _ptr(kept), _ptr(sampled), _ptr(lse),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(logits.device)))
    return ids, probs, kept, sampled, lse


def w4a8_gemm_prepared(prepared, M, K, w_packed, s_packed, N, y=None):
    """fp16 y [M, N] from a buffer made by w4a8_prepare (one kernel launch)."""
    import torch
    y = _empty((M, N), torch.float16, prepared) if y is None else y
    _check("w4a8_gemm_prepared", lib.w4a8_gemm_prepared(_ptr(prepared), M, K, N, _ptr(w_packed), _ptr(s_packed),
                                                        _ptr(y), _stream(prepared.device)))
    return y


def w4a8_gemm_debug(x, w_packed, s_packed, N, window=None, y=None, workspace=None):
    """w4a8_gemm plus its integer stages: returns (y, q, scale, partials) where
    partials is int32 [m1-m0, n1-n0, K/128] for window = (m0, m1, n0, n1)."""
    import torch
    M, K = x.shape
    m0, m1, n0, n1 = window if window is not None else (0, M, 0, N)
    y = _empty((M, N), torch.float16, x) if y is None else y
    q = _empty((M, K), torch.int8, x)
    sc = _empty((M,), torch.float32, x)
    part = _empty((max(0, m1 - m0), max(0, n1 - n0), K // 128), torch.int32, x)
    ws, wsz = _workspace(QG_OP_W4A8, M, K, N, x, workspace)
    _check("w4a8_gemm_debug", lib.w4a8_gemm_debug(
        _ptr(x), M, K, N, _ldx(x), _ptr(w_packed), _ptr(s_packed), _ptr(y), _ptr(ws), wsz, _stream(x.device),
        _ptr(q), _ptr(sc), _ptr(part) if part.numel() else None, m0, m1, n0, n1))
    return y, q, sc, part


def w8a16_gemm(x, w, s, y=None, workspace=None):
    """fp16 y [M, N] = x [M, K] times the row-major int8 table w [N, K] (transposed)."""
    import torch
    M, K = x.shape
    N = w.shape[0]
    y = _empty((M, N), torch.float16, x) if y is None else y
    ws, wsz = _workspace(QG_OP_W8A16, M, K, N, x, workspace)
    _check("w8a16_gemm", lib.w8a16_gemm(_ptr(x), M, K, N, _ldx(x), _ptr(w), _ptr(s), _ptr(y),
                                        _ptr(ws), wsz, _stream(x.device)))
    return y


def embed_gather_dequant_int8(ids, table, scales, out=None):
    """fp16 rows [T, H] of the int8 table for int32 ids [T]."""
    import torch
    T = ids.shape[0]
    V, H = table.shape
    out = _empty((T, H), torch.float16, table) if out is None else out
    _check("embed_gather_dequant_int8", lib.embed_gather_dequant_int8(
        _ptr(ids), T, _ptr(table), _ptr(scales), V, H, _ptr(out), _stream(table.device)))
    return out


def quant_table_int8(src_bf16, Q=None, S=None):
    """int8 table [V, H] and fp16 group scales [V, H/128] of a bf16 table."""
    import torch
    V, H = src_bf16.shape
    Q = _empty((V, H), torch.int8, src_bf16) if Q is None else Q
    S = _empty((V, H // 128), torch.float16, src_bf16) if S is None else S
    _check("quant_table_int8", lib.quant_table_int8(_ptr(src_bf16), V, H, _ptr(Q), _ptr(S),
                                                    _stream(src_bf16.device)))
    return Q, S


def qg_probe_read(a, c=None, share=1, wgs=256, threads=512, nontemporal=True, sink=None):
    """Run the library's diagnostic read over the device tensors a (and c)
    with the given split (see qg_probe_read in qgemm.h); returns the sink."""
    import torch
    if sink is None:
        sink = torch.empty((wgs * threads // 64,), dtype=torch.int32, device=a.device)
    c_ptr, c_bytes = (None, 0) if c is None else (_ptr(c), c.numel() * c.element_size())
    _check("qg_probe_read", lib.qg_probe_read(_ptr(a), a.numel() * a.element_size(), c_ptr, c_bytes, share, wgs,
                                              threads, 1 if nontemporal else 0, _ptr(sink), _stream(a.device)))
    return sink


def qg_selftest_quant_division(device=None):
    """Run the library's exhaustive check of the quantiser's division on the
    device; returns (pairs checked, pairs whose rounded quotients differ)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    counts = torch.zeros((2,), dtype=torch.int64, device=dev)
    _check("qg_selftest_quant_division", lib.qg_selftest_quant_division(_ptr(counts), _stream(dev)))
    c = counts.cpu()
    return int(c[0]), int(c[1])
