// C-ABI entry points of libqgemm: host-side validation, workspace layout and
// dispatch to the gfx950 kernels.  Nothing here allocates device memory or
// synchronises the host; every check happens before the first launch.
#include <atomic>
#include <cmath>
#include <mutex>
#include "qgemm.h"

#include <stdint.h>

#include "common.h"

namespace {

using qg::kGroup;

constexpr int64_t kMaxDim = INT32_MAX;     // kernels index rows/columns with 32-bit ints
// Longest K: the kernels address one workgroup's operand block (up to 128
// rows of K bytes, or 64 rows of K fp16) with 32-bit buffer offsets.
constexpr int64_t kMaxK = int64_t(1) << 22;
constexpr int64_t kSkinnyMaxM = 64;         // largest M the weight-streaming kernel takes per launch
// Longest K of w4a16_gemm / w8a16_gemm: their kernel keeps a workgroup's
// group scales (64 columns x K/128 groups of fp16) in LDS.
constexpr int64_t kMaxK16 = 65536;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// HIP error behind the calling thread's most recent QG_ERR_LAUNCH.
thread_local hipError_t t_last_hip_error = hipSuccess;

inline int launch_status(hipError_t e) {
  if (e == hipSuccess) return QG_OK;
  t_last_hip_error = e;
  return QG_ERR_LAUNCH;
}

// hipGetLastError reports the thread's last error from any earlier runtime
// call, not only from our launches; drop such a stale error before launching
// so that a launch is judged by its own result.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Shape checks shared by the three GEMMs.
int check_gemm_shape(int64_t M, int64_t K, int64_t N, int64_t ldx) {
  if (M < 0 || K <= 0 || N <= 0) return QG_ERR_INVALID_ARG;
  if (K % kGroup != 0 || N % 16 != 0) return QG_ERR_UNSUPPORTED_SHAPE;
  if (M > kMaxDim || K > kMaxK || N > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  if (ldx < K || ldx % 8 != 0 || ldx > kMaxK) return QG_ERR_INVALID_ARG;
  return QG_OK;
}

int check_ptrs(int64_t M, const void* x, const void* w, const void* s, const void* y) {
  if (M == 0) return QG_OK;
  if (!x || !w || !s || !y) return QG_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return QG_ERR_INVALID_ARG;
  return QG_OK;
}

// Workspace layout of w4a8_gemm: the int8 activation codes (fragment order
// in tiles of 16 rows for the weight-streaming kernel, M <= 64; row-major
// [M][K] for the tiled kernel), then the fp32 token scales [M], each on a
// 256-byte boundary.
struct W4A8Layout {
  size_t q_off, s_off, total;
};

W4A8Layout w4a8_layout(int64_t M, int64_t K) {
  W4A8Layout L;
  const int64_t rows = M <= kSkinnyMaxM ? (M + 15) / 16 * 16 : M;
  L.q_off = 0;
  L.s_off = round_up((size_t)rows * (size_t)K, 256);
  L.total = L.s_off + (size_t)M * 4;
  return L;
}

int gemm_streaming(int mode, const void* x, int64_t M, int64_t K, int64_t N, int64_t ldx,
                   const void* w, const void* s, void* y, void* ws, size_t ws_bytes, void* stream) {
  int st = check_gemm_shape(M, K, N, ldx);
  if (st != QG_OK) return st;
  if (K > kMaxK16) return QG_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_ptrs(M, x, w, s, y)) != QG_OK) return st;
  if (M == 0) return QG_OK;
  (void)ws;
  (void)ws_bytes;
  clear_stale_error();
  for (int64_t m0 = 0; m0 < M; m0 += kSkinnyMaxM) {
    qg::SkinnyArgs a = {};
    a.mode = mode;
    a.act = reinterpret_cast<const uint16_t*>(x) + m0 * ldx;
    a.lda = ldx;
    a.tok_scale = nullptr;
    a.w = w;
    a.s = reinterpret_cast<const uint16_t*>(s);
    a.M = (M - m0) < kSkinnyMaxM ? (M - m0) : kSkinnyMaxM;
    a.N = N;
    a.K = K;
    a.y = reinterpret_cast<uint16_t*>(y) + m0 * N;
    a.dbg = nullptr;
    st = launch_status(qg::launch_skinny(a, as_stream(stream)));
    if (st != QG_OK) return st;
  }
  return QG_OK;
}

int check_w4a8_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0) return QG_ERR_INVALID_ARG;
  if (K % kGroup != 0 || N % 16 != 0) return QG_ERR_UNSUPPORTED_SHAPE;
  if (M > kMaxDim || K > kMaxK || N > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  return QG_OK;
}

// Quantise x into a prepared buffer (codes in the order the GEMM for this M
// reads, then the token scales).  q_row: optional extra row-major copy.
int prepare_impl(const void* x, int64_t M, int64_t K, int64_t ldx, void* prepared, int8_t* q_row,
                 hipStream_t hs) {
  const W4A8Layout L = w4a8_layout(M, K);
  char* base = reinterpret_cast<char*>(prepared);
  int8_t* q = reinterpret_cast<int8_t*>(base + L.q_off);
  float* ts = reinterpret_cast<float*>(base + L.s_off);
  const bool skinny = M <= kSkinnyMaxM;
  // Codes: fragment order for the weight-streaming kernel, row-major for the
  // tiled one; the optional extra copy is always row-major.
  return launch_status(qg::launch_act_quant(reinterpret_cast<const uint16_t*>(x), M, K, ldx,
                                            skinny ? q_row : q, K, skinny ? q : nullptr, ts, hs));
}

int gemm_prepared_impl(const void* prepared, int64_t M, int64_t K, int64_t N, const void* w_packed,
                       const void* s_packed, void* y, hipStream_t hs, int32_t* dbg, int64_t m0, int64_t m1,
                       int64_t n0, int64_t n1) {
  const W4A8Layout L = w4a8_layout(M, K);
  const char* base = reinterpret_cast<const char*>(prepared);
  const int8_t* q = reinterpret_cast<const int8_t*>(base + L.q_off);
  const float* ts = reinterpret_cast<const float*>(base + L.s_off);
  if (M <= kSkinnyMaxM) {
    qg::SkinnyArgs a = {};
    a.mode = qg::kW4A8;
    a.act = q;
    a.lda = K;
    a.tok_scale = ts;
    a.w = w_packed;
    a.s = reinterpret_cast<const uint16_t*>(s_packed);
    a.M = M; a.N = N; a.K = K;
    a.y = reinterpret_cast<uint16_t*>(y);
    a.dbg = dbg;
    a.dm0 = m0; a.dm1 = m1; a.dn0 = n0; a.dn1 = n1;
    return launch_status(qg::launch_skinny(a, hs));
  }
  qg::LargeArgs a = {};
  a.codes = q;
  a.tok_scale = ts;
  a.w = w_packed;
  a.s = reinterpret_cast<const uint16_t*>(s_packed);
  a.M = M; a.N = N; a.K = K;
  a.y = reinterpret_cast<uint16_t*>(y);
  a.dbg = dbg;
  a.dm0 = m0; a.dm1 = m1; a.dn0 = n0; a.dn1 = n1;
  return launch_status(qg::launch_w4a8_large(a, hs));
}

int w4a8_impl(const void* x, int64_t M, int64_t K, int64_t N, int64_t ldx, const void* w_packed,
              const void* s_packed, void* y, void* ws, size_t ws_bytes, void* stream, int8_t* q_out,
              float* scale_out, int32_t* partials, int64_t m0, int64_t m1, int64_t n0, int64_t n1) {
  int st = check_gemm_shape(M, K, N, ldx);
  if (st != QG_OK) return st;
  if ((st = check_ptrs(M, x, w_packed, s_packed, y)) != QG_OK) return st;
  if (partials && !(0 <= m0 && m0 <= m1 && m1 <= M && 0 <= n0 && n0 <= n1 && n1 <= N))
    return QG_ERR_INVALID_ARG;
  if (M == 0) return QG_OK;
  const W4A8Layout L = w4a8_layout(M, K);
  if (!ws || ws_bytes < L.total) return QG_ERR_WORKSPACE;
  if (!aligned16(ws)) return QG_ERR_INVALID_ARG;
  if ((q_out && !aligned16(q_out)) || (partials && (reinterpret_cast<uintptr_t>(partials) & 3u)) ||
      (scale_out && (reinterpret_cast<uintptr_t>(scale_out) & 3u)))
    return QG_ERR_INVALID_ARG;
  hipStream_t hs = as_stream(stream);
  int32_t* dbg = (partials && m1 > m0 && n1 > n0) ? partials : nullptr;
  const bool skinny = M <= kSkinnyMaxM;

  clear_stale_error();
  st = prepare_impl(x, M, K, ldx, ws, skinny ? q_out : nullptr, hs);
  if (st != QG_OK) return st;
  st = gemm_prepared_impl(ws, M, K, N, w_packed, s_packed, y, hs, dbg, m0, m1, n0, n1);
  if (st != QG_OK) return st;
  const char* base = reinterpret_cast<const char*>(ws);
  if (!skinny && q_out &&
      (st = launch_status(hipMemcpyAsync(q_out, base + L.q_off, (size_t)M * K, hipMemcpyDeviceToDevice, hs))) != QG_OK)
    return st;
  if (scale_out &&
      (st = launch_status(hipMemcpyAsync(scale_out, base + L.s_off, (size_t)M * 4, hipMemcpyDeviceToDevice, hs))) != QG_OK)
    return st;
  return QG_OK;
}

}  // namespace

extern "C" {

const char* qg_status_string(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, negative size, ldx, window or op)";
    case QG_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (K and H must be multiples of 128, N of 16)";
    case QG_ERR_WORKSPACE: return "workspace smaller than qg_workspace_bytes()";
    case QG_ERR_LAUNCH: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* qg_last_hip_error(void) {
  return t_last_hip_error == hipSuccess ? "none" : hipGetErrorString(t_last_hip_error);
}

size_t w4_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % kGroup || N > kMaxDim || K > kMaxDim) return 0;
  return (size_t)N * (size_t)K / 2;
}

size_t w4_scales_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % kGroup || N > kMaxDim || K > kMaxDim) return 0;
  return (size_t)N * (size_t)(K / kGroup) * 2;
}

size_t qg_workspace_bytes(int op, int64_t M, int64_t K, int64_t N) {
  if (check_gemm_shape(M, K, N, K + (8 - K % 8) % 8) != QG_OK) return (size_t)-1;
  switch (op) {
    case QG_OP_W4A8: return M == 0 ? 0 : w4a8_layout(M, K).total;
    case QG_OP_W4A16:
    case QG_OP_W8A16: return K > kMaxK16 ? (size_t)-1 : 0;
    default: return (size_t)-1;
  }
}

int act_quant_int8(const void* x_f16, int64_t M, int64_t K, int64_t ldx, int8_t* q, float* scale,
                   void* stream) {
  if (M < 0 || K <= 0) return QG_ERR_INVALID_ARG;
  if (K % kGroup != 0 || M > kMaxDim || K > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  if (ldx < K || ldx % 8 != 0) return QG_ERR_INVALID_ARG;
  if (M == 0) return QG_OK;
  if (!x_f16 || !q || !scale || !aligned16(x_f16) || !aligned16(q) || !aligned16(scale))
    return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_act_quant(reinterpret_cast<const uint16_t*>(x_f16), M, K, ldx, q, K,
                                            nullptr, scale, as_stream(stream)));
}

int w4_repack(const int8_t* codes, const void* scales_f16, int64_t N, int64_t K, void* w_packed,
              void* s_packed, void* stream) {
  if (N <= 0 || K <= 0) return QG_ERR_INVALID_ARG;
  if (N % 16 || K % kGroup || N > kMaxDim || K > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  if (!codes || !scales_f16 || !w_packed || !s_packed) return QG_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales_f16) || !aligned16(w_packed) || !aligned16(s_packed))
    return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_w4_repack(codes, reinterpret_cast<const uint16_t*>(scales_f16), N, K,
                                            w_packed, reinterpret_cast<uint16_t*>(s_packed),
                                            as_stream(stream)));
}

int w4a16_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx, const void* w_packed,
               const void* s_packed, void* y_f16, void* workspace, size_t ws_bytes, void* stream) {
  return gemm_streaming(qg::kW4A16, x_f16, M, K, N, ldx, w_packed, s_packed, y_f16, workspace, ws_bytes,
                        stream);
}

int w4a8_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx, const void* w_packed,
              const void* s_packed, void* y_f16, void* workspace, size_t ws_bytes, void* stream) {
  return w4a8_impl(x_f16, M, K, N, ldx, w_packed, s_packed, y_f16, workspace, ws_bytes, stream, nullptr,
                   nullptr, nullptr, 0, 0, 0, 0);
}

int w4a8_gemm_debug(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx, const void* w_packed,
                    const void* s_packed, void* y_f16, void* workspace, size_t ws_bytes, void* stream,
                    int8_t* q_out, float* scale_out, int32_t* partials, int64_t m0, int64_t m1, int64_t n0,
                    int64_t n1) {
  return w4a8_impl(x_f16, M, K, N, ldx, w_packed, s_packed, y_f16, workspace, ws_bytes, stream, q_out,
                   scale_out, partials, m0, m1, n0, n1);
}

size_t w4a8_prepared_bytes(int64_t M, int64_t K) {
  if (check_w4a8_shape(M, K, 16) != QG_OK) return (size_t)-1;
  return M == 0 ? 0 : w4a8_layout(M, K).total;
}

int w4a8_prepare(const void* x_f16, int64_t M, int64_t K, int64_t ldx, void* prepared, size_t prepared_bytes,
                 void* stream) {
  int st = check_w4a8_shape(M, K, 16);
  if (st != QG_OK) return st;
  if (ldx < K || ldx % 8 != 0) return QG_ERR_INVALID_ARG;
  if (M == 0) return QG_OK;
  if (!x_f16 || !prepared || !aligned16(x_f16) || !aligned16(prepared)) return QG_ERR_INVALID_ARG;
  if (prepared_bytes < w4a8_layout(M, K).total) return QG_ERR_WORKSPACE;
  clear_stale_error();
  return prepare_impl(x_f16, M, K, ldx, prepared, nullptr, as_stream(stream));
}

int rmsnorm_w4a8_prepare(const void* x_f16, const void* w_f16, int64_t M, int64_t H, int64_t ldx, float eps,
                         void* y_f16, void* prepared, size_t prepared_bytes, void* stream) {
  int st = check_w4a8_shape(M, H, 16);
  if (st != QG_OK) return st;
  if (H > kMaxK16) return QG_ERR_UNSUPPORTED_SHAPE;
  if (ldx < H || ldx % 8 != 0 || !(eps >= 0.0f) || !std::isfinite(eps)) return QG_ERR_INVALID_ARG;
  if (M == 0) return QG_OK;
  if (!x_f16 || !w_f16 || !prepared || !aligned16(x_f16) || !aligned16(w_f16) || !aligned16(prepared) ||
      (y_f16 && !aligned16(y_f16)))
    return QG_ERR_INVALID_ARG;
  if (prepared_bytes < w4a8_layout(M, H).total) return QG_ERR_WORKSPACE;
  const W4A8Layout L = w4a8_layout(M, H);
  char* base = reinterpret_cast<char*>(prepared);
  int8_t* q = reinterpret_cast<int8_t*>(base + L.q_off);
  float* ts = reinterpret_cast<float*>(base + L.s_off);
  const bool skinny = M <= kSkinnyMaxM;
  clear_stale_error();
  return launch_status(qg::launch_rmsnorm_quant(reinterpret_cast<const uint16_t*>(x_f16),
                                                reinterpret_cast<const uint16_t*>(w_f16), M, H, ldx, eps,
                                                reinterpret_cast<uint16_t*>(y_f16), skinny ? nullptr : q, H,
                                                skinny ? q : nullptr, ts, as_stream(stream)));
}

namespace {
// Shape rules of verify_attention_f16 (QG_OK or the status to return).
int check_attention(int64_t T, int64_t Hq, int64_t Hkv, int64_t L) {
  if (T < 1 || Hq < 1 || Hkv < 1 || L < 1) return QG_ERR_INVALID_ARG;
  if (Hq % Hkv != 0 || T > 16 || Hq / Hkv * T > 128 || L < T) return QG_ERR_UNSUPPORTED_SHAPE;
  if (Hq > 4096 || L > (int64_t)1 << 24) return QG_ERR_UNSUPPORTED_SHAPE;
  return QG_OK;
}
}  // namespace

size_t verify_attention_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t L) {
  if (check_attention(T, Hq, Hkv, L) != QG_OK) return (size_t)-1;
  return qg::attn_plan(T, Hq, Hkv, L).ws_bytes;
}

int verify_attention_f16(const void* q, const void* k_cache, const void* v_cache, int64_t T, int64_t Hq, int64_t Hkv,
                         int64_t L, void* o, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_attention(T, Hq, Hkv, L);
  if (st != QG_OK) return st;
  if (!q || !k_cache || !v_cache || !o || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(o))
    return QG_ERR_INVALID_ARG;
  const qg::AttnPlan pl = qg::attn_plan(T, Hq, Hkv, L);
  if (!workspace || ws_bytes < pl.ws_bytes) return QG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_verify_attention(
      reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k_cache),
      reinterpret_cast<const uint16_t*>(v_cache), reinterpret_cast<uint16_t*>(o), T, Hq, Hkv, L, workspace,
      as_stream(stream)));
}

namespace {
// Shape and parameter rules of sample_topk_topp (QG_OK or the status to return).
int check_sampler(int64_t R, int64_t V, int64_t k) {
  if (R < 0 || V < 1 || k < 1) return QG_ERR_INVALID_ARG;
  if (k > 64 || k > V || R > 65536 || V >= (int64_t)1 << 24) return QG_ERR_UNSUPPORTED_SHAPE;
  if (qg::sampler_plan(R > 0 ? R : 1, V, k).E == 0) return QG_ERR_UNSUPPORTED_SHAPE;
  return QG_OK;
}
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
}  // namespace

size_t sampler_workspace_bytes(int64_t R, int64_t V, int64_t k) {
  if (check_sampler(R, V, k) != QG_OK) return (size_t)-1;
  return qg::sampler_plan(R, V, k).ws_bytes;
}

int sample_topk_topp(const void* logits_f16, int64_t R, int64_t V, int64_t ld, int64_t k, float top_p,
                     float temperature, const float* u, int32_t* ids, float* probs, int32_t* kept, int32_t* sampled,
                     float* lse, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_sampler(R, V, k);
  if (st != QG_OK) return st;
  if (ld < V || ld % 8 != 0) return QG_ERR_INVALID_ARG;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return QG_ERR_INVALID_ARG;
  if (!(temperature >= 1e-6f && temperature <= 1e6f)) return QG_ERR_INVALID_ARG;
  if (R == 0) return QG_OK;
  if (!logits_f16 || !u || !ids || !probs || !kept || !sampled || !lse || !aligned16(logits_f16) || !aligned4(u) ||
      !aligned4(ids) || !aligned4(probs) || !aligned4(kept) || !aligned4(sampled) || !aligned4(lse))
    return QG_ERR_INVALID_ARG;
  const qg::SamplerPlan pl = qg::sampler_plan(R, V, k);
  if (!workspace || ws_bytes < pl.ws_bytes) return QG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_sampler(reinterpret_cast<const uint16_t*>(logits_f16), R, V, ld, k, top_p,
                                          temperature, u, ids, probs, kept, sampled, lse, workspace,
                                          as_stream(stream)));
}

int w4a8_gemm_prepared(const void* prepared, int64_t M, int64_t K, int64_t N, const void* w_packed,
                       const void* s_packed, void* y_f16, void* stream) {
  int st = check_w4a8_shape(M, K, N);
  if (st != QG_OK) return st;
  if ((st = check_ptrs(M, prepared, w_packed, s_packed, y_f16)) != QG_OK) return st;
  if (M == 0) return QG_OK;
  clear_stale_error();
  return gemm_prepared_impl(prepared, M, K, N, w_packed, s_packed, y_f16, as_stream(stream), nullptr, 0, 0, 0, 0);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// w4a8_gemm without a caller workspace (w4a8_gemm_noalloc).  The int8 codes
// and token scales that w4a8_gemm keeps in its workspace live here in a
// file-scope device array, `scratch`; each GPU holds its own copy, at its
// own address, for the life of the process.  Host code never passes the
// array's name to a kernel (in host code it names a host-side stand-in, not
// device memory): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[QG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // device address of scratch per device, null until looked up
std::mutex g_scratch_mutex;

// Device address of `scratch` on the device that runs `stream` (looked up
// on the first call for that device), or null with *err set.
void* scratch_for_stream(hipStream_t stream, hipError_t* err) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* addr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (addr) return addr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (addr) return addr;
  int cur = -1;
  if ((e = hipGetDevice(&cur)) != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
    *err = e;
    return nullptr;
  }
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t back = hipSetDevice(cur);
    if (e == hipSuccess) e = back;
  }
  if (e != hipSuccess || addr == nullptr) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  g_scratch_addr[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

size_t w4a8_noalloc_scratch_bytes(void) { return QG_NOALLOC_SCRATCH_BYTES; }

int w4a8_gemm_noalloc(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx, const void* w_packed,
                      const void* s_packed, void* y_f16, void* stream) {
  int st = check_gemm_shape(M, K, N, ldx);
  if (st != QG_OK) return st;
  if ((st = check_ptrs(M, x_f16, w_packed, s_packed, y_f16)) != QG_OK) return st;
  if (M == 0) return QG_OK;
  const size_t need = w4a8_layout(M, K).total;
  if (need > QG_NOALLOC_SCRATCH_BYTES) return QG_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_for_stream(as_stream(stream), &e);
  if (ws == nullptr) return launch_status(e);
  return w4a8_impl(x_f16, M, K, N, ldx, w_packed, s_packed, y_f16, ws, need, stream, nullptr, nullptr, nullptr, 0, 0,
                   0, 0);
}

int w8a16_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx, const int8_t* w,
               const void* s_f16, void* y_f16, void* workspace, size_t ws_bytes, void* stream) {
  return gemm_streaming(qg::kW8A16, x_f16, M, K, N, ldx, w, s_f16, y_f16, workspace, ws_bytes, stream);
}

int embed_gather_dequant_int8(const int32_t* ids, int64_t T, const int8_t* table, const void* scales_f16,
                              int64_t V, int64_t H, void* out_f16, void* stream) {
  if (T < 0 || V <= 0 || H <= 0) return QG_ERR_INVALID_ARG;
  if (H % kGroup || V > kMaxDim || H > kMaxDim || T > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return QG_OK;
  if (!ids || !table || !scales_f16 || !out_f16) return QG_ERR_INVALID_ARG;
  if (!aligned16(ids) || !aligned16(table) || !aligned16(scales_f16) || !aligned16(out_f16))
    return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_gather(ids, T, table, reinterpret_cast<const uint16_t*>(scales_f16), V, H,
                                         reinterpret_cast<uint16_t*>(out_f16), as_stream(stream)));
}

int qg_selftest_quant_division(unsigned long long* counts, void* stream) {
  if (!counts || (reinterpret_cast<uintptr_t>(counts) & 7u)) return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_quant_division_check(counts, as_stream(stream)));
}

int qg_probe_read(const void* a, int64_t a_bytes, const void* c, int64_t c_bytes, int share, int wgs, int threads,
                  int nontemporal, uint32_t* sink, void* stream) {
  if (a_bytes < 0 || c_bytes < 0 || (a_bytes > 0 && !a) || (c_bytes > 0 && !c) || !sink) return QG_ERR_INVALID_ARG;
  if (share < 1 || wgs < share || wgs % share || wgs > 65536 || threads < 64 || threads > 1024 || threads % 64)
    return QG_ERR_INVALID_ARG;
  // every slice must fit one buffer resource (byte offsets below 2^31)
  if (a_bytes / (wgs / share) >= ((int64_t)1 << 31) - 16 || c_bytes / share >= ((int64_t)1 << 31) - 16)
    return QG_ERR_UNSUPPORTED_SHAPE;
  clear_stale_error();
  return launch_status(qg::launch_probe_read(a, a_bytes, c, c_bytes, share, wgs, threads, nontemporal != 0, sink,
                                             as_stream(stream)));
}

int quant_table_int8(const uint16_t* src_bf16, int64_t V, int64_t H, int8_t* Q, void* S_f16, void* stream) {
  if (V <= 0 || H <= 0) return QG_ERR_INVALID_ARG;
  if (H % kGroup || V > kMaxDim || H > kMaxDim) return QG_ERR_UNSUPPORTED_SHAPE;
  if (!src_bf16 || !Q || !S_f16) return QG_ERR_INVALID_ARG;
  if (!aligned16(src_bf16) || !aligned16(Q) || !aligned16(S_f16)) return QG_ERR_INVALID_ARG;
  clear_stale_error();
  return launch_status(qg::launch_quant_table(src_bf16, V, H, Q, reinterpret_cast<uint16_t*>(S_f16),
                                              as_stream(stream)));
}

}  // extern "C"
