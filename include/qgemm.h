/*
 * qgemm: weight-only-int4 GEMMs and the int8 vocabulary-table kernels for
 * MI355X (gfx950), as a plain C ABI.
 *
 * Sources (pages cited by title and section):
 *   [OPT]  "What this repo does that stock vLLM doesn't" (the project's
 *          optimisations page), "In full" items 1, 2, 4, 5, 6 and the
 *          section "int8 prefill for single-user mode".
 *   [README] the project README, section "What each step buys".
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Device pointers must be 16-byte aligned; leading dimensions are in
 *     elements and must keep every row 16-byte aligned (ldx % 8 == 0 for
 *     fp16 rows).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it asynchronously; no call synchronises the
 *     host.  Outputs are valid once that stream reaches the enqueued work.
 *   - Arguments are validated on the host before anything is launched.  On
 *     an error nothing is launched, nothing is written and the status code
 *     says why.  No entry point aborts or throws.
 *   - Row-major layouts.  fp16 is IEEE binary16, stored as uint16.
 *   - Calls that share a workspace buffer must be ordered on one stream.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics; every reduction runs in a fixed order).
 *
 * Weight format (int4 body, [OPT] "In full" item 4)
 *   Canonical weights are codes[N][K] (int8 storage, values in [-8, 7], the
 *   two's complement int4 range) and signed fp16 group scales
 *   scales[N][K/128]: w[n][k] = codes[n][k] * scales[n][k/128].  Negative
 *   scales are honoured as they are (no sign is folded into the codes).
 *   w4_repack turns them into the opaque pre-shuffled layout the GEMMs read.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
#define QG_OK 0
#define QG_ERR_INVALID_ARG 1       /* null/misaligned pointer, negative size, ldx < K, bad op */
#define QG_ERR_UNSUPPORTED_SHAPE 2 /* K % 128 != 0, N % 16 != 0, H % 128 != 0, K too long, size too large */
#define QG_ERR_WORKSPACE 3         /* ws_bytes smaller than qg_workspace_bytes() */
#define QG_ERR_LAUNCH 4            /* the HIP runtime reported an error at launch */

/* Operation ids for qg_workspace_bytes. */
#define QG_OP_W4A16 1
#define QG_OP_W4A8 2
#define QG_OP_W8A16 3

/* Static, NUL-terminated description of a status code (never NULL). */
const char* qg_status_string(int status);

/* The HIP runtime's description of the error behind the calling thread's
 * most recent QG_ERR_LAUNCH ("none" if there was none).  Thread-local; the
 * pointer stays valid for the life of the process. */
const char* qg_last_hip_error(void);

/* Bytes of the packed weight / packed scale buffers w4_repack writes for an
 * [N, K] weight.  0 if the shape is unsupported. */
size_t w4_packed_bytes(int64_t N, int64_t K);
size_t w4_scales_bytes(int64_t N, int64_t K);

/* Bytes of device workspace the GEMM `op` needs for this shape (0 is a valid
 * answer: no workspace needed, as for w4a16_gemm and w8a16_gemm).  Returns
 * (size_t)-1 for an invalid op or shape.  The W4A8 workspace holds the int8
 * activation codes and the token scales; it needs no initialisation and its
 * contents after a call are unspecified. */
size_t qg_workspace_bytes(int op, int64_t M, int64_t K, int64_t N);

/*
 * act_quant_int8 -- per-token int8 activation quantisation ([OPT] "In full"
 * item 4: activations are quantised to int8 per token).
 *   x      fp16 [M][ldx] (first K columns used), ldx >= K, ldx % 8 == 0
 *   q      int8 [M][K] out:  q[m][k] = clamp(rne(fp32(x[m][k]) / scale[m]), -127, 127)
 *   scale  fp32 [M]    out:  scale[m] = fp32(max_k |x[m][k]|) / 127 (IEEE division);
 *                            a row of zeros gets scale 0 and codes 0.
 *   M >= 0, K > 0, K % 128 == 0 and K < 2^31.  Codes and scales are
 *   bit-exact against that definition.  NaN/Inf inputs give unspecified
 *   codes.
 */
int act_quant_int8(const void* x_f16, int64_t M, int64_t K, int64_t ldx,
                   int8_t* q, float* scale, void* stream);

/*
 * w4_repack -- load-time reshuffle of canonical int4 weights into the layout
 * the GEMMs stream with 128-bit loads ([OPT] "In full" item 4).
 *   codes     int8 [N][K], values in [-8, 7] (only the low 4 bits are used)
 *   scales    fp16 [N][K/128], signed
 *   w_packed  out, w4_packed_bytes(N, K) bytes (K*N/2)
 *   s_packed  out, w4_scales_bytes(N, K) bytes (same size as scales)
 *   N % 16 == 0, K % 128 == 0.  Not a sign fold: codes and scales keep
 *   their signs.  One packed buffer serves both w4a16_gemm and w4a8_gemm.
 */
int w4_repack(const int8_t* codes, const void* scales_f16, int64_t N, int64_t K,
              void* w_packed, void* s_packed, void* stream);

/*
 * w4a16_gemm -- y = x * W^T with int4 weights and fp16 activations ([README]
 * "What each step buys": the W4A16 body; used for decode and speculative
 * verify, M = 1 + draft tokens).
 *   x         fp16 [M][ldx]
 *   w_packed, s_packed  from w4_repack for [N, K]
 *   y         fp16 [M][N] out: y[m][n] = fp16(sum_k x[m][k] * codes[n][k] * scales[n][k/128]),
 *             products of fp16 x and exact int4 codes accumulated in fp32,
 *             each 128-wide group rescaled by its fp32 scale.
 *   workspace, ws_bytes  unused (qg_workspace_bytes gives 0); may be NULL, 0
 *   K <= 65536 (for w8a16_gemm too): the kernel holds a workgroup's group
 *   scales in LDS; a longer K returns QG_ERR_UNSUPPORTED_SHAPE.
 */
int w4a16_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx,
               const void* w_packed, const void* s_packed, void* y_f16,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * w4a8_gemm -- W4A8: per-token int8 activations times int4 weights on the
 * int8 matrix cores ([OPT] "In full" item 4 and "int8 prefill for
 * single-user mode").  Quantises x inside the call (as act_quant_int8, into
 * the workspace), then
 *   P[m][n][g] = sum_{j<128} q[m][128g+j] * codes[n][128g+j]   (exact int32)
 *   y[m][n]    = fp16(scale[m] * sum_g fp32(P[m][n][g]) * scales[n][g])   (fp32)
 * Same arguments as w4a16_gemm; the workspace must hold
 * qg_workspace_bytes(QG_OP_W4A8, M, K, N) bytes.  K <= 2^22 (4,194,304):
 * the kernels address a workgroup's operand block (up to 128 rows of K
 * codes) with 32-bit buffer offsets; a longer K returns
 * QG_ERR_UNSUPPORTED_SHAPE.
 */
int w4a8_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx,
              const void* w_packed, const void* s_packed, void* y_f16,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * w4a8_prepare / w4a8_gemm_prepared -- w4a8_gemm in two steps, so one
 * quantised activation can feed several GEMMs (for example the fused
 * gate/up projection and the q/k/v projections of the same hidden state).
 *   w4a8_prepared_bytes(M, K)  size of the opaque prepared buffer ((size_t)-1
 *                              for an unsupported shape, 0 for M == 0)
 *   w4a8_prepare   quantises x per token (exactly as act_quant_int8) into
 *                  `prepared` (prepared_bytes >= w4a8_prepared_bytes(M, K)),
 *                  codes in the order the GEMM for this M reads, plus the
 *                  fp32 token scales.  The buffer is only meaningful to
 *                  w4a8_gemm_prepared with the same M and K.
 *   w4a8_gemm_prepared  y = the W4A8 product of that quantised x with the
 *                  packed weights; bit-identical to w4a8_gemm on the same x.
 *                  Launches exactly one kernel.
 */
size_t w4a8_prepared_bytes(int64_t M, int64_t K);
int w4a8_prepare(const void* x_f16, int64_t M, int64_t K, int64_t ldx, void* prepared, size_t prepared_bytes,
                 void* stream);
int w4a8_gemm_prepared(const void* prepared, int64_t M, int64_t K, int64_t N, const void* w_packed,
                       const void* s_packed, void* y_f16, void* stream);

/*
 * rmsnorm_w4a8_prepare -- the quantiser fused into the norm that produces
 * the GEMM's input, so the activations are quantised once, where they are
 * made, and the prepared buffer feeds every W4A8 GEMM of that hidden state
 * ([OPT] "In full" item 4: activations are quantised to int8 per token; the
 * pages name no norm, so the norm below is a plain reading).
 *   x         fp16 [M][ldx] (first H columns used), ldx >= H, ldx % 8 == 0
 *   w         fp16 [H], the norm's weight
 *   eps       >= 0, finite
 *   y         fp16 [M][H] out, contiguous, or NULL to skip it:
 *             y[m][h] = x[m][h] * w[h] / sqrt(sum_h' x[m][h']^2 / H + eps)
 *             rounded to fp16, evaluated in fp32 (a tree-ordered sum of
 *             squares, IEEE division and square root, (x * r) * w; y = 0
 *             where sum / H + eps == 0).  Within one fp16 unit in the last
 *             place of the correctly rounded value, and equal to it except
 *             where the exact value lies within a few fp32 ulps of a point
 *             halfway between two fp16 numbers.
 *   prepared  out, prepared_bytes >= w4a8_prepared_bytes(M, H): exactly what
 *             w4a8_prepare writes for that y (codes and token scales of
 *             act_quant_int8 on the y this call computes, bit-exact), for
 *             w4a8_gemm_prepared with K = H
 *   H % 128 == 0, H <= 65536.  One kernel launch.
 */
int rmsnorm_w4a8_prepare(const void* x_f16, const void* w_f16, int64_t M, int64_t H, int64_t ldx, float eps,
                         void* y_f16, void* prepared, size_t prepared_bytes, void* stream);

/*
 * verify_attention_f16 -- split-KV attention for the speculative-verify step
 * ([OPT] "In full" item 6: on a multi-query verify step the KV sequence must
 * be split across workgroups too, or most of the GPU idles; 24 query heads,
 * head_dim 256 on the pages).  One sequence, T query tokens whose keys and
 * values are the last T entries of the cache.
 *   q        fp16 [T][Hq][256], contiguous
 *   k, v     fp16 [L][Hkv][256], contiguous (the cache, positions 0 .. L-1)
 *   o        fp16 [T][Hq][256] out:
 *            o[t][h] = sum_p softmax_p(s) v[p][h/G] over p <= L - T + t, with
 *            s = (q[t][h] . k[p][h/G]) / 16 and G = Hq / Hkv (grouped-query
 *            heads); scores, softmax and sums in fp32
 *   workspace, ws_bytes  >= verify_attention_workspace_bytes(T, Hq, Hkv, L)
 *            (fp32 per-split partials; no initialisation needed)
 *   1 <= T <= 16, Hq % Hkv == 0, (Hq / Hkv) * T <= 128, T <= L <= 2^24,
 *   Hq <= 4096.  Two kernel launches (the splits, then their combination).
 *   verify_attention_workspace_bytes returns (size_t)-1 for a rejected shape.
 */
size_t verify_attention_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t L);
int verify_attention_f16(const void* q, const void* k_cache, const void* v_cache, int64_t T, int64_t Hq, int64_t Hkv,
                         int64_t L, void* o, void* workspace, size_t ws_bytes, void* stream);

/*
 * sample_topk_topp -- small-k top-k / top-p sampling of a step's logits
 * ([OPT] "In full" item 6: with k <= 64 known up front the mask is a top-k
 * selection, not a sort of the 248k-wide row; the softmax over the row runs
 * on many workgroups; target and drafts sample from the same truncated
 * support).  Per row r of R:
 *   logits   fp16 [R][ld], the first V values of each row are used
 *            (ld >= V, ld % 8 == 0, 16-byte aligned); finite or -inf (a
 *            NaN, or a row that is all -inf, gives undefined results)
 *   ids      int32 [R][k] out: the k largest logits' ids, larger logit
 *            first, equal logits by lower id
 *   probs    fp32 [R][k] out: softmax of logits / T over those k,
 *            renormalised over the kept ranks, 0 after them
 *   kept     int32 [R] out: ranks j with sum_{i<j} mass_i < top_p, where
 *            mass is the softmax over the k (at least 1)
 *   sampled  int32 [R] out: the id at the smallest kept rank whose
 *            cumulative probability exceeds u[r] (the last kept rank if
 *            none); u fp32 [R], the caller's uniforms in [0, 1)
 *   lse      fp32 [R] out: log sum_v exp(logits[r][v] / T) over all V
 *   workspace, ws_bytes >= sampler_workspace_bytes(R, V, k) (candidates and
 *            partial sums; no initialisation needed)
 *   1 <= k <= 64, k <= V < 2^24, ceil(V / 8192) * k <= 16384, R <= 65536,
 *   0 < top_p <= 1, 1e-6 <= temperature <= 1e6.  fp32 arithmetic.  Two
 *   kernel launches (chunks, then rows).  sampler_workspace_bytes returns
 *   (size_t)-1 for a rejected shape.
 */
size_t sampler_workspace_bytes(int64_t R, int64_t V, int64_t k);
int sample_topk_topp(const void* logits_f16, int64_t R, int64_t V, int64_t ld, int64_t k, float top_p,
                     float temperature, const float* u, int32_t* ids, float* probs, int32_t* kept, int32_t* sampled,
                     float* lse, void* workspace, size_t ws_bytes, void* stream);

/*
 * w4a8_gemm_debug -- w4a8_gemm that also exposes its integer stages, for
 * bit-exact checks.  For every M it runs the kernels w4a8_gemm runs (the
 * quantiser, then the same GEMM kernel with the same work split, compiled
 * with stores of the group partials), so y is bit-identical to w4a8_gemm's,
 * and in addition writes
 *   q_out     int8 [M][K]   the activation codes   (may be NULL)
 *   scale_out fp32 [M]      the token scales       (may be NULL)
 *   partials  int32 [m1-m0][n1-n0][K/128]  P[m][n][g] for m0 <= m < m1,
 *             n0 <= n < n1, at index ((m-m0)*(n1-n0) + (n-n0))*(K/128) + g
 *             (may be NULL; then the window is ignored)
 *   0 <= m0 <= m1 <= M, 0 <= n0 <= n1 <= N.
 */
int w4a8_gemm_debug(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx,
                    const void* w_packed, const void* s_packed, void* y_f16,
                    void* workspace, size_t ws_bytes, void* stream,
                    int8_t* q_out, float* scale_out, int32_t* partials,
                    int64_t m0, int64_t m1, int64_t n0, int64_t n1);

/*
 * w8a16_gemm -- the int8-weight lm_head product over the same row-major
 * table the embedding gather reads ([OPT] "In full" items 1 and 5).
 *   w   int8 [N][K] row-major (the vocabulary table, N = V rows, K = H)
 *   s   fp16 [N][K/128] (its group scales)
 *   y   fp16 [M][N] out: y[m][n] = fp16(sum_k x[m][k] * w[n][k] * s[n][k/128])
 *       (fp32 accumulation, per-group fp32 rescale)
 *   Other arguments as w4a16_gemm; op id QG_OP_W8A16 for the workspace.
 */
int w8a16_gemm(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx,
               const int8_t* w, const void* s_f16, void* y_f16,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * embed_gather_dequant_int8 -- dequant-on-gather embedding lookup ([OPT]
 * "In full" item 2).
 *   ids     int32 [T]
 *   table   int8 [V][H], scales fp16 [V][H/128]
 *   out     fp16 [T][H]: out[t][h] = fp16(fp32(table[id][h]) * fp32(scales[id][h/128]))
 *           (one rounding: the fp32 product is exact).  An id outside
 *           [0, V) gives a row of zeros.
 *   T >= 0, V > 0, H % 128 == 0; T, V and H below 2^31.
 */
int embed_gather_dequant_int8(const int32_t* ids, int64_t T, const int8_t* table,
                              const void* scales_f16, int64_t V, int64_t H,
                              void* out_f16, void* stream);

/*
 * quant_table_int8 -- the offline requantisation of a bf16 vocabulary table
 * to int8 group-128 ([OPT] "In full" item 1), on the device.
 *   src   bf16 [V][H] (uint16 bit patterns)
 *   Q     int8 [V][H] out, S fp16 [V][H/128] out:
 *         S = fp16(fp32(absmax of the group) / 127),
 *         Q = clamp(rne(fp32(src) / fp32(S)), -127, 127), and Q = 0 where S == 0.
 *   H % 128 == 0; V and H below 2^31.  Bit-exact against that definition.
 */
int quant_table_int8(const uint16_t* src_bf16, int64_t V, int64_t H,
                     int8_t* Q, void* S_f16, void* stream);

/*
 * w4a8_gemm_noalloc -- w4a8_gemm for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as w4a8_gemm (bit-identical y), minus the workspace: the int8
 * activation codes and token scales go to a device array inside the
 * library, QG_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held from the first
 * call on that GPU until the process ends.  Nothing is allocated and the
 * host is not synchronised (the first call on a GPU looks up the array's
 * device address once).
 *   Requires w4a8_prepared_bytes(M, K) <= QG_NOALLOC_SCRATCH_BYTES (any
 *   M <= 64 with K <= 130,944; M = 4096 with K <= 1,920); a larger shape
 *   returns QG_ERR_WORKSPACE before anything runs.
 *   The array needs no initialisation and keeps the last call's codes.
 *   Every call on one GPU shares that GPU's array: calls that overlap on
 *   one GPU (on different streams, or from several threads without an
 *   ordering between their streams) race and give undefined results.
 * w4a8_noalloc_scratch_bytes() returns QG_NOALLOC_SCRATCH_BYTES.
 */
#define QG_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
size_t w4a8_noalloc_scratch_bytes(void);
int w4a8_gemm_noalloc(const void* x_f16, int64_t M, int64_t K, int64_t N, int64_t ldx,
                      const void* w_packed, const void* s_packed, void* y_f16, void* stream);

/*
 * qg_selftest_quant_division -- exhaustive device check of the quantiser's
 * division ([OPT] "In full" item 4: per-token int8 activations; codes are
 * rint(x / scale) with scale = absmax / 127).  The kernels form x / scale as
 * a reciprocal product with one correction step instead of a division per
 * element; this runs that step beside the IEEE division for every finite
 * positive fp16 absmax and every fp16 x with |x| <= absmax (1,007,713,278
 * pairs) and adds, to the caller's zero-initialised device counters,
 *   counts[0]  the pairs checked
 *   counts[1]  the pairs where the two rounded quotients differ
 * counts: 2 x uint64, 8-byte aligned device memory.  One kernel launch.
 */
int qg_selftest_quant_division(unsigned long long* counts, void* stream);

/*
 * qg_probe_read -- diagnostic read with the access pattern of a weight-
 * streaming GEMM and none of its arithmetic: the load floor its kernels are
 * measured against (bench.py --floor times it).  Workgroup b of `wgs`
 * (with `threads` threads, a multiple of 64 up to 1024) reads:
 *   slice lin / share of a, where a's a_bytes are dealt into wgs / share
 *     equal slices, with the non-temporal hint when `nontemporal` != 0;
 *   slice lin % share of c, c's c_bytes dealt into share slices;
 * lin being b walked as the row-split W4A8 decode kernel walks its grid
 * (when wgs is a multiple of 8 and wgs / 8 of share, the `share`
 * workgroups reading one slice of a are consecutive on one XCD).  Each
 * thread issues its 16-byte loads 16 at a time, its slice of a first; the
 * only store is one checksum word per wave into sink (device memory,
 * wgs * threads / 64 uint32).  a and c are read-only and may alias.  share >= 1, wgs a
 * multiple of share, wgs <= 65536; each slice under 2 GiB.  One launch.
 */
int qg_probe_read(const void* a, int64_t a_bytes, const void* c, int64_t c_bytes, int share, int wgs, int threads,
                  int nontemporal, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
