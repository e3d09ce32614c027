/*
 * pqg.h -- C ABI of the MI355X (gfx950) quantized linear layer.
 *
 * Operations, by the passage that defines them:
 *   [P1] "量化、蒸馏与模型压缩" (LLM knowledge atlas, notes 03-05): core formula; §1.1 group quantization and
 *        its metadata; §2.3 SmoothQuant, eq. (1)-(2).
 *   [P2] "模型压缩：量化、ZeroQuant、LLM.int8() 与 SmoothQuant" (LLM tutorial, lesson 19): §3 basic formula,
 *        §4 granularity, §11 vector-wise scaling, §13 alpha.
 *   [P3] "第11章 模型量化与压缩" (AI infra guide, chapter 11): §11.1.1 affine quantization; §11.1.2
 *        symmetric / asymmetric; §11.1.3 Table 11-1 granularity; §11.1.4 dynamic quantization; §11.1.6
 *        INT4 group example; §11.4.3 smoothing factor; §11.4.5 W8A8 pipeline; §11.10.1 bandwidth model.
 *   [P5] "大模型压缩：从研究到生产的完整攻略（1）" (CSDN blog): symmetric / asymmetric worked examples.
 *
 * Conventions shared by every entry point:
 *   - All pointers except `stream` are DEVICE pointers into memory the caller allocated and owns; the
 *     library allocates nothing and keeps no state besides a thread-local error string (the one exception,
 *     pqg_qlinear_w8a8_noalloc, uses a fixed device array of the library's own, described there).
 *   - Tensors are row-major and contiguous. bf16 is the 16-bit brain float (upper half of a binary32).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is enqueued on it and never
 *     synchronised: execution errors surface at the caller's next synchronisation.
 *   - Every argument is checked on the host BEFORE anything is enqueued. On error nothing is launched and
 *     the call returns PQG_EINVAL (bad argument) or PQG_EUNSUPPORTED (valid but not implemented); a failed
 *     launch returns PQG_EHIP. pqg_last_error() then describes the problem.
 *   - Device pointers must be 16-byte aligned (scale / zero / smoothing vectors: 4-byte aligned).
 *   - A tensor with zero rows is accepted and nothing is launched.
 *   - Inputs must be finite; NaN / Inf inputs give unspecified codes.
 *   - Calls on one stream are ordered; calls that share output buffers on different streams race.
 */
#ifndef PQG_H
#define PQG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQG_ABI_VERSION 1

/* status codes */
#define PQG_OK 0
#define PQG_EINVAL 1
#define PQG_EUNSUPPORTED 2
#define PQG_EHIP 3

/* float element types */
#define PQG_F32 0
#define PQG_BF16 1

/* granularity of the (scale, zero) parameters [P2 §4; P3 §11.1.3 Table 11-1]:
 *   PQG_TENSOR : one pair for the whole tensor;
 *   PQG_ROW    : one pair per row -- per output channel for a weight [N, K], per token for activations [M, K];
 *   PQG_GROUP  : one pair per `group_size` consecutive elements of a row (along the input dimension),
 *                rows*cols/group_size pairs [P1 §1.1; P3 §11.1.6]. */
#define PQG_TENSOR 0
#define PQG_ROW 1
#define PQG_GROUP 2

/* smoothing applied before quantization, per input channel j (column) [P3 §11.4.2, §11.4.5]:
 *   PQG_SMOOTH_DIV : x'[.., j] = x[.., j] / s[j]  (activations, X diag(s)^-1)
 *   PQG_SMOOTH_MUL : x'[.., j] = x[.., j] * s[j]  (weights, diag(s) W with W stored [N, K]) */
#define PQG_SMOOTH_NONE 0
#define PQG_SMOOTH_DIV 1
#define PQG_SMOOTH_MUL 2

/* Version of this ABI (PQG_ABI_VERSION). */
int32_t pqg_abi_version(void);

/* Text of the last error on the calling thread ("" if none). Valid until the thread's next pqg_* call. */
const char *pqg_last_error(void);

/*
 * Workspace needed by pqg_quantize for this shape and granularity (bytes; 0 if none).
 * Only PQG_TENSOR needs one (per-block partial ranges).
 */
size_t pqg_quantize_workspace_bytes(int64_t rows, int64_t cols, int32_t granularity);

/*
 * Affine quantization  q = clamp(round(x / s) + z, qmin, qmax)  [P1 core formula; P2 §3; P3 §11.1.1].
 *   x            : [rows, cols] of x_dtype (PQG_F32 or PQG_BF16).
 *   smooth       : [cols] fp32 smoothing vector, required iff smooth_mode != PQG_SMOOTH_NONE.
 *   bits         : 4 or 8.
 *   symmetric    : 1 -> z = 0, s = max|x| / qmax, codes in [-qmax, qmax], qmax = 2^(bits-1) - 1
 *                  (INT4 [-7, 7], INT8 [-127, 127]) [P3 §11.1.2, §11.1.6; P5 symmetric example];
 *                  0 -> unsigned codes [0, 2^bits - 1], s = (hi - lo) / (2^bits - 1), z = round(-lo / s),
 *                  with the range [lo, hi] widened to contain 0 so that 0 is coded exactly
 *                  [P3 §11.1.1; P5 asymmetric example].
 *   granularity  : PQG_TENSOR / PQG_ROW / PQG_GROUP; group_size in {32, 64, 128} for PQG_GROUP (else ignored).
 *   codes (out)  : bits == 8: int8 (symmetric) or uint8 (asymmetric) [rows, cols];
 *                  bits == 4: uint8 [rows, cols / 2], two codes per byte, element 2i of a row in the low
 *                  nibble of byte i, signed codes as two's-complement nibbles.
 *   scales (out) : fp32 [1], [rows] or [rows * cols / group_size].
 *   zeros (out)  : uint8, same count as scales; required iff symmetric == 0, must be NULL otherwise.
 *   workspace    : device scratch of at least pqg_quantize_workspace_bytes() bytes (may be NULL if 0).
 * Rounding is round-half-to-even of the correctly rounded fp32 quotient x / s; smoothing divides or
 * multiplies in fp32; a segment whose step would be 0 (an all-zero or underflowing range) codes every value
 * to 0 with z = 0 and stores the scale 0, so that it dequantizes to exactly 0. Results are bit-identical to a
 * strict-IEEE CPU evaluation of the same formulas.
 * Requires cols % 32 == 0 and, for PQG_ROW, cols <= 65536.
 */
int32_t pqg_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, const float *smooth,
                     int32_t smooth_mode, int32_t bits, int32_t symmetric, int32_t granularity,
                     int32_t group_size, void *codes, float *scales, uint8_t *zeros, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Static per-tensor quantization with calibrated parameters [P3 §11.4.5 step 5 (per-tensor INT8
 * activations); P3 §11.1.4 (static scales fixed offline from calibration data, against dynamic ones
 * computed at run time)]: q = clamp(round(x / scale) + zero, qmin, qmax) for every element, with (scale,
 * zero) given by the caller, e.g. from pqg_quantize with PQG_TENSOR over calibration activations. Values
 * beyond the calibrated range clip to qmin / qmax.
 *   x            : [rows, cols] of x_dtype (PQG_F32 or PQG_BF16), e.g. the smoothed activations X diag(s)^-1
 *                  as a LayerNorm with the factor folded into its gain produces them [P3 §11.4.4].
 *   bits         : 4 or 8; symmetric: 1 -> codes in [-qmax, qmax] and zero must be 0; 0 -> codes in
 *                  [0, 2^bits - 1] and zero in that range.
 *   scale        : finite and > 0.
 *   codes (out)  : as pqg_quantize (bits == 8: int8 / uint8 [rows, cols]; bits == 4: packed uint8
 *                  [rows, cols / 2]).
 *   row_scales (out, optional): fp32 [rows], every entry set to `scale`: the per-token scale vector that
 *                  pqg_qlinear_w8a8 takes with x == NULL, so that the static path reuses its GEMM and
 *                  epilogue; NULL to skip.
 * Rounding as in pqg_quantize (round-half-to-even of the correctly rounded fp32 quotient); bit-identical to a
 * strict-IEEE CPU evaluation. Requires cols % 32 == 0.
 */
int32_t pqg_quantize_static(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t bits,
                            int32_t symmetric, float scale, int32_t zero, void *codes, float *row_scales,
                            void *stream);

/*
 * Dequantization  x_hat = s * (q - z)  [P1 core formula; P2 §3; P3 §11.1.1]: one fp32 multiply per element,
 * rounded to nearest-even when out_dtype is PQG_BF16.
 *   codes / scales / zeros / bits / symmetric / granularity / group_size: as produced by pqg_quantize
 *   (zeros NULL iff symmetric). out: [rows, cols] of out_dtype.
 */
int32_t pqg_dequantize(const void *codes, const float *scales, const uint8_t *zeros, int64_t rows, int64_t cols,
                       int32_t bits, int32_t symmetric, int32_t granularity, int32_t group_size, void *out,
                       int32_t out_dtype, void *stream);

/* Workspace needed by pqg_smooth (bytes). */
size_t pqg_smooth_workspace_bytes(int64_t tokens, int64_t out_features, int64_t in_features);

/*
 * SmoothQuant factor  s_j = max_t |X[t, j]|^alpha / max_n |W[n, j]|^(1 - alpha)
 * [P1 §2.3 eq. (1); P2 §13; P3 §11.4.3].
 *   x : activations [tokens, in_features] (x_dtype); w : weights [out_features, in_features] (w_dtype);
 *   s (out) : fp32 [in_features]; alpha in [0, 1].
 * Evaluation in fp32: alpha = 0.5 -> sqrt(ax) / sqrt(aw) (correctly rounded); alpha = 1 -> ax;
 * alpha = 0 -> 1 / aw; other alpha -> binary64 pow quotient rounded to fp32 (may differ by 1 ulp from
 * another libm). A channel with ax = 0 or aw = 0 gets s_j = 1.
 * Requires in_features % 8 == 0 and tokens, out_features >= 1.
 */
int32_t pqg_smooth(const void *x, int32_t x_dtype, int64_t tokens, const void *w, int32_t w_dtype,
                   int64_t out_features, int64_t in_features, double alpha, float *s, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Weight-only W4A16 linear  y[m, n] = sum_k x[m, k] * s[n, g(k)] * (q[n, k] - z[n, g(k)])
 * [P3 §11.1.6 step 5 (dequantize and multiply with 16-bit activations); P3 §11.10.1 (decode streams every
 * weight once per step)]. The dequantization happens in registers; no dequantized weight is written.
 *   x        : bf16 [M, K].
 *   w_packed : uint8 [N, K / 2], INT4 codes as pqg_quantize writes them (symmetric: two's complement).
 *   scales   : fp32 [N, K / group_size]; zeros: uint8 [N, K / group_size], NULL iff symmetric.
 *   group_size in {32, 64, 128}; K % group_size == 0.
 *   y (out)  : [M, N] of y_dtype (PQG_F32 or PQG_BF16); fp32 accumulation.
 * The sum is evaluated in a different order than a sequential loop; results agree with an exact
 * evaluation to well within bf16 output rounding (and to ~1e-6 relative for fp32 output).
 */
int32_t pqg_qlinear_w4a16(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *w_packed,
                          const float *scales, const uint8_t *zeros, int32_t group_size, int32_t symmetric,
                          void *y, int32_t y_dtype, void *stream);

/*
 * Grouped product: several independent W4A16 products y_i = x_i W_i^T (as pqg_qlinear_w4a16), in ONE launch
 * up to 32 tokens [P3 §11.10.1: at decode every weight of the layer is read once per generated token, so the
 * time is the whole weight stream; P3 §11.1.6: INT4 groups; P3 §11.3.7: the same products batched]. Streaming
 * the row blocks of all the problems as one grid removes the launch gap and the partly idle tail of each small
 * product (the Llama-70B k and v projections, 1024 x 8192, do not fill the GPU on their own). Use it for
 * products whose inputs are ready together: the projections that read the same normalised hidden state, or
 * expert weights. Up to 4 tokens the decode kernel runs; 5 to 32 tokens the staged matrix-core kernel, in one
 * launch when every problem has K % 128 == 0 (else one launch per problem); above 32 tokens one launch per
 * problem, exactly as pqg_qlinear_w4a16 on each.
 *   problems : HOST array of `count` descriptors (1 <= count <= 8), read during the call only (they are
 *              copied into the launch), each with
 *                x        bf16 [M, K] activations (device),
 *                w_packed uint8 [N, K / 2] INT4 codes as pqg_quantize writes them (device),
 *                scales   fp32 [N, K / group_size]; zeros uint8 [N, K / group_size], NULL iff symmetric (device),
 *                y        [M, N] of y_dtype (device, out),
 *                N, K     the problem's shape (K % group_size == 0; a problem with N == 0 is skipped).
 *   M        : tokens, M >= 0, common to all.
 *   group_size, symmetric, y_dtype : common to all problems, as pqg_qlinear_w4a16.
 * Every problem is checked before anything is enqueued. Each result is that of pqg_qlinear_w4a16 on the
 * problem alone up to the order of the fp32 partial sums: both run the same per-row-block code, but a single
 * small product may split K over more waves than the grouped grid does (the grid size decides the split), so
 * partial sums are added in a different order. Both are within the tolerance of the exact product.
 * Alignment per problem as pqg_qlinear_w4a16.
 */
typedef struct {
    const void *x;
    const uint8_t *w_packed;
    const float *scales;
    const uint8_t *zeros;
    void *y;
    int64_t N, K;
} pqg_w4a16_problem;

int32_t pqg_qlinear_w4a16_grouped(const pqg_w4a16_problem *problems, int32_t count, int64_t M, int32_t group_size,
                                  int32_t symmetric, int32_t y_dtype, void *stream);

/*
 * W8A8 linear layer  y[m, n] = (sum_k q_x[m, k] q_w[n, k]) * s_x[m] * s_w[n]
 * [P3 §11.4.5 steps 5-6 (INT8 GEMM, INT32 accumulation, dequantized output); P3 §11.1.4 dynamic
 * activation statistics; P2 §11 vector-wise scales].
 * The activations are quantized on the fly: per token (row), symmetric INT8 [-127, 127], after the
 * smoothing division X diag(s)^-1 when `smooth` is non-NULL (exactly as pqg_quantize with PQG_ROW,
 * bits 8, symmetric, PQG_SMOOTH_DIV); then the INT8 GEMM with exact INT32 accumulation and the epilogue
 * y = bf16/fp32(float(acc) * (s_x[m] * s_w[n])).
 *   x        : bf16 [M, K] activations, or NULL: the activations are then already quantized and x_q /
 *              x_scales are INPUTS (e.g. codes from pqg_quantize with PQG_ROW, bits 8, symmetric), and only
 *              the GEMM + epilogue launch is enqueued.
 *   smooth   : fp32 [K] or NULL (must be NULL when x is NULL).
 *   w_q      : int8 [N, K] per-output-channel symmetric codes (pqg_quantize, PQG_ROW, bits 8; the
 *              smoothing multiply diag(s) W is applied there, offline); w_scales: fp32 [N].
 *   y (out)  : [M, N] of y_dtype (PQG_BF16 or PQG_F32).
 *   x_q, x_scales : int8 [M, K] and fp32 [M]. With x given they are caller scratch that the call fills
 *              with the activation codes and scales (and leaves readable); with x NULL they are inputs.
 * Requires K % 32 == 0 and K <= 65536.
 */
int32_t pqg_qlinear_w8a8(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales, int64_t M,
                         int64_t N, int64_t K, void *y, int32_t y_dtype, int8_t *x_q, float *x_scales,
                         void *stream);

/*
 * The INT8 x INT8 -> INT32 product of the W8A8 layer without the epilogue:
 *   c[m, n] = sum_k a[m, k] * b[n, k]   (exact: |c| <= K * 128^2 < 2^31 for every K the call accepts).
 *   a : int8 [M, K]; b : int8 [N, K]; c (out) : int32 [M, N].
 * Requires K % 16 == 0 and 0 < K <= 65536 (the bound of pqg_qlinear_w8a8; it keeps the int32 accumulators
 * exact and the kernels' 32-bit offsets inside a tile in range). K == 0 with M, N > 0 returns
 * PQG_EUNSUPPORTED, K above the bound PQG_EUNSUPPORTED; neither enqueues anything.
 * Same kernel and tiling as pqg_qlinear_w8a8; exposed so the accumulators can be checked bit-exactly.
 */
int32_t pqg_gemm_s8s8s32(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K, int32_t *c,
                         void *stream);

/*
 * W4A8 linear layer  y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] * (q_w[n, k] - z[n, g])
 * [P3 §11.4.5 (SmoothQuant combined with group-wise INT4 weights gives W4A8); P3 §11.10.2 (weight and
 * activation quantization are independent and stack: W4A8 is AWQ-style INT4 weights with SmoothQuant INT8
 * activations); P3 §11.1.6 (INT4 groups); P2 §11 (one scale per token)].
 * Each group's integer sum is exact (int32); the group scales weight them in fp32; the token scale is applied
 * last, and the result is rounded to y_dtype.
 *   x_q      : int8 [M, K] per-token symmetric activation codes and x_scales fp32 [M], e.g. pqg_quantize with
 *              PQG_ROW, bits 8, symmetric, PQG_SMOOTH_DIV.
 *   w_packed : uint8 [N, K / 2] INT4 codes as pqg_quantize writes them with PQG_GROUP, bits 4 (symmetric:
 *              two's complement; asymmetric: unsigned with zero points), e.g. on diag(s) W (PQG_SMOOTH_MUL);
 *              w_scales fp32 [N, K / group_size]; w_zeros uint8 [N, K / group_size], NULL iff symmetric.
 *   group_size in {32, 64, 128}. Requires K % 128 == 0 and 0 < K <= 2^24 (the kernel addresses a tile's rows
 *   with 32-bit offsets); K == 0 with M, N > 0 returns PQG_EUNSUPPORTED and enqueues nothing.
 *   y (out)  : [M, N] of y_dtype (PQG_F32 or PQG_BF16).
 */
int32_t pqg_qlinear_w4a8(const int8_t *x_q, const float *x_scales, int64_t M, int64_t N, int64_t K,
                         const uint8_t *w_packed, const float *w_scales, const uint8_t *w_zeros, int32_t group_size,
                         int32_t symmetric, void *y, int32_t y_dtype, void *stream);

/*
 * KV cache, keys: INT8 per channel over groups of block_tokens consecutive tokens
 * [P3 §11.6.3 (per-channel granularity: one scale per head-dimension channel); §11.6.4 (the outliers of K sit
 * in a few channels, so K takes per-channel scales); §11.6.5 (KIVI: K per channel within groups of tokens)].
 * For token group b = t / T and channel c: (s, z) from the range of k[bT .. bT + T - 1, c] (symmetric:
 * s = max|k| / 127; asymmetric: range widened to contain 0, s = (hi - lo) / 255, z = clamp(rne(-lo / s))),
 * codes clamp(rne(k / s) + z) -- the same arithmetic as pqg_quantize.
 *   k        : [tokens, channels] token-major, bf16 or fp32 (k_dtype); one layer's keys, heads side by side.
 *   codes    : int8 (symmetric) or uint8 [tokens, channels] (out).
 *   scales   : fp32 [tokens / T, channels] (out); zeros: uint8, same shape, NULL iff symmetric (out).
 *   block_tokens T in {32, 64, 128, 256}; tokens % T == 0 (the tokens of an incomplete group stay at full
 *   precision with the caller, see pqg_kv_append); channels % 64 == 0.
 * Alignment: k 16 bytes, codes 8, scales 4.
 */
int32_t pqg_kv_quantize_keys(const void *k, int32_t k_dtype, int64_t tokens, int64_t channels, int32_t block_tokens,
                             int32_t symmetric, void *codes, float *scales, uint8_t *zeros, void *stream);

/*
 * KV cache, keys back: out[t, c] = s[t / T, c] * (q[t, c] - z[t / T, c]), one fp32 multiply, then rounded to
 * out_dtype [P1 core formula; P3 §11.1.1].
 *   codes / scales / zeros as pqg_kv_quantize_keys writes them; out [tokens, channels] of out_dtype.
 *   tokens % T == 0; channels % 8 == 0. Alignment: codes 8 bytes, scales 4, out 16.
 * Values (per token or per group) come back with pqg_dequantize (PQG_ROW or PQG_GROUP, bits 8).
 */
int32_t pqg_kv_dequantize_keys(const void *codes, const float *scales, const uint8_t *zeros, int64_t tokens,
                               int64_t channels, int32_t block_tokens, int32_t symmetric, void *out, int32_t out_dtype,
                               void *stream);

/*
 * KV cache, one online append step for a batch of sequences, each appending one token
 * [P3 §11.6.2 (the cache is made during decoding, so it is quantized online, a few tokens per step);
 * §11.6.3 (per-token scales for V); §11.6.5 (KIVI's grouped on-demand quantization: the most recent keys stay
 * at full precision, and a complete group of T keys is quantized per channel)].
 * For each sequence b with 0 <= p = positions[b] < max_tokens (others are skipped):
 *   values: v_new[b] is quantized to INT8, one scale per token (v_group_size = 0) or per group of
 *     v_group_size channels (e.g. one head), into row p: v_codes[b, p, :], v_scales[b, p, :], v_zeros[b, p, :];
 *   keys: k_new[b] is copied to residual slot p % T of k_residual[b]; when p % T == T - 1 the group of tokens
 *     p - T + 1 .. p is complete and is quantized per channel (as pqg_kv_quantize_keys) into rows
 *     p - T + 1 .. p of k_codes[b] and group p / T of k_scales[b] (k_zeros[b]).
 *   k_new, v_new : [batch, channels], bf16 or fp32 (dtype); positions: int64 [batch], device memory.
 *   k_residual   : [batch, T, channels] of dtype (in/out, caller-owned; slots hold the keys not yet quantized).
 *   k_codes      : int8 / uint8 [batch, max_tokens, channels]; k_scales fp32 [batch, max_tokens / T, channels];
 *   k_zeros      : uint8 like k_scales, NULL iff symmetric.
 *   v_codes      : int8 / uint8 [batch, max_tokens, channels]; v_scales fp32 [batch, max_tokens, nv] with
 *                  nv = 1 or channels / v_group_size; v_zeros uint8 like v_scales, NULL iff symmetric.
 *   block_tokens T in {32, 64, 128, 256}; max_tokens % T == 0; v_group_size in {0, 32, 64, 128};
 *   channels % 64 == 0 (and % v_group_size), channels <= 8192.
 * Alignment: k_new, v_new, k_residual 16 bytes; positions, codes 8; scales 4. One block per sequence and 64
 * channels: a step reads one row of values and keys per sequence, plus T rows of keys for each sequence whose
 * group completes.
 */
int32_t pqg_kv_append(const void *k_new, const void *v_new, int32_t dtype, int64_t batch, int64_t channels,
                      const int64_t *positions, int64_t max_tokens, int32_t block_tokens, int32_t v_group_size,
                      int32_t symmetric, void *k_residual, void *k_codes, float *k_scales, uint8_t *k_zeros,
                      void *v_codes, float *v_scales, uint8_t *v_zeros, void *stream);

/*
 * INT4 group quantization with 16-bit metadata [P1 §1.1 and P3 §11.3.7: one 16-bit scale per group, about 3 %
 * of the INT4 weight bytes at g = 128 and 13 % at g = 32; the fp32 scales of pqg_quantize take twice that].
 * Per group of group_size consecutive elements of a row: the range and (s, z) exactly as pqg_quantize (bits 4,
 * PQG_GROUP); the scale is stored as binary16 s16 = fp16(s), round to nearest even (a result of 0 becomes the
 * smallest subnormal 2^-24, an overflow the largest finite 65504); the codes and the asymmetric zero point use
 * the stored scale: q = clamp(rne(x / s16) + z), z = clamp(rne(-lo / s16)), so s16 (q - z) is what the
 * metadata encodes. A group whose fp32 step is 0 stores 0 (and codes 0), as pqg_quantize does.
 *   x        : [rows, cols] bf16 or fp32 (x_dtype). cols % group_size == 0; group_size in {32, 64, 128}.
 *   codes    : packed INT4 [rows, cols / 2], as pqg_quantize writes them (out).
 *   scales16 : binary16 bits [rows * cols / group_size], row-major, the group index fastest (out).
 *   zeros4   : asymmetric zero points two per byte over the flattened group index e: byte e / 2, low nibble
 *              for even e; (rows * cols / group_size + 1) / 2 bytes; NULL iff symmetric (out).
 * Alignment: x 16 bytes, codes 4, scales16 2.
 */
int32_t pqg_quantize_meta16(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t symmetric,
                            int32_t group_size, uint8_t *codes, uint16_t *scales16, uint8_t *zeros4, void *stream);

/*
 * Dequantization of INT4 groups with 16-bit metadata: out = s16 * (q - z), one fp32 multiply, rounded to
 * out_dtype [P1 core formula; P3 §11.1.1]. Arguments as pqg_quantize_meta16 writes them; out [rows, cols].
 * Alignment: codes 4 bytes, scales16 2, out 16.
 */
int32_t pqg_dequantize_meta16(const uint8_t *codes, const uint16_t *scales16, const uint8_t *zeros4, int64_t rows,
                              int64_t cols, int32_t symmetric, int32_t group_size, void *out, int32_t out_dtype,
                              void *stream);

/*
 * W4A16 decode with 16-bit metadata: y = x W^T as pqg_qlinear_w4a16, with the weights' scales as binary16 and
 * asymmetric zero points packed (pqg_quantize_meta16), which halves the metadata bytes the decode stream reads
 * [P3 §11.1.6, §11.10.1 (decode reads every weight); P3 §11.3.7 (metadata share)].
 *   M in [0, 4] (the decode kernel; larger M returns PQG_EUNSUPPORTED: the batched kernels are bound by
 *   compute, not by these bytes). Other arguments as pqg_qlinear_w4a16.
 * Alignment: x, w_packed 16 bytes; scales16 2; y 4.
 */
int32_t pqg_qlinear_w4a16_meta16(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *w_packed,
                                 const uint16_t *scales16, const uint8_t *zeros4, int32_t group_size,
                                 int32_t symmetric, void *y, int32_t y_dtype, void *stream);

/*
 * W8A8 linear layer without any allocation: the same computation, kernels and results as pqg_qlinear_w8a8 with
 * x given, for callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Here the caller passes only the inputs and the output; the
 * per-token activation codes and scales that pqg_qlinear_w8a8 keeps in the caller's x_q / x_scales live in
 * a fixed device array inside the library (16 MiB of codes + 64 KiB of scales, one copy per GPU, held until
 * the process ends). The call itself allocates nothing.
 *   x (bf16 [M, K], required), smooth, w_q, w_scales, y, y_dtype: as pqg_qlinear_w8a8.
 *   Limits: M <= 16384 and M * K <= 2^24 (the array's size), besides those of pqg_qlinear_w8a8; larger shapes
 *   return PQG_EUNSUPPORTED before anything is enqueued.
 *   The device of `stream` must be the current device (else PQG_EINVAL). The first call on a device looks up
 *   the array's address there (a failure returns PQG_EHIP).
 * Every call on one GPU shares that GPU's array, which keeps the last call's codes and scales: two calls that
 * overlap on one GPU (different streams, or different threads without ordering) race and give undefined
 * results. Calls ordered on one stream are safe; nothing in the array needs to start at zero.
 */
int32_t pqg_qlinear_w8a8_noalloc(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales,
                                 int64_t M, int64_t N, int64_t K, void *y, int32_t y_dtype, void *stream);

/*
 * A measurement utility, no step of the method: reads a device buffer once, as a streaming read (16-byte
 * non-temporal loads, two in flight per lane, a large grid of short-lived blocks), so that the device's
 * achievable read rate can be measured and the kernels' rates set beside it.
 *   src   : device memory, 16-byte aligned; bytes: a multiple of 16 (0 enqueues nothing).
 *   sink  : device memory for one uint32; the call may write an arbitrary word there.
 * Returns PQG_EINVAL for a NULL or misaligned src (with bytes > 0), a NULL sink, or bytes not a multiple of 16.
 */
int32_t pqg_stream_read_probe(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/*
 * A measurement utility, no step of the method: the int8 matrix-core rate with no memory traffic. Enqueues
 * `blocks` blocks of 8 waves (two per SIMD, the INT8 GEMM's layout); each wave issues 12 * iters
 * v_mfma_i32_32x32x32_i8 (32 x 32 x 32 int8 products each, 65,536 ops) on 12 independent accumulators from
 * register operands. The work is blocks * 8 * 12 * iters * 65,536 ops; its rate, timed by the caller, is what the chip sustains at the clock
 * it holds under int8 matrix load, the ceiling to set the GEMM's rate against.
 *   blocks : 0 .. 65535 (0 enqueues nothing); iters: 0 .. 2^20.
 *   sink   : device memory for one uint32; the call may write an arbitrary word there.
 * Returns PQG_EINVAL for arguments out of range or a NULL sink.
 */
int32_t pqg_mfma_i8_probe(int64_t blocks, int32_t iters, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PQG_H */
