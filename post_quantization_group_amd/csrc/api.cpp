// api.cpp -- the C ABI (include/pqg.h): argument validation, dispatch, error reporting.
//
// Every check runs on the host before anything is enqueued, so a rejected call leaves the stream
// untouched. The library holds no device state and allocates nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/pqg.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int32_t hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(PQG_EHIP, "%s: %s", what, hipGetErrorString(e));
    return PQG_OK;
}

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

bool valid_float_dtype(int32_t d) { return d == PQG_F32 || d == PQG_BF16; }

int32_t check_qspec(int32_t bits, int32_t symmetric, int32_t granularity, int32_t group_size, int64_t cols)
{
    if (bits != 4 && bits != 8)
        return fail(PQG_EINVAL, "bits must be 4 or 8 (got %d)", bits);
    if (symmetric != 0 && symmetric != 1)
        return fail(PQG_EINVAL, "symmetric must be 0 or 1 (got %d)", symmetric);
    if (granularity != PQG_TENSOR && granularity != PQG_ROW && granularity != PQG_GROUP)
        return fail(PQG_EINVAL, "unknown granularity %d", granularity);
    if (granularity == PQG_GROUP) {
        if (group_size != 32 && group_size != 64 && group_size != 128)
            return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
        if (cols % group_size != 0)
            return fail(PQG_EINVAL, "cols (%lld) must be a multiple of group_size (%d)", (long long)cols,
                        group_size);
    }
    return PQG_OK;
}

// Checks shared by the two W8A8 entry points (everything but the activation scratch x_q / x_scales).
int32_t check_w8a8(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales, int64_t M, int64_t N,
                   int64_t K, const void *y, int32_t y_dtype)
{
    if (M < 0 || N < 0 || K < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(y_dtype))
        return fail(PQG_EINVAL, "unknown y_dtype %d", y_dtype);
    if (K % 32 != 0)
        return fail(PQG_EINVAL, "K (%lld) must be a multiple of 32", (long long)K);
    if (K > 65536)
        return fail(PQG_EUNSUPPORTED, "K (%lld) above 65536", (long long)K);
    if (M == 0 || N == 0)
        return PQG_OK;
    if (K == 0)
        return fail(PQG_EUNSUPPORTED, "K == 0");
    if (!w_q || !w_scales || !y)
        return fail(PQG_EINVAL, "w_q, w_scales and y are required");
    if (!x && smooth)
        return fail(PQG_EINVAL, "smooth must be NULL when x is NULL (x_q / x_scales are then inputs)");
    if ((x && !aligned(x, 16)) || !aligned(w_q, 16) || !aligned(w_scales, 4) || !aligned(y, 4) ||
        (smooth && !aligned(smooth, 16)))
        return fail(PQG_EINVAL, "misaligned pointer (x, w_q, smooth: 16 bytes; scales, y: 4 bytes)");
    return PQG_OK;
}

// The activation quantize (when x is given) and the GEMM + epilogue, after the checks.
int32_t run_w8a8(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales, int64_t M, int64_t N,
                 int64_t K, void *y, int32_t y_dtype, int8_t *x_q, float *x_scales, hipStream_t st)
{
    if (x) {
        pqg::QuantArgs q{x, true, M, K, smooth, smooth ? pqg::SMOOTH_DIV : pqg::SMOOTH_NONE, 8, true, pqg::QG_ROW, 0,
                         x_q, x_scales, nullptr, nullptr};
        if (int32_t e = hip_status(pqg::launch_quantize(q, st), "W8A8 activation quantize launch"))
            return e;
    }
    pqg::GemmI8Args g{x_q, w_q, M, N, K, x_scales, w_scales, y, y_dtype == PQG_BF16};
    return hip_status(pqg::launch_gemm_i8(g, st), "W8A8 gemm launch");
}

}  // namespace

extern "C" {

int32_t pqg_abi_version(void) { return PQG_ABI_VERSION; }

const char *pqg_last_error(void) { return g_err; }

size_t pqg_quantize_workspace_bytes(int64_t rows, int64_t cols, int32_t granularity)
{
    (void)rows;
    (void)cols;
    return pqg::quantize_workspace_bytes(granularity);
}

int32_t pqg_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, const float *smooth,
                     int32_t smooth_mode, int32_t bits, int32_t symmetric, int32_t granularity, int32_t group_size,
                     void *codes, float *scales, uint8_t *zeros, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    g_err[0] = 0;
    if (rows < 0 || cols < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(x_dtype))
        return fail(PQG_EINVAL, "unknown x_dtype %d", x_dtype);
    if (int32_t e = check_qspec(bits, symmetric, granularity, group_size, cols))
        return e;
    if (smooth_mode != PQG_SMOOTH_NONE && smooth_mode != PQG_SMOOTH_DIV && smooth_mode != PQG_SMOOTH_MUL)
        return fail(PQG_EINVAL, "unknown smooth_mode %d", smooth_mode);
    if (cols % 32 != 0)
        return fail(PQG_EINVAL, "cols (%lld) must be a multiple of 32", (long long)cols);
    if (granularity == PQG_ROW && cols > 65536)
        return fail(PQG_EUNSUPPORTED, "per-row quantization supports cols <= 65536 (got %lld)", (long long)cols);
    if (rows == 0 || cols == 0)
        return PQG_OK;
    if (!x || !codes || !scales)
        return fail(PQG_EINVAL, "x, codes and scales are required");
    if (smooth_mode != PQG_SMOOTH_NONE && !smooth)
        return fail(PQG_EINVAL, "smooth vector required for smooth_mode %d", smooth_mode);
    if (smooth_mode == PQG_SMOOTH_NONE && smooth)
        return fail(PQG_EINVAL, "smooth vector given with PQG_SMOOTH_NONE");
    if (symmetric && zeros)
        return fail(PQG_EINVAL, "zeros must be NULL for symmetric quantization");
    if (!symmetric && !zeros)
        return fail(PQG_EINVAL, "zeros is required for asymmetric quantization");
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || (smooth && !aligned(smooth, 16)))
        return fail(PQG_EINVAL, "misaligned pointer (x, codes: 16 bytes; smooth: 16 bytes; scales: 4 bytes)");
    const size_t need = pqg::quantize_workspace_bytes(granularity);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(PQG_EINVAL, "workspace of %zu bytes (16-byte aligned) required", need);
    pqg::QuantArgs a{x, x_dtype == PQG_BF16, rows, cols, smooth, smooth_mode, bits, symmetric != 0,
                     granularity, group_size, codes, scales, zeros, workspace};
    return hip_status(pqg::launch_quantize(a, as_stream(stream)), "pqg_quantize launch");
}

int32_t pqg_quantize_static(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t bits,
                            int32_t symmetric, float scale, int32_t zero, void *codes, float *row_scales,
                            void *stream)
{
    g_err[0] = 0;
    if (rows < 0 || cols < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(x_dtype))
        return fail(PQG_EINVAL, "unknown x_dtype %d", x_dtype);
    if (bits != 4 && bits != 8)
        return fail(PQG_EINVAL, "bits must be 4 or 8 (got %d)", bits);
    if (!(scale > 0.0f) || !(scale <= 3.4028234663852886e38f))
        return fail(PQG_EINVAL, "scale must be finite and > 0");
    if (symmetric && zero != 0)
        return fail(PQG_EINVAL, "zero must be 0 for symmetric quantization (got %d)", zero);
    if (!symmetric && (zero < 0 || zero > (1 << bits) - 1))
        return fail(PQG_EINVAL, "zero %d outside the %d-bit code range", zero, bits);
    if (cols % 32 != 0)
        return fail(PQG_EINVAL, "cols (%lld) must be a multiple of 32", (long long)cols);
    if (rows == 0 || cols == 0)
        return PQG_OK;
    if (!x || !codes)
        return fail(PQG_EINVAL, "x and codes are required");
    if (!aligned(x, 16) || !aligned(codes, 16) || (row_scales && !aligned(row_scales, 4)))
        return fail(PQG_EINVAL, "misaligned pointer (x, codes: 16 bytes; row_scales: 4 bytes)");
    pqg::StaticQuantArgs a{x, x_dtype == PQG_BF16, rows, cols, bits, symmetric != 0, scale, zero, codes, row_scales};
    return hip_status(pqg::launch_quantize_static(a, as_stream(stream)), "pqg_quantize_static launch");
}

int32_t pqg_dequantize(const void *codes, const float *scales, const uint8_t *zeros, int64_t rows, int64_t cols,
                       int32_t bits, int32_t symmetric, int32_t granularity, int32_t group_size, void *out,
                       int32_t out_dtype, void *stream)
{
    g_err[0] = 0;
    if (rows < 0 || cols < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(out_dtype))
        return fail(PQG_EINVAL, "unknown out_dtype %d", out_dtype);
    if (int32_t e = check_qspec(bits, symmetric, granularity, group_size, cols))
        return e;
    if (cols % 32 != 0)
        return fail(PQG_EINVAL, "cols (%lld) must be a multiple of 32", (long long)cols);
    if (rows == 0 || cols == 0)
        return PQG_OK;
    if (!codes || !scales || !out)
        return fail(PQG_EINVAL, "codes, scales and out are required");
    if (symmetric && zeros)
        return fail(PQG_EINVAL, "zeros must be NULL for symmetric codes");
    if (!symmetric && !zeros)
        return fail(PQG_EINVAL, "zeros is required for asymmetric codes");
    if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(scales, 4))
        return fail(PQG_EINVAL, "misaligned pointer (codes, out: 16 bytes; scales: 4 bytes)");
    pqg::DequantArgs a{codes, scales, zeros, rows, cols, bits, symmetric != 0, granularity, group_size, out,
                       out_dtype == PQG_BF16};
    return hip_status(pqg::launch_dequantize(a, as_stream(stream)), "pqg_dequantize launch");
}

size_t pqg_smooth_workspace_bytes(int64_t tokens, int64_t out_features, int64_t in_features)
{
    if (tokens < 0 || out_features < 0 || in_features < 0)
        return 0;
    return pqg::smooth_workspace_bytes(tokens, out_features, in_features);
}

int32_t pqg_smooth(const void *x, int32_t x_dtype, int64_t tokens, const void *w, int32_t w_dtype,
                   int64_t out_features, int64_t in_features, double alpha, float *s, void *workspace,
                   size_t workspace_bytes, void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(x_dtype) || !valid_float_dtype(w_dtype))
        return fail(PQG_EINVAL, "unknown dtype");
    if (tokens < 1 || out_features < 1 || in_features < 0)
        return fail(PQG_EINVAL, "tokens and out_features must be >= 1");
    if (in_features % 8 != 0)
        return fail(PQG_EINVAL, "in_features (%lld) must be a multiple of 8", (long long)in_features);
    if (!(alpha >= 0.0 && alpha <= 1.0))
        return fail(PQG_EINVAL, "alpha must lie in [0, 1]");
    if (in_features == 0)
        return PQG_OK;
    if (!x || !w || !s)
        return fail(PQG_EINVAL, "x, w and s are required");
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(s, 4))
        return fail(PQG_EINVAL, "misaligned pointer (x, w: 16 bytes; s: 4 bytes)");
    const size_t need = pqg::smooth_workspace_bytes(tokens, out_features, in_features);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(PQG_EINVAL, "workspace of %zu bytes (16-byte aligned) required", need);
    pqg::SmoothArgs a{x, x_dtype == PQG_BF16, tokens, w, w_dtype == PQG_BF16, out_features, in_features, alpha, s,
                      workspace};
    return hip_status(pqg::launch_smooth(a, as_stream(stream)), "pqg_smooth launch");
}

int32_t pqg_qlinear_w4a16(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *w_packed,
                          const float *scales, const uint8_t *zeros, int32_t group_size, int32_t symmetric, void *y,
                          int32_t y_dtype, void *stream)
{
    g_err[0] = 0;
    if (M < 0 || N < 0 || K < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(y_dtype))
        return fail(PQG_EINVAL, "unknown y_dtype %d", y_dtype);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (K % group_size != 0)
        return fail(PQG_EINVAL, "K (%lld) must be a multiple of group_size (%d)", (long long)K, group_size);
    if (symmetric != 0 && symmetric != 1)
        return fail(PQG_EINVAL, "symmetric must be 0 or 1");
    if (M == 0 || N == 0)
        return PQG_OK;
    if (K == 0)
        return fail(PQG_EUNSUPPORTED, "K == 0");
    if (!x || !w_packed || !scales || !y)
        return fail(PQG_EINVAL, "x, w_packed, scales and y are required");
    if (symmetric && zeros)
        return fail(PQG_EINVAL, "zeros must be NULL for symmetric codes");
    if (!symmetric && !zeros)
        return fail(PQG_EINVAL, "zeros is required for asymmetric codes");
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return fail(PQG_EINVAL, "misaligned pointer (x, w_packed: 16 bytes; scales, y: 4 bytes)");
    pqg::W4A16Args a{static_cast<const uint16_t *>(x), M, N, K, w_packed, scales, zeros, group_size, symmetric != 0,
                     y, y_dtype == PQG_BF16};
    return hip_status(pqg::launch_w4a16(a, as_stream(stream)), "pqg_qlinear_w4a16 launch");
}

int32_t pqg_qlinear_w4a16_grouped(const pqg_w4a16_problem *problems, int32_t count, int64_t M, int32_t group_size,
                                  int32_t symmetric, int32_t y_dtype, void *stream)
{
    g_err[0] = 0;
    if (count < 1 || count > pqg::kMaxGroupedProblems)
        return fail(PQG_EINVAL, "count must be 1 .. %d (got %d)", pqg::kMaxGroupedProblems, count);
    if (!problems)
        return fail(PQG_EINVAL, "problems is required");
    if (M < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(y_dtype))
        return fail(PQG_EINVAL, "unknown y_dtype %d", y_dtype);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (symmetric != 0 && symmetric != 1)
        return fail(PQG_EINVAL, "symmetric must be 0 or 1");
    pqg::W4A16Args q[pqg::kMaxGroupedProblems];
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) {
        const pqg_w4a16_problem &p = problems[i];
        if (p.N < 0 || p.K < 0)
            return fail(PQG_EINVAL, "problem %d: negative shape", i);
        if (p.K % group_size != 0)
            return fail(PQG_EINVAL, "problem %d: K (%lld) must be a multiple of group_size (%d)", i, (long long)p.K,
                        group_size);
        if (M > 0 && p.N > 0) {
            if (p.K == 0)
                return fail(PQG_EUNSUPPORTED, "problem %d: K == 0", i);
            if (!p.x || !p.w_packed || !p.scales || !p.y)
                return fail(PQG_EINVAL, "problem %d: x, w_packed, scales and y are required", i);
            if (symmetric && p.zeros)
                return fail(PQG_EINVAL, "problem %d: zeros must be NULL for symmetric codes", i);
            if (!symmetric && !p.zeros)
                return fail(PQG_EINVAL, "problem %d: zeros is required for asymmetric codes", i);
            if (!aligned(p.x, 16) || !aligned(p.w_packed, 16) || !aligned(p.scales, 4) || !aligned(p.y, 4))
                return fail(PQG_EINVAL, "problem %d: misaligned pointer (x, w_packed: 16 bytes; scales, y: 4 bytes)",
                            i);
            rows += p.N;
        }
        q[i] = pqg::W4A16Args{static_cast<const uint16_t *>(p.x), M, p.N, p.K, p.w_packed, p.scales, p.zeros,
                              group_size, symmetric != 0, p.y, y_dtype == PQG_BF16};
    }
    if (M == 0 || rows == 0)
        return PQG_OK;
    if (rows > ((int64_t)1 << 33))
        return fail(PQG_EUNSUPPORTED, "more than 2^33 output rows in one launch");
    pqg::W4A16GroupedArgs a{q, count, M, group_size, symmetric != 0, y_dtype == PQG_BF16};
    return hip_status(pqg::launch_w4a16_grouped(a, as_stream(stream)), "pqg_qlinear_w4a16_grouped launch");
}

int32_t pqg_qlinear_w8a8(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales, int64_t M,
                         int64_t N, int64_t K, void *y, int32_t y_dtype, int8_t *x_q, float *x_scales, void *stream)
{
    g_err[0] = 0;
    if (int32_t e = check_w8a8(x, smooth, w_q, w_scales, M, N, K, y, y_dtype))
        return e;
    if (M == 0 || N == 0)
        return PQG_OK;
    if (!x_q || !x_scales)
        return fail(PQG_EINVAL, "x_q and x_scales are required");
    if (!aligned(x_q, 16) || !aligned(x_scales, 4))
        return fail(PQG_EINVAL, "misaligned pointer (x_q: 16 bytes; x_scales: 4 bytes)");
    return run_w8a8(x, smooth, w_q, w_scales, M, N, K, y, y_dtype, x_q, x_scales, as_stream(stream));
}

int32_t pqg_gemm_s8s8s32(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K, int32_t *c,
                         void *stream)
{
    g_err[0] = 0;
    if (M < 0 || N < 0 || K < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (K % 16 != 0)
        return fail(PQG_EINVAL, "K (%lld) must be a multiple of 16", (long long)K);
    // The kernels form 32-bit element offsets inside a tile (row * K + k) and accumulate in int32: K <= 65536
    // keeps both in range (|acc| <= 65536 * 127^2 < 2^31).
    if (K > 65536)
        return fail(PQG_EUNSUPPORTED, "K (%lld) above 65536", (long long)K);
    if (M == 0 || N == 0)
        return PQG_OK;
    if (K == 0)
        return fail(PQG_EUNSUPPORTED, "K == 0");
    if (!a || !b || !c)
        return fail(PQG_EINVAL, "a, b and c are required");
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 4))
        return fail(PQG_EINVAL, "misaligned pointer (a, b: 16 bytes; c: 4 bytes)");
    pqg::GemmI8Args g{a, b, M, N, K, nullptr, nullptr, c, false};
    return hip_status(pqg::launch_gemm_i8(g, as_stream(stream)), "pqg_gemm_s8s8s32 launch");
}

int32_t pqg_qlinear_w4a8(const int8_t *x_q, const float *x_scales, int64_t M, int64_t N, int64_t K,
                         const uint8_t *w_packed, const float *w_scales, const uint8_t *w_zeros, int32_t group_size,
                         int32_t symmetric, void *y, int32_t y_dtype, void *stream)
{
    g_err[0] = 0;
    if (M < 0 || N < 0 || K < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (!valid_float_dtype(y_dtype))
        return fail(PQG_EINVAL, "unknown y_dtype %d", y_dtype);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (K % 128 != 0)
        return fail(PQG_EINVAL, "K (%lld) must be a multiple of 128", (long long)K);
    if (K > ((int64_t)1 << 24))
        return fail(PQG_EINVAL, "K (%lld) must be at most 2^24", (long long)K);
    if (M == 0 || N == 0)
        return PQG_OK;
    if (K == 0)
        return fail(PQG_EUNSUPPORTED, "K == 0");
    if (!x_q || !x_scales || !w_packed || !w_scales || !y)
        return fail(PQG_EINVAL, "x_q, x_scales, w_packed, w_scales and y are required");
    if (symmetric && w_zeros)
        return fail(PQG_EINVAL, "w_zeros must be NULL for symmetric weight codes");
    if (!symmetric && !w_zeros)
        return fail(PQG_EINVAL, "w_zeros is required for asymmetric weight codes");
    if (!aligned(x_q, 16) || !aligned(w_packed, 16) || !aligned(x_scales, 4) || !aligned(w_scales, 4) ||
        !aligned(y, 4))
        return fail(PQG_EINVAL, "misaligned pointer (x_q, w_packed: 16 bytes; scales, y: 4 bytes)");
    pqg::W4A8Args a{x_q, x_scales, M, N, K, w_packed, w_scales, w_zeros, group_size, symmetric != 0, y,
                    y_dtype == PQG_BF16};
    return hip_status(pqg::launch_w4a8(a, as_stream(stream)), "pqg_qlinear_w4a8 launch");
}

int32_t pqg_kv_quantize_keys(const void *k, int32_t k_dtype, int64_t tokens, int64_t channels, int32_t block_tokens,
                             int32_t symmetric, void *codes, float *scales, uint8_t *zeros, void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(k_dtype))
        return fail(PQG_EINVAL, "unknown k_dtype %d", k_dtype);
    if (block_tokens != 32 && block_tokens != 64 && block_tokens != 128 && block_tokens != 256)
        return fail(PQG_EINVAL, "block_tokens must be 32, 64, 128 or 256 (got %d)", block_tokens);
    if (tokens < 0 || channels < 0 || tokens % block_tokens != 0)
        return fail(PQG_EINVAL, "tokens (%lld) must be a non-negative multiple of block_tokens", (long long)tokens);
    if (channels % 64 != 0)
        return fail(PQG_EINVAL, "channels (%lld) must be a multiple of 64", (long long)channels);
    if (tokens / block_tokens > 0x7FFFFFFF || channels / 64 > 65535)
        return fail(PQG_EINVAL, "shape too large");
    if (tokens == 0 || channels == 0)
        return PQG_OK;
    if (!k || !codes || !scales)
        return fail(PQG_EINVAL, "k, codes and scales are required");
    if (symmetric && zeros)
        return fail(PQG_EINVAL, "zeros must be NULL for symmetric codes");
    if (!symmetric && !zeros)
        return fail(PQG_EINVAL, "zeros are required for asymmetric codes");
    if (!aligned(k, 16) || !aligned(codes, 8) || !aligned(scales, 4))
        return fail(PQG_EINVAL, "misaligned pointer (k: 16 bytes, codes: 8, scales: 4)");
    pqg::KvKeysArgs a{k, k_dtype == PQG_BF16, tokens, channels, block_tokens, symmetric != 0, codes, scales, zeros};
    return hip_status(pqg::launch_kv_keys(a, as_stream(stream)), "pqg_kv_quantize_keys launch");
}

int32_t pqg_kv_dequantize_keys(const void *codes, const float *scales, const uint8_t *zeros, int64_t tokens,
                               int64_t channels, int32_t block_tokens, int32_t symmetric, void *out, int32_t out_dtype,
                               void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(out_dtype))
        return fail(PQG_EINVAL, "unknown out_dtype %d", out_dtype);
    if (block_tokens != 32 && block_tokens != 64 && block_tokens != 128 && block_tokens != 256)
        return fail(PQG_EINVAL, "block_tokens must be 32, 64, 128 or 256 (got %d)", block_tokens);
    if (tokens < 0 || channels < 0 || tokens % block_tokens != 0)
        return fail(PQG_EINVAL, "tokens (%lld) must be a non-negative multiple of block_tokens", (long long)tokens);
    if (channels % 8 != 0)
        return fail(PQG_EINVAL, "channels (%lld) must be a multiple of 8", (long long)channels);
    if (tokens == 0 || channels == 0)
        return PQG_OK;
    if (!codes || !scales || !out)
        return fail(PQG_EINVAL, "codes, scales and out are required");
    if (symmetric && zeros)
        return fail(PQG_EINVAL, "zeros must be NULL for symmetric codes");
    if (!symmetric && !zeros)
        return fail(PQG_EINVAL, "zeros are required for asymmetric codes");
    if (!aligned(codes, 8) || !aligned(scales, 4) || !aligned(out, 16))
        return fail(PQG_EINVAL, "misaligned pointer (codes: 8 bytes, scales: 4, out: 16)");
    pqg::KvKeysArgs a{nullptr, false, tokens, channels, block_tokens, symmetric != 0, const_cast<void *>(codes),
                      const_cast<float *>(scales), const_cast<uint8_t *>(zeros)};
    return hip_status(pqg::launch_kv_dequant_keys(a, out, out_dtype == PQG_BF16, as_stream(stream)),
                      "pqg_kv_dequantize_keys launch");
}

int32_t pqg_kv_append(const void *k_new, const void *v_new, int32_t dtype, int64_t batch, int64_t channels,
                      const int64_t *positions, int64_t max_tokens, int32_t block_tokens, int32_t v_group_size,
                      int32_t symmetric, void *k_residual, void *k_codes, float *k_scales, uint8_t *k_zeros,
                      void *v_codes, float *v_scales, uint8_t *v_zeros, void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(dtype))
        return fail(PQG_EINVAL, "unknown dtype %d", dtype);
    if (block_tokens != 32 && block_tokens != 64 && block_tokens != 128 && block_tokens != 256)
        return fail(PQG_EINVAL, "block_tokens must be 32, 64, 128 or 256 (got %d)", block_tokens);
    if (v_group_size != 0 && v_group_size != 32 && v_group_size != 64 && v_group_size != 128)
        return fail(PQG_EINVAL, "v_group_size must be 0 (per token), 32, 64 or 128 (got %d)", v_group_size);
    if (batch < 0 || channels < 0 || max_tokens < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (channels % 64 != 0 || channels > 8192 || (v_group_size && channels % v_group_size != 0))
        return fail(PQG_EINVAL, "channels (%lld) must be a multiple of 64 (and of v_group_size), at most 8192",
                    (long long)channels);
    if (max_tokens % block_tokens != 0)
        return fail(PQG_EINVAL, "max_tokens (%lld) must be a multiple of block_tokens", (long long)max_tokens);
    if (batch > 0x7FFFFFFF)
        return fail(PQG_EINVAL, "batch too large");
    if (batch == 0 || channels == 0 || max_tokens == 0)
        return PQG_OK;
    if (!k_new || !v_new || !positions || !k_residual || !k_codes || !k_scales || !v_codes || !v_scales)
        return fail(PQG_EINVAL, "k_new, v_new, positions, k_residual, k_codes, k_scales, v_codes and v_scales are "
                                "required");
    if (symmetric && (k_zeros || v_zeros))
        return fail(PQG_EINVAL, "k_zeros and v_zeros must be NULL for symmetric codes");
    if (!symmetric && (!k_zeros || !v_zeros))
        return fail(PQG_EINVAL, "k_zeros and v_zeros are required for asymmetric codes");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_residual, 16) || !aligned(positions, 8) ||
        !aligned(k_codes, 8) || !aligned(v_codes, 8) || !aligned(k_scales, 4) || !aligned(v_scales, 4))
        return fail(PQG_EINVAL, "misaligned pointer (k_new, v_new, k_residual: 16 bytes; positions, codes: 8; "
                                "scales: 4)");
    pqg::KvAppendArgs a{k_new,    v_new,     dtype == PQG_BF16, batch,   channels, positions, max_tokens,
                        block_tokens, v_group_size, symmetric != 0, k_residual, k_codes, k_scales, k_zeros,
                        v_codes,  v_scales,  v_zeros};
    return hip_status(pqg::launch_kv_append(a, as_stream(stream)), "pqg_kv_append launch");
}

int32_t pqg_quantize_meta16(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t symmetric,
                            int32_t group_size, uint8_t *codes, uint16_t *scales16, uint8_t *zeros4, void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(x_dtype))
        return fail(PQG_EINVAL, "unknown x_dtype %d", x_dtype);
    if (rows < 0 || cols < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (cols % group_size != 0)
        return fail(PQG_EINVAL, "cols (%lld) must be a multiple of group_size", (long long)cols);
    if (rows == 0 || cols == 0)
        return PQG_OK;
    if (!x || !codes || !scales16)
        return fail(PQG_EINVAL, "x, codes and scales16 are required");
    if (symmetric && zeros4)
        return fail(PQG_EINVAL, "zeros4 must be NULL for symmetric codes");
    if (!symmetric && !zeros4)
        return fail(PQG_EINVAL, "zeros4 is required for asymmetric codes");
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales16, 2))
        return fail(PQG_EINVAL, "misaligned pointer (x: 16 bytes, codes: 4, scales16: 2)");
    pqg::Meta16Args a{x, x_dtype == PQG_BF16, rows, cols, symmetric != 0, group_size, codes, scales16, zeros4};
    return hip_status(pqg::launch_quantize_meta16(a, as_stream(stream)), "pqg_quantize_meta16 launch");
}

int32_t pqg_dequantize_meta16(const uint8_t *codes, const uint16_t *scales16, const uint8_t *zeros4, int64_t rows,
                              int64_t cols, int32_t symmetric, int32_t group_size, void *out, int32_t out_dtype,
                              void *stream)
{
    g_err[0] = 0;
    if (!valid_float_dtype(out_dtype))
        return fail(PQG_EINVAL, "unknown out_dtype %d", out_dtype);
    if (rows < 0 || cols < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (cols % group_size != 0)
        return fail(PQG_EINVAL, "cols (%lld) must be a multiple of group_size", (long long)cols);
    if (rows == 0 || cols == 0)
        return PQG_OK;
    if (!codes || !scales16 || !out)
        return fail(PQG_EINVAL, "codes, scales16 and out are required");
    if (symmetric && zeros4)
        return fail(PQG_EINVAL, "zeros4 must be NULL for symmetric codes");
    if (!symmetric && !zeros4)
        return fail(PQG_EINVAL, "zeros4 is required for asymmetric codes");
    if (!aligned(codes, 4) || !aligned(scales16, 2) || !aligned(out, 16))
        return fail(PQG_EINVAL, "misaligned pointer (codes: 4 bytes, scales16: 2, out: 16)");
    pqg::Meta16Args a{nullptr, false, rows, cols, symmetric != 0, group_size, const_cast<uint8_t *>(codes),
                      const_cast<uint16_t *>(scales16), const_cast<uint8_t *>(zeros4)};
    return hip_status(pqg::launch_dequantize_meta16(a, out, out_dtype == PQG_BF16, as_stream(stream)),
                      "pqg_dequantize_meta16 launch");
}

int32_t pqg_qlinear_w4a16_meta16(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *w_packed,
                                 const uint16_t *scales16, const uint8_t *zeros4, int32_t group_size,
                                 int32_t symmetric, void *y, int32_t y_dtype, void *stream)
{
    g_err[0] = 0;
    if (M < 0 || N < 0 || K < 0)
        return fail(PQG_EINVAL, "negative shape");
    if (M > 4)
        return fail(PQG_EUNSUPPORTED, "16-bit metadata is read by the decode kernel only: M must be at most 4");
    if (!valid_float_dtype(y_dtype))
        return fail(PQG_EINVAL, "unknown y_dtype %d", y_dtype);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(PQG_EINVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
    if (K % group_size != 0)
        return fail(PQG_EINVAL, "K (%lld) must be a multiple of group_size (%d)", (long long)K, group_size);
    if (M == 0 || N == 0)
        return PQG_OK;
    if (K == 0)
        return fail(PQG_EUNSUPPORTED, "K == 0");
    if (!x || !w_packed || !scales16 || !y)
        return fail(PQG_EINVAL, "x, w_packed, scales16 and y are required");
    if (symmetric && zeros4)
        return fail(PQG_EINVAL, "zeros4 must be NULL for symmetric codes");
    if (!symmetric && !zeros4)
        return fail(PQG_EINVAL, "zeros4 is required for asymmetric codes");
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scales16, 2) || !aligned(y, 4))
        return fail(PQG_EINVAL, "misaligned pointer (x, w_packed: 16 bytes; scales16: 2; y: 4)");
    pqg::W4A16Args a{static_cast<const uint16_t *>(x), M, N, K, w_packed, nullptr, zeros4, group_size, symmetric != 0,
                     y, y_dtype == PQG_BF16, true, scales16};
    return hip_status(pqg::launch_w4a16(a, as_stream(stream)), "pqg_qlinear_w4a16_meta16 launch");
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free W8A8 (scratch)
//
// pqg_qlinear_w8a8_noalloc keeps the activation codes and per-token scales between its two kernels in the
// file-scope device array `scratch`: codes at offset 0 (at most kScratchCodeBytes = M * K bytes), scales at
// kScratchCodeBytes (at most kScratchTokens floats). Every GPU the library runs on holds its own copy for the
// life of the process. In host code `scratch` only names the symbol: its device address on the current device
// comes from hipGetSymbolAddress, looked up once per device on the first call there and kept in
// g_scratch_addr, and only that address is ever passed to kernels.
namespace {

constexpr int64_t kScratchCodeBytes = int64_t(1) << 24;  // 16 MiB of INT8 activation codes
constexpr int64_t kScratchTokens = 16384;                // per-token scales
constexpr int kScratchMaxDevices = 64;

}  // namespace

static __device__ __align__(256) int8_t scratch[kScratchCodeBytes + kScratchTokens * sizeof(float)];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_addr[kScratchMaxDevices];  // device address of `scratch` per device, null until looked up

// The scratch address on the current device, which must be the device of `stream` (a non-null stream).
int32_t scratch_address(void *stream, int8_t **out)
{
    int dev = -1;
    if (int32_t e = hip_status(hipGetDevice(&dev), "hipGetDevice"))
        return e;
    if (dev < 0 || dev >= kScratchMaxDevices)
        return fail(PQG_EUNSUPPORTED, "device %d: at most %d devices", dev, kScratchMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        if (int32_t e = hip_status(hipStreamGetDevice(as_stream(stream), &sdev), "hipStreamGetDevice"))
            return e;
        if (sdev != dev)
            return fail(PQG_EINVAL, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        if (int32_t e = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
            return e;
        if (!p)
            return fail(PQG_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_addr[dev] = p;
    }
    *out = static_cast<int8_t *>(g_scratch_addr[dev]);
    return PQG_OK;
}

}  // namespace

extern "C" {

int32_t pqg_qlinear_w8a8_noalloc(const void *x, const float *smooth, const int8_t *w_q, const float *w_scales,
                                 int64_t M, int64_t N, int64_t K, void *y, int32_t y_dtype, void *stream)
{
    g_err[0] = 0;
    if (int32_t e = check_w8a8(x, smooth, w_q, w_scales, M, N, K, y, y_dtype))
        return e;
    if (M > kScratchTokens)
        return fail(PQG_EUNSUPPORTED, "M (%lld) above the %lld tokens the scratch holds", (long long)M,
                    (long long)kScratchTokens);
    if (M * K > kScratchCodeBytes)
        return fail(PQG_EUNSUPPORTED, "M * K (%lld) above the %lld activation codes the scratch holds",
                    (long long)(M * K), (long long)kScratchCodeBytes);
    if (M == 0 || N == 0)
        return PQG_OK;
    if (!x)
        return fail(PQG_EINVAL, "x is required (the activation codes live in the library's scratch)");
    int8_t *base = nullptr;
    if (int32_t e = scratch_address(stream, &base))
        return e;
    int8_t *x_q = base;
    float *x_scales = reinterpret_cast<float *>(base + kScratchCodeBytes);
    return run_w8a8(x, smooth, w_q, w_scales, M, N, K, y, y_dtype, x_q, x_scales, as_stream(stream));
}

int32_t pqg_stream_read_probe(const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    g_err[0] = 0;
    if (bytes < 0 || bytes % 16 != 0)
        return fail(PQG_EINVAL, "bytes must be a non-negative multiple of 16 (got %lld)", (long long)bytes);
    if (!sink)
        return fail(PQG_EINVAL, "sink is required");
    if (bytes == 0)
        return PQG_OK;
    if (!src || !aligned(src, 16))
        return fail(PQG_EINVAL, "src must be a 16-byte aligned device pointer");
    return hip_status(pqg::launch_stream_read(src, bytes, sink, as_stream(stream)), "stream read probe");
}

int32_t pqg_mfma_i8_probe(int64_t blocks, int32_t iters, uint32_t *sink, void *stream)
{
    g_err[0] = 0;
    if (blocks < 0 || blocks > 65535)
        return fail(PQG_EINVAL, "blocks must be in [0, 65535] (got %lld)", (long long)blocks);
    if (iters < 0 || iters > (1 << 20))
        return fail(PQG_EINVAL, "iters must be in [0, 2^20] (got %d)", iters);
    if (!sink)
        return fail(PQG_EINVAL, "sink is required");
    return hip_status(pqg::launch_mfma_i8(blocks, iters, sink, as_stream(stream)), "int8 matrix-core probe");
}

}  // extern "C"
