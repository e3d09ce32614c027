/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, deliberately unoptimised CPU model of the quantized linear layer. It exists to check the
 * HIP library; only the test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library and includes nothing from it.
 *
 * Numerics contract (what "bit-exact" means for the integer and fp32 results):
 *   - fp32 arithmetic is strict IEEE binary32: built with -O2 -ffp-contract=off and no fast-math, on
 *     x86-64 SSE2 (no excess precision, no fused multiply-add, no flush-to-zero);
 *   - every division and square root is the correctly rounded IEEE operation;
 *   - "round" is round-half-to-even, done with nearbyintf() in the default FE_TONEAREST mode;
 *   - reference outputs of products (W4A16, W8A8) are accumulated in binary64 / int64.
 *
 * Sources (cited by page title and section; no code is taken from them):
 *   [P1] "量化、蒸馏与模型压缩" (LLM knowledge atlas, notes 03-05)
 *   [P2] "模型压缩：量化、ZeroQuant、LLM.int8() 与 SmoothQuant" (LLM tutorial, lesson 19)
 *   [P3] "第11章 模型量化与压缩" (AI infra guide, chapter 11)
 *   [P5] "大模型压缩：从研究到生产的完整攻略（1）" (CSDN blog)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* granularity codes: the same numbering the python side uses */
enum { OR_TENSOR = 0, OR_ROW = 1, OR_GROUP = 2 };
/* smoothing modes */
enum { OR_SMOOTH_NONE = 0, OR_SMOOTH_DIV = 1, OR_SMOOTH_MUL = 2 };
/* element types of float inputs */
enum { OR_F32 = 0, OR_BF16 = 1 };

/* ---------------------------------------------------------------- bf16 <-> fp32 */

/* A bf16 value is the upper half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite binary32 to bf16, nearest, ties to even. Written as an explicit comparison of the
 * discarded 16 bits against one half so that it can be checked by eye. A carry out of the mantissa moves
 * into the exponent, which is the correct next representable value. */
uint16_t or_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == OR_BF16)
        return bf16_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

/* ---------------------------------------------------------------- affine quantization */

/* Parameters of one segment (a tensor, a row or a group). */
typedef struct {
    float s;      /* step the codes are taken with */
    float stored; /* the scale written out: s, or 0 for a segment whose step is 0 */
    int z;     /* zero point (0 when symmetric) */
    int qmin;  /* integer range */
    int qmax;
} seg_params;

/*
 * Scale and zero point of one segment from its range.
 *   symmetric  [P3 §11.1.2, §11.1.6 step 3; P5 "对称量化"]: z = 0, s = max|x| / qmax with the restricted
 *              range [-qmax, qmax], qmax = 2^(b-1) - 1 (7 for INT4, 127 for INT8).
 *   asymmetric [P3 §11.1.1; P5 "非对称量化"]: unsigned range [0, 2^b - 1],
 *              s = (hi - lo) / (2^b - 1), z = round(-lo / s) clamped into the range.
 *              The range [lo, hi] is widened to contain 0 so that z is a valid code and a real 0
 *              maps to q = z and back to exactly 0 [P5: the zero point keeps 0 exact].
 * A segment whose computed step is 0 (all values zero, or so tiny that the fp32 division underflows) has
 * no step to divide by. Its codes are taken with a unit step and z = 0 (every value then codes to 0, and no
 * division by zero can occur), and the scale it stores is the step the formula gives, 0: the dequantized
 * segment s (q - z) is exactly 0 whatever way a consumer forms the product.
 */
static seg_params segment_params(float absmax, float lo, float hi, int bits, int symmetric)
{
    seg_params p;
    if (symmetric) {
        p.qmax = (1 << (bits - 1)) - 1;
        p.qmin = -p.qmax;
        p.z = 0;
        p.s = absmax / (float)p.qmax;
        p.stored = p.s;
        if (!(p.s > 0.0f)) {
            p.s = 1.0f;
            p.stored = 0.0f;
        }
    } else {
        p.qmin = 0;
        p.qmax = (1 << bits) - 1;
        if (lo > 0.0f)
            lo = 0.0f;
        if (hi < 0.0f)
            hi = 0.0f;
        p.s = (hi - lo) / (float)p.qmax;
        p.stored = p.s;
        if (!(p.s > 0.0f)) {
            p.s = 1.0f;
            p.stored = 0.0f;
            p.z = 0;
        } else {
            /* clamped as a float, then converted (the quotient is in range here, but the order is that of
             * the definition: clamp the rounded value) */
            float zf = nearbyintf(-lo / p.s);
            if (zf < (float)p.qmin)
                zf = (float)p.qmin;
            if (zf > (float)p.qmax)
                zf = (float)p.qmax;
            p.z = (int)zf;
        }
    }
    return p;
}

/* q = clamp(round(x / s) + z, qmin, qmax)  [P1 core formula; P2 §3; P3 §11.1.1].
 * The rounding applies to x/s and z is added afterwards, as the formula is written. The sum and the clamp
 * are taken in binary32 before the conversion to int: the rounded quotient can lie far outside the int
 * range (a binary16 scale saturated at 65504 under values of 1e14 and more), and the clamp belongs to the
 * mathematical integer. Below 2^24 the sum is exact; above it, it stays beyond the code range either way. */
static int quantize_one(float v, seg_params p)
{
    float t = nearbyintf(v / p.s) + (float)p.z;
    if (t < (float)p.qmin)
        t = (float)p.qmin;
    if (t > (float)p.qmax)
        t = (float)p.qmax;
    return (int)t;
}

/* The value that enters quantization: the input, optionally divided (activations, X diag(s)^-1) or
 * multiplied (weights, diag(s) W) by the per-input-channel smoothing factor [P3 §11.4.2, §11.4.5]. */
static float smoothed(const void *x, int dtype, int64_t cols, int64_t i, const float *smooth, int mode)
{
    float v = load_elem(x, dtype, i);
    if (mode == OR_SMOOTH_DIV)
        v = v / smooth[i % cols];
    else if (mode == OR_SMOOTH_MUL)
        v = v * smooth[i % cols];
    return v;
}

/*
 * Quantize a row-major [rows, cols] tensor.
 *   granularity [P2 §4; P3 §11.1.3 Table 11-1; P1 §1.1]: one (s, z) for the whole tensor, per row (a
 *   weight output channel or an activation token), or per group of `group_size` consecutive elements
 *   along a row (the input dimension), giving rows*cols/group_size groups.
 * Outputs (caller-allocated): codes q[rows*cols] as plain ints (unpacked), scales[nseg], zeros[nseg]
 * (zeros may be NULL for symmetric). nseg = 1, rows or rows*cols/group_size.
 * Returns 0, or -1 on bad arguments.
 */
int or_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, const float *smooth, int smooth_mode,
                int bits, int symmetric, int granularity, int group_size, int32_t *q, float *scales,
                uint8_t *zeros)
{
    if (bits != 4 && bits != 8)
        return -1;
    int64_t seg_rows, seg_cols; /* shape of one segment */
    if (granularity == OR_TENSOR) {
        seg_rows = rows;
        seg_cols = cols;
    } else if (granularity == OR_ROW) {
        seg_rows = 1;
        seg_cols = cols;
    } else if (granularity == OR_GROUP) {
        if (group_size <= 0 || cols % group_size != 0)
            return -1;
        seg_rows = 1;
        seg_cols = group_size;
    } else {
        return -1;
    }
    if (rows == 0 || cols == 0)
        return 0;
    int64_t segs_per_row = cols / seg_cols;
    int64_t nseg = (rows / seg_rows) * segs_per_row;

#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t e = 0; e < nseg; ++e) {
        int64_t r0 = (e / segs_per_row) * seg_rows;
        int64_t c0 = (e % segs_per_row) * seg_cols;
        /* range of the segment */
        float absmax = 0.0f, lo = 0.0f, hi = 0.0f;
        int first = 1;
        for (int64_t r = r0; r < r0 + seg_rows; ++r) {
            for (int64_t c = c0; c < c0 + seg_cols; ++c) {
                float v = smoothed(x, x_dtype, cols, r * cols + c, smooth, smooth_mode);
                float a = fabsf(v);
                if (a > absmax)
                    absmax = a;
                if (first || v < lo)
                    lo = v;
                if (first || v > hi)
                    hi = v;
                first = 0;
            }
        }
        seg_params p = segment_params(absmax, lo, hi, bits, symmetric);
        scales[e] = p.stored;
        if (zeros)
            zeros[e] = (uint8_t)p.z;
        for (int64_t r = r0; r < r0 + seg_rows; ++r)
            for (int64_t c = c0; c < c0 + seg_cols; ++c) {
                int64_t i = r * cols + c;
                q[i] = quantize_one(smoothed(x, x_dtype, cols, i, smooth, smooth_mode), p);
            }
    }
    return 0;
}

/*
 * Static per-tensor quantization [P3 §11.1.4 static quantization: parameters fixed beforehand from
 * calibration data; §11.4.5 step 5: per-tensor INT8 activations]: every element takes the same given
 * (s, z), q = clamp(round(x / s) + z, qmin, qmax). Inputs beyond the calibrated range clip. The sum and the
 * clamp are done in binary32 before the conversion to int, so a quotient far outside the code range cannot
 * overflow an int.
 * Returns 0, or -1 on bad arguments (bits, a non-positive scale, a zero point outside the code range).
 */
int or_quantize_static(const void *x, int x_dtype, int64_t rows, int64_t cols, int bits, int symmetric,
                       float scale, int zero, int32_t *q)
{
    if (bits != 4 && bits != 8)
        return -1;
    if (!(scale > 0.0f))
        return -1;
    int qmin, qmax;
    if (symmetric) {
        qmax = (1 << (bits - 1)) - 1;
        qmin = -qmax;
        if (zero != 0)
            return -1;
    } else {
        qmin = 0;
        qmax = (1 << bits) - 1;
        if (zero < qmin || zero > qmax)
            return -1;
    }
    int64_t n = rows * cols;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float t = nearbyintf(load_elem(x, x_dtype, i) / scale) + (float)zero;
        if (t < (float)qmin)
            t = (float)qmin;
        if (t > (float)qmax)
            t = (float)qmax;
        q[i] = (int32_t)t;
    }
    return 0;
}

/*
 * The smoothed activations as a LayerNorm with the SmoothQuant factor folded into its gain would emit them
 * [P3 §11.4.4: LayerNorm(X) diag(s)^-1 = LayerNorm'(X), gamma' = gamma / s]: x'[t, j] = bf16(x[t, j] / s[j]),
 * one correctly rounded binary32 division, then round to nearest even bf16. (Reading: the folded LayerNorm
 * output is the unfolded one divided by s_j and rounded once to the activation type.)
 */
void or_fold_smoothing_bf16(const uint16_t *x, int64_t rows, int64_t cols, const float *s, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * cols; ++i)
        out[i] = or_f32_to_bf16(bf16_to_f32(x[i]) / s[i % cols]);
}

/* Segment index of flat element i, for the three granularities. */
static int64_t segment_of(int64_t i, int64_t cols, int granularity, int group_size)
{
    if (granularity == OR_TENSOR)
        return 0;
    if (granularity == OR_ROW)
        return i / cols;
    return i / group_size; /* groups are contiguous in row-major order because cols % group_size == 0 */
}

/* ---------------------------------------------------------------- 16-bit metadata */

/* binary32 -> binary16 bits, round to nearest, ties to even, with subnormal results; overflow gives inf. */
uint16_t or_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    int32_t exp = (int32_t)((u >> 23) & 0xFFu);
    uint32_t mant = u & 0x7FFFFFu;
    if (exp == 0xFF)
        return (uint16_t)(sign | 0x7C00u | (mant ? 0x200u : 0u));
    int32_t e = exp - 127 + 15; /* binary16 biased exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);
    uint32_t m;
    int shift;
    if (e <= 0) { /* subnormal result: value / 2^-24 */
        if (e < -10)
            return (uint16_t)sign; /* below 2^-25: rounds to zero */
        m = mant | 0x800000u;
        shift = 14 - e;
    } else {
        m = mant;
        shift = 13;
    }
    uint32_t q = m >> shift, rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    if (e <= 0)
        return (uint16_t)(sign | q); /* q = 0x400 is the smallest normal, encoded as such */
    return (uint16_t)(sign | (((uint32_t)e << 10) + q)); /* a carry moves into the exponent (up to inf) */
}

float or_f16_to_f32(uint16_t h)
{
    int exp = (h >> 10) & 0x1F, mant = h & 0x3FF;
    float v;
    if (exp == 0)
        v = ldexpf((float)mant, -24);
    else if (exp == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + mant), exp - 25);
    return (h & 0x8000) ? -v : v;
}

/*
 * INT4 group quantization with 16-bit metadata [P1 §1.1 and P3 §11.3.7 count one 16-bit scale per group:
 * about 3 % of the INT4 weight bytes at g = 128 and 13 % at g = 32]. Per group: the range and (s, z) as in
 * or_quantize; the scale is stored as binary16, s16 = fp16(s) rounded to nearest even (a result of 0 becomes
 * the smallest subnormal 2^-24, an overflow the largest finite 65504); the codes (and the asymmetric zero
 * point) are computed with the stored scale, q = clamp(round(x / s16) + z), z = clamp(round(-lo / s16)), so
 * that s16 (q - z) is the value the stored metadata encodes. A segment whose fp32 step is 0 stores 0 (its codes
 * are all 0, taken with the unit step as in or_quantize).
 * Outputs: q[rows * cols] unpacked, s16[rows * cols / g] binary16 bits, zeros[rows * cols / g] (NULL when
 * symmetric). Returns 0, or -1 on bad arguments.
 */
int or_quantize_meta16(const void *x, int x_dtype, int64_t rows, int64_t cols, int symmetric, int group_size,
                       int32_t *q, uint16_t *s16, uint8_t *zeros)
{
    if (group_size <= 0 || cols % group_size != 0)
        return -1;
    int64_t nseg = rows * (cols / group_size);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < nseg; ++e) {
        int64_t i0 = e * group_size; /* groups are contiguous in row-major order */
        float absmax = 0.0f, lo = 0.0f, hi = 0.0f;
        for (int64_t i = i0; i < i0 + group_size; ++i) {
            float v = load_elem(x, x_dtype, i);
            float a = fabsf(v);
            if (a > absmax)
                absmax = a;
            if (i == i0 || v < lo)
                lo = v;
            if (i == i0 || v > hi)
                hi = v;
        }
        seg_params p = segment_params(absmax, lo, hi, 4, symmetric);
        uint16_t h = or_f32_to_f16(p.s);
        if ((h & 0x7FFFu) == 0)
            h = 0x0001u;
        else if ((h & 0x7C00u) == 0x7C00u)
            h = 0x7BFFu;
        s16[e] = p.stored > 0.0f ? h : 0u;
        p.s = or_f16_to_f32(h);
        if (!symmetric) {
            /* -l / s16 can lie far beyond the int range when s16 saturated at 65504: clamp the rounded
             * value as a float, then convert */
            float l = lo > 0.0f ? 0.0f : lo;
            float zf = nearbyintf(-l / p.s);
            p.z = zf < 0.0f ? 0 : zf > 15.0f ? 15 : (int)zf;
            zeros[e] = (uint8_t)p.z;
        }
        for (int64_t i = i0; i < i0 + group_size; ++i)
            q[i] = quantize_one(load_elem(x, x_dtype, i), p);
    }
    return 0;
}

/* ---------------------------------------------------------------- KV cache */

/*
 * Keys of a KV cache, INT8 per channel over blocks of consecutive tokens [P3 §11.6.3: per-channel granularity,
 * one scale per head-dimension channel; §11.6.4: K's outliers sit in a few channels, so K takes per-channel
 * scales; §11.6.5: KIVI quantizes K per channel within groups of tokens]. x is token-major [tokens, channels]
 * (one layer's keys, all heads side by side); block b holds tokens [b T, (b + 1) T). For each block and
 * channel: the range of the channel's T values, (s, z) as for any segment, codes clamp(round(x / s) + z).
 * Outputs (caller-allocated): q[tokens * channels] unpacked, scales[tokens / T * channels] and zeros (NULL
 * when symmetric), indexed [block][channel].
 * Returns 0, or -1 when T does not divide the token count.
 */
int or_kv_keys(const void *x, int x_dtype, int64_t tokens, int64_t channels, int64_t block_tokens, int symmetric,
               int32_t *q, float *scales, uint8_t *zeros)
{
    if (block_tokens <= 0 || tokens % block_tokens != 0 || channels <= 0)
        return -1;
    int64_t nseg = tokens / block_tokens * channels;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < nseg; ++e) {
        int64_t b = e / channels, c = e % channels;
        int64_t t0 = b * block_tokens, t1 = t0 + block_tokens;
        float absmax = 0.0f, lo = 0.0f, hi = 0.0f;
        for (int64_t t = t0; t < t1; ++t) {
            float v = load_elem(x, x_dtype, t * channels + c);
            float a = fabsf(v);
            if (a > absmax)
                absmax = a;
            if (t == t0 || v < lo)
                lo = v;
            if (t == t0 || v > hi)
                hi = v;
        }
        seg_params p = segment_params(absmax, lo, hi, 8, symmetric);
        scales[e] = p.stored;
        if (zeros)
            zeros[e] = (uint8_t)p.z;
        for (int64_t t = t0; t < t1; ++t)
            q[t * channels + c] = quantize_one(load_elem(x, x_dtype, t * channels + c), p);
    }
    return 0;
}

/* Keys back from their per-channel codes: x_hat[t, c] = s[b, c] (q[t, c] - z[b, c]), b = t / T, one fp32
 * multiply; fp32 values and their bf16 rounding, as or_dequantize. */
int or_kv_dequant_keys(const int32_t *q, const float *scales, const uint8_t *zeros, int64_t tokens, int64_t channels,
                       int64_t block_tokens, float *out_f32, uint16_t *out_bf16)
{
    if (block_tokens <= 0 || tokens % block_tokens != 0)
        return -1;
    int64_t n = tokens * channels;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = i / channels, c = i % channels;
        int64_t e = t / block_tokens * channels + c;
        int z = zeros ? (int)zeros[e] : 0;
        float v = scales[e] * (float)(q[i] - z);
        if (out_f32)
            out_f32[i] = v;
        if (out_bf16)
            out_bf16[i] = or_f32_to_bf16(v);
    }
    return 0;
}

/* x_hat = s (q - z), one fp32 multiply [P1 core formula; P2 §3; P3 §11.1.1].
 * Writes fp32 values to out_f32 if non-NULL and their bf16 rounding to out_bf16 if non-NULL. */
int or_dequantize(const int32_t *q, const float *scales, const uint8_t *zeros, int64_t rows, int64_t cols,
                  int granularity, int group_size, float *out_f32, uint16_t *out_bf16)
{
    if (granularity == OR_GROUP && (group_size <= 0 || cols % group_size != 0))
        return -1;
    int64_t n = rows * cols;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t e = segment_of(i, cols, granularity, group_size);
        int z = zeros ? (int)zeros[e] : 0;
        float v = scales[e] * (float)(q[i] - z);
        if (out_f32)
            out_f32[i] = v;
        if (out_bf16)
            out_bf16[i] = or_f32_to_bf16(v);
    }
    return 0;
}

/* ---------------------------------------------------------------- INT4 storage */

/* Two 4-bit codes per byte [P3 §11.1.6 step 4 stores the codes as 4-bit integers; the byte layout is
 * not given there]. Layout used: row-major [rows, cols/2]; element 2i of a row in the low nibble of byte
 * i and element 2i+1 in the high nibble; signed codes as two's-complement nibbles. */
int or_pack_int4(const int32_t *q, int64_t rows, int64_t cols, uint8_t *out)
{
    if (cols % 2 != 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < cols / 2; ++i) {
            uint32_t lo = (uint32_t)q[r * cols + 2 * i] & 0xFu;
            uint32_t hi = (uint32_t)q[r * cols + 2 * i + 1] & 0xFu;
            out[r * (cols / 2) + i] = (uint8_t)(lo | (hi << 4));
        }
    return 0;
}

int or_unpack_int4(const uint8_t *in, int64_t rows, int64_t cols, int symmetric, int32_t *q)
{
    if (cols % 2 != 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = in[r * (cols / 2) + c / 2];
            int nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            if (symmetric && nib >= 8)
                nib -= 16;
            q[r * cols + c] = nib;
        }
    return 0;
}

/* ---------------------------------------------------------------- W4A16 reference */

/*
 * y[m, n] = sum_k x[m, k] * w_hat[n, k] with w_hat = s (q - z) per group [P3 §11.1.6 step 5: dequantize,
 * then a 16-bit matmul; here the matmul is done exactly in binary64]. x is bf16 [M, K], q unpacked
 * [N, K], scales/zeros [N, K/g]; zeros NULL for symmetric. y is binary64 [M, N], not rounded.
 */
int or_w4a16(const uint16_t *x, int64_t M, int64_t N, int64_t K, const int32_t *q, const float *scales,
             const uint8_t *zeros, int group_size, double *y)
{
    if (group_size <= 0 || K % group_size != 0)
        return -1;
    int64_t G = K / group_size;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = k / group_size;
                int z = zeros ? (int)zeros[n * G + g] : 0;
                double w_hat = (double)scales[n * G + g] * (double)(q[n * K + k] - z);
                acc += (double)bf16_to_f32(x[m * K + k]) * w_hat;
            }
            y[m * N + n] = acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- SmoothQuant factor */

/* max_t |X[t, j]| over the rows of a [rows, cols] tensor, per column j. */
static void column_absmax(const void *x, int dtype, int64_t rows, int64_t cols, float *out)
{
    for (int64_t j = 0; j < cols; ++j)
        out[j] = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            float a = fabsf(load_elem(x, dtype, r * cols + j));
            if (a > out[j])
                out[j] = a;
        }
}

/*
 * Smoothing factor per input channel j [P1 §2.3 eq. (1); P2 §13; P3 §11.4.3]:
 *   s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)
 * X is [tokens, K] (activations), W is [N, K] (our weights are stored transposed to the pages' C_in x C_out,
 * so max|W_j| is the maximum over the output rows n of column j).
 * fp32 evaluation, fixed so that the result is a single well-defined binary32:
 *   alpha = 0.5: sqrtf(ax) / sqrtf(aw)        (two correctly rounded square roots, one division)
 *   alpha = 1  : ax                          (the pages' special case: s_j = max|X_j|)
 *   alpha = 0  : 1 / aw                      (the pages' special case: s_j = 1 / max|W_j|)
 *   otherwise  : (float)(pow(ax, alpha) / pow(aw, 1 - alpha)) in binary64
 * A channel with ax = 0 or aw = 0 gets s_j = 1 (the factor is undefined there; 1 leaves it unchanged).
 */
int or_smooth(const void *x, int x_dtype, int64_t tokens, const void *w, int w_dtype, int64_t n_out, int64_t k_in,
              double alpha, float *s)
{
    float *ax = (float *)malloc(sizeof(float) * (size_t)(k_in ? k_in : 1));
    float *aw = (float *)malloc(sizeof(float) * (size_t)(k_in ? k_in : 1));
    if (!ax || !aw) {
        free(ax);
        free(aw);
        return -1;
    }
    column_absmax(x, x_dtype, tokens, k_in, ax);
    column_absmax(w, w_dtype, n_out, k_in, aw);
    for (int64_t j = 0; j < k_in; ++j) {
        float a = ax[j], b = aw[j];
        float r;
        if (a == 0.0f || b == 0.0f)
            r = 1.0f;
        else if (alpha == 0.5)
            r = sqrtf(a) / sqrtf(b);
        else if (alpha == 1.0)
            r = a;
        else if (alpha == 0.0)
            r = 1.0f / b;
        else
            r = (float)(pow((double)a, alpha) / pow((double)b, 1.0 - alpha));
        s[j] = r;
    }
    free(ax);
    free(aw);
    return 0;
}

/* ---------------------------------------------------------------- INT8 GEMM and epilogue */

/* acc[m, n] = sum_k a[m, k] * b[n, k] with exact integer arithmetic [P3 §11.1.4 and §11.4.5 step 6: INT8
 * multiply with INT32 accumulation]. Accumulates in int64; returns 1 if any result leaves int32, else 0. */
int or_gemm_s8(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K, int64_t *acc)
{
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            acc[m * N + n] = sum;
            if (sum > INT32_MAX || sum < INT32_MIN)
                overflow = 1;
        }
    return overflow;
}

/* Dequantize the integer product with the per-token activation scale and the per-output-channel weight
 * scale [P3 §11.4.5 step 6; P2 §11 vector-wise scaling]: y[m, n] = acc[m, n] * s_x[m] * s_w[n] in binary64. */
/*
 * W4A8 [P3 §11.4.5, §11.10.2: INT4 group weights stacked on INT8 per-token activations, each with its own
 * scales]: y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] * (q_w[n, k] - z[n, g]).
 * The integer sum of each group is exact (int64); the scaling and the sum over groups are binary64.
 * q_w are the unpacked codes [N, K]; z may be NULL (symmetric codes, z = 0); any g dividing K.
 */
int or_w4a8(const int8_t *xq, const float *sx, int64_t M, int64_t N, int64_t K, const int32_t *qw, const float *sw,
            const uint8_t *zw, int64_t g, double *y)
{
    if (g <= 0 || K % g != 0)
        return -1;
    const int64_t groups = K / g;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0;
            for (int64_t gi = 0; gi < groups; ++gi) {
                const int64_t z = zw ? (int64_t)zw[n * groups + gi] : 0;
                int64_t acc = 0;
                for (int64_t k = gi * g; k < (gi + 1) * g; ++k)
                    acc += (int64_t)xq[m * K + k] * ((int64_t)qw[n * K + k] - z);
                t += (double)sw[n * groups + gi] * (double)acc;
            }
            y[m * N + n] = (double)sx[m] * t;
        }
    return 0;
}

void or_w8a8_epilogue(const int64_t *acc, const float *s_x, const float *s_w, int64_t M, int64_t N, double *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * (double)s_x[m] * (double)s_w[n];
}

/* Number of host threads OpenMP will use (reported beside oracle timings). */
#ifdef _OPENMP
#include <omp.h>
int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { omp_set_num_threads(n); }
#else
int or_num_threads(void) { return 1; }
void or_set_num_threads(int n) { (void)n; }
#endif
