// quantize.hip -- affine quantize / dequantize kernels for gfx950.
//
// Defines  q = clamp(round(x / s) + z, qmin, qmax)  and  x_hat = s (q - z)  ("量化、蒸馏与模型压缩", core
// formula; "第11章 模型量化与压缩" §11.1.1) at tensor, row and group granularity (§11.1.3 Table 11-1), with
// the optional SmoothQuant scaling of the input channels applied first (§11.4.2, §11.4.5).
//
// Layout on the device. Every kernel walks the tensor in chunks of 8 consecutive elements of a row: one
// 16-byte load of bf16 (two of fp32), 8 codes -> one 32-bit store (INT4, 8 nibbles) or 64-bit store
// (INT8). Groups of g elements are contiguous in row-major order (cols % g == 0), so a group is g/8
// consecutive lanes of one wave and its range is reduced with in-wave shuffles; no LDS, no barrier.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

// ------------------------------------------------------------------ shared per-chunk pieces

// 8 consecutive elements starting at element `elem`, whose first column is `col`, with the smoothing factor of
// each column applied (divided or multiplied) when SMOOTH asks for it.
template <typename XT, int SMOOTH>
__device__ __forceinline__ void load_smoothed8(const XT *__restrict__ x, const float *__restrict__ smooth,
                                               int64_t elem, int64_t col, float v[8])
{
    load8<XT>(x + elem, v);
    if (SMOOTH != SMOOTH_NONE) {
        float sv[8];
        load8<float>(smooth + col, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = (SMOOTH == SMOOTH_DIV) ? v[i] / sv[i] : v[i] * sv[i];
    }
}

template <bool SYM>
__device__ __forceinline__ void range8(const float v[8], float &absmax, float &lo, float &hi)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (SYM) {
            absmax = __builtin_fmaxf(absmax, __builtin_fabsf(v[i]));
        } else {
            lo = __builtin_fminf(lo, v[i]);
            hi = __builtin_fmaxf(hi, v[i]);
        }
    }
}

// Quantize 8 values and store their codes at element offset `elem` of the code tensor. Each code is formed as
// a float in [0, 2^BITS): clamp(rne(v / s) + z) for asymmetric codes, and for symmetric ones the
// two's-complement code plus 2^(BITS-1) (clamp(rne(v / s) + 2^(BITS-1)) over the shifted range, the same
// integer shifted). v_cvt_pk_u8_f32 writes each into a byte of a word; INT4 fields then take their nibble
// place with one shift-or (even codes in one word, odd in the other), and an xor with each field's top bit
// turns the symmetric offset codes back into two's complement.
template <int BITS, bool SYM>
__device__ __forceinline__ void store_codes8(const float v[8], const SegParams &p, void *__restrict__ codes,
                                             int64_t elem)
{
    constexpr float bias = SYM ? (float)(1 << (BITS - 1)) : 0.0f;
    constexpr uint32_t flip = SYM ? (BITS == 4 ? 0x88888888u : 0x80808080u) : 0u;
    float q[8];
    rne_quotient8(v, p.s, p.r, q);
    const float off = SYM ? bias : p.z, lo = p.qmin + bias, hi = p.qmax + bias;
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = __builtin_fminf(__builtin_fmaxf(q[i] + off, lo), hi);
    if (BITS == 4) {
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ev = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j], j, ev);
            od = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j + 1], j, od);
        }
        reinterpret_cast<uint32_t *>(codes)[elem / 8] = (ev | (od << 4)) ^ flip;
    } else {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w0 = __builtin_amdgcn_cvt_pk_u8_f32(c[j], j, w0);
            w1 = __builtin_amdgcn_cvt_pk_u8_f32(c[j + 4], j, w1);
        }
        reinterpret_cast<uint2 *>(codes)[elem / 8] = make_uint2(w0 ^ flip, w1 ^ flip);
    }
}

// ------------------------------------------------------------------ per-group

// One thread per chunk of 8; a group is LPG = g/8 consecutive lanes. (Two to eight chunks per thread, their
// loads issued together, ran 5 to 30 % slower on a 28672 x 8192 layer.)
template <typename XT, int BITS, bool SYM, int SMOOTH, int G>
__global__ __launch_bounds__(256) void k_quant_group(const XT *__restrict__ x, const float *__restrict__ smooth,
                                                     int64_t n_chunks, int64_t cols, void *__restrict__ codes,
                                                     float *__restrict__ scales, uint8_t *__restrict__ zeros)
{
    constexpr int LPG = G / 8;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // n_chunks is a multiple of LPG and groups are lane-aligned, so a group is either wholly in range or
    // wholly out of it; the reductions below only read lanes of the same group.
    if (c >= n_chunks)
        return;
    float v[8];
    load_smoothed8<XT, SMOOTH>(x, smooth, c * 8, SMOOTH != SMOOTH_NONE ? (c * 8) % cols : 0, v);
    float absmax = 0.0f, lo = v[0], hi = v[0];
    range8<SYM>(v, absmax, lo, hi);
    if (SYM) {
        absmax = group_max<LPG>(absmax);
    } else {
        lo = group_min<LPG>(lo);
        hi = group_max<LPG>(hi);
    }
    const SegParams p = seg_params<BITS, SYM>(absmax, lo, hi);
    store_codes8<BITS, SYM>(v, p, codes, c * 8);
    if ((c % LPG) == 0) {
        scales[c / LPG] = p.st;
        if (!SYM)
            zeros[c / LPG] = (uint8_t)p.z;
    }
}

// ------------------------------------------------------------------ per-group, 16-bit metadata
//
// INT4 groups with binary16 scales and zero points packed two per byte ("第11章 模型量化与压缩" §11.3.7 and
// the atlas's §1.1 count one 16-bit scale per group). The group's (s, z) as above; the scale is stored as the
// nearest-even binary16 (0 -> the smallest subnormal, overflow -> the largest finite value), and the codes and
// the asymmetric zero point are computed with the stored scale, so that s16 (q - z) is what the metadata encodes.
// A segment whose fp32 step is 0 stores 0 (its codes, all 0, are taken with the unit step).
template <bool SYM>
__device__ __forceinline__ uint16_t meta16_params(SegParams &p, float lo)
{
    uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)p.s);
    if ((h & 0x7FFFu) == 0)
        h = 0x0001u;
    else if ((h & 0x7C00u) == 0x7C00u)
        h = 0x7BFFu;
    p.s = (float)__builtin_bit_cast(_Float16, h);
    p.r = recip_scale(p.s);  // a binary16 scale: 1/s is a normal fp32 number
    if (!SYM) {
        const float l = lo > 0.0f ? 0.0f : lo;
        p.z = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(-l / p.s), 0.0f), 15.0f);
    }
    return p.st > 0.0f ? h : (uint16_t)0;
}

// One thread per chunk of 8 as k_quant_group; the zero points of groups 2i and 2i + 1 (LPG lanes apart, in one
// wave) are combined by the first group's leader into byte i.
template <typename XT, bool SYM, int G>
__global__ __launch_bounds__(256) void k_quant_group16(const XT *__restrict__ x, int64_t n_chunks,
                                                       uint8_t *__restrict__ codes, uint16_t *__restrict__ scales16,
                                                       uint8_t *__restrict__ zeros4)
{
    constexpr int LPG = G / 8;
    static_assert(2 * LPG <= kWave, "a pair of groups lies in one wave");
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = c < n_chunks;  // groups are wholly in or out of range (n_chunks % LPG == 0)
    float v[8];
    if (live)
        load8<XT>(x + c * 8, v);
    else
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = 0.0f;
    float absmax = 0.0f, lo = v[0], hi = v[0];
    range8<SYM>(v, absmax, lo, hi);
    if (SYM) {
        absmax = group_max<LPG>(absmax);
    } else {
        lo = group_min<LPG>(lo);
        hi = group_max<LPG>(hi);
    }
    SegParams p = seg_params<4, SYM>(absmax, lo, hi);
    const uint16_t h = meta16_params<SYM>(p, lo);
    const int zn = __shfl_down((int)p.z, LPG, kWave);  // the next group's zero point (leader lanes only)
    if (!live)
        return;
    store_codes8<4, SYM>(v, p, codes, c * 8);
    if ((c % LPG) == 0) {
        const int64_t e = c / LPG;
        scales16[e] = h;
        if (!SYM && (e % 2) == 0) {
            const int64_t ngroups = n_chunks / LPG;
            const uint32_t hi4 = e + 1 < ngroups ? (uint32_t)zn : 0u;
            zeros4[e / 2] = (uint8_t)((uint32_t)p.z | (hi4 << 4));
        }
    }
}

// ------------------------------------------------------------------ per-row

constexpr int kRowCache = 8;  // chunks of 8 kept in registers per thread: cols <= 1024 * 8 * 8

template <int BITS, bool SYM, int NT>
__device__ __forceinline__ void block_range(float &absmax, float &lo, float &hi, float *red)
{
    // red: LDS of 3 * (NT / 64) floats
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    if (SYM) {
        absmax = wave_max_uniform(absmax);
    } else {
        lo = wave_min_uniform(lo);
        hi = wave_max_uniform(hi);
    }
    if (lane == 0) {
        red[wv] = absmax;
        red[NW + wv] = lo;
        red[2 * NW + wv] = hi;
    }
    __syncthreads();
    absmax = red[0];
    lo = red[NW];
    hi = red[2 * NW];
    for (int i = 1; i < NW; ++i) {
        absmax = __builtin_fmaxf(absmax, red[i]);
        lo = __builtin_fminf(lo, red[NW + i]);
        hi = __builtin_fmaxf(hi, red[2 * NW + i]);
    }
}

// One block of NT threads per row. The smoothed values are computed once and kept in registers between
// the range pass and the code pass.
template <typename XT, int BITS, bool SYM, int SMOOTH, int NT, int RC = kRowCache>
__global__ __launch_bounds__(NT) void k_quant_row(const XT *__restrict__ x, const float *__restrict__ smooth,
                                                  int64_t cols, void *__restrict__ codes,
                                                  float *__restrict__ scales, uint8_t *__restrict__ zeros)
{
    __shared__ float red[3 * (NT / kWave)];
    const int64_t row = blockIdx.x;
    const int64_t nch = cols / 8;
    const int64_t base = row * cols;
    float v[RC][8];
    // Loads first, all in flight together: the iteration count is uniform, and a lane past the row's end in the
    // last iteration re-reads the row's last chunk (no load sits under a divergent branch, which would make
    // the compiler wait for every outstanding load at the branch's join). Then the range, over own chunks only.
    // The raw loads of every chunk go out in one loop, and the arithmetic follows in another, so that no
    // chunk's smoothing waits for its data before the next chunk's loads are issued.
    const int iters = (int)((nch + NT - 1) / NT);
    constexpr int XW = sizeof(XT) * 8 / 16;  // 16-byte words per chunk of x: 1 (bf16) or 2 (fp32)
    uint4 xr[RC][XW];
    float4 sr[RC][SMOOTH != SMOOTH_NONE ? 2 : 1];
#pragma unroll
    for (int i = 0; i < RC; ++i)
        if (i < iters) {
            const int64_t ch = std::min<int64_t>(threadIdx.x + (int64_t)i * NT, nch - 1);
            const uint4 *xp = reinterpret_cast<const uint4 *>(x + base + ch * 8);
#pragma unroll
            for (int q = 0; q < XW; ++q)
                xr[i][q] = xp[q];
            if (SMOOTH != SMOOTH_NONE) {
                sr[i][0] = reinterpret_cast<const float4 *>(smooth + ch * 8)[0];
                sr[i][SMOOTH != SMOOTH_NONE ? 1 : 0] = reinterpret_cast<const float4 *>(smooth + ch * 8)[1];
            }
        }
#pragma unroll
    for (int i = 0; i < RC; ++i)
        if (i < iters) {
            if (XW == 1) {
                v[i][0] = bf16_lo(xr[i][0].x);
                v[i][1] = bf16_hi(xr[i][0].x);
                v[i][2] = bf16_lo(xr[i][0].y);
                v[i][3] = bf16_hi(xr[i][0].y);
                v[i][4] = bf16_lo(xr[i][0].z);
                v[i][5] = bf16_hi(xr[i][0].z);
                v[i][6] = bf16_lo(xr[i][0].w);
                v[i][7] = bf16_hi(xr[i][0].w);
            } else {
#pragma unroll
                for (int q = 0; q < XW; ++q) {
                    v[i][4 * q + 0] = __uint_as_float(xr[i][q].x);
                    v[i][4 * q + 1] = __uint_as_float(xr[i][q].y);
                    v[i][4 * q + 2] = __uint_as_float(xr[i][q].z);
                    v[i][4 * q + 3] = __uint_as_float(xr[i][q].w);
                }
            }
            if (SMOOTH != SMOOTH_NONE) {
                const float4 a0 = sr[i][0], a1 = sr[i][SMOOTH != SMOOTH_NONE ? 1 : 0];
                const float sv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[i][e] = (SMOOTH == SMOOTH_DIV) ? v[i][e] / sv[e] : v[i][e] * sv[e];
            }
        }
    // a thread without elements must not disturb the reduction: lo = +inf, hi = -inf until its first chunk
    float absmax = 0.0f, lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < RC; ++i)
        if (i < iters && threadIdx.x + (int64_t)i * NT < nch)
            range8<SYM>(v[i], absmax, lo, hi);
    block_range<BITS, SYM, NT>(absmax, lo, hi, red);
    const SegParams p = seg_params<BITS, SYM>(absmax, lo, hi);
#pragma unroll
    for (int i = 0; i < RC; ++i) {
        const int64_t ch = threadIdx.x + (int64_t)i * NT;
        if (ch < nch)
            store_codes8<BITS, SYM>(v[i], p, codes, base + ch * 8);
    }
    if (threadIdx.x == 0) {
        scales[row] = p.st;
        if (!SYM)
            zeros[row] = (uint8_t)p.z;
    }
}

// ------------------------------------------------------------------ per-tensor (two launches)

constexpr int kTensorBlocks = 1024;

// Pass 1: per-block range over a grid-stride range of chunks -> ws[3 * blockIdx.x + {0,1,2}].
template <typename XT, bool SYM, int SMOOTH>
__global__ __launch_bounds__(256) void k_tensor_range(const XT *__restrict__ x, const float *__restrict__ smooth,
                                                      int64_t n_chunks, int64_t cols, float *__restrict__ ws)
{
    __shared__ float red[3 * 4];
    float absmax = 0.0f, lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n_chunks; c += (int64_t)gridDim.x * 256) {
        float v[8];
        load_smoothed8<XT, SMOOTH>(x, smooth, c * 8, SMOOTH != SMOOTH_NONE ? (c * 8) % cols : 0, v);
        range8<SYM>(v, absmax, lo, hi);
    }
    block_range<8, SYM, 256>(absmax, lo, hi, red);
    if (threadIdx.x == 0) {
        ws[3 * blockIdx.x + 0] = absmax;
        ws[3 * blockIdx.x + 1] = lo;
        ws[3 * blockIdx.x + 2] = hi;
    }
}

// Pass 2: every block reduces the partial ranges itself (max / min are exact and order independent, so
// all blocks agree), then quantizes its grid-stride share.
template <typename XT, int BITS, bool SYM, int SMOOTH>
__global__ __launch_bounds__(256) void k_tensor_quant(const XT *__restrict__ x, const float *__restrict__ smooth,
                                                      int64_t n_chunks, int64_t cols, const float *__restrict__ ws,
                                                      int n_partials, void *__restrict__ codes,
                                                      float *__restrict__ scales, uint8_t *__restrict__ zeros)
{
    __shared__ float red[3 * 4];
    float absmax = 0.0f, lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    for (int i = threadIdx.x; i < n_partials; i += 256) {
        absmax = __builtin_fmaxf(absmax, ws[3 * i + 0]);
        lo = __builtin_fminf(lo, ws[3 * i + 1]);
        hi = __builtin_fmaxf(hi, ws[3 * i + 2]);
    }
    block_range<BITS, SYM, 256>(absmax, lo, hi, red);
    const SegParams p = seg_params<BITS, SYM>(absmax, lo, hi);
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n_chunks; c += (int64_t)gridDim.x * 256) {
        float v[8];
        load_smoothed8<XT, SMOOTH>(x, smooth, c * 8, SMOOTH != SMOOTH_NONE ? (c * 8) % cols : 0, v);
        store_codes8<BITS, SYM>(v, p, codes, c * 8);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        scales[0] = p.st;
        if (!SYM)
            zeros[0] = (uint8_t)p.z;
    }
}

// ------------------------------------------------------------------ static per-tensor

// Fixed (scale, zero) from calibration ("第11章 模型量化与压缩" §11.1.4 static quantization; §11.4.5 step 5):
// the same code step as above with the segment parameters given instead of measured. Grid-stride over
// chunks of 8, kStaticUnroll chunks per thread per pass with their loads issued together (one chunk per
// thread left the stream latency-bound); the first `rows` threads also write the per-token copy of the scale.
constexpr int kStaticUnroll = 4;

template <typename XT, int BITS, bool SYM>
__global__ __launch_bounds__(256) void k_quant_static(const XT *__restrict__ x, int64_t n_chunks, float scale,
                                                      float zero, void *__restrict__ codes,
                                                      float *__restrict__ row_scales, int64_t rows)
{
    SegParams p;
    p.s = scale;
    p.st = scale;
    p.r = 1.0f / scale;  // any scale a caller passes: the correctly rounded reciprocal (once per thread)
    p.z = zero;
    p.qmax = SYM ? (float)((1 << (BITS - 1)) - 1) : (float)((1 << BITS) - 1);
    p.qmin = SYM ? -p.qmax : 0.0f;
    const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x, stride = (int64_t)gridDim.x * 256;
    if (row_scales)
        for (int64_t r = t0; r < rows; r += stride)
            row_scales[r] = scale;
    for (int64_t c0 = t0; c0 < n_chunks; c0 += stride * kStaticUnroll) {
        float v[kStaticUnroll][8];
#pragma unroll
        for (int u = 0; u < kStaticUnroll; ++u)
            if (c0 + u * stride < n_chunks)
                load8<XT>(x + (c0 + u * stride) * 8, v[u]);
#pragma unroll
        for (int u = 0; u < kStaticUnroll; ++u)
            if (c0 + u * stride < n_chunks)
                store_codes8<BITS, SYM>(v[u], p, codes, (c0 + u * stride) * 8);
    }
}

// ------------------------------------------------------------------ dequantize

template <int BITS, bool SYM, int GRAN, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_dequant(const void *__restrict__ codes, const float *__restrict__ scales,
                                                 const uint8_t *__restrict__ zeros, int64_t n_chunks,
                                                 int64_t cols, int group_size, int seg_shift,
                                                 void *__restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n_chunks)
        return;
    const int64_t e = c * 8;
    // the segment: a shift when its length (row or group) is a power of two (seg_shift >= 0, uniform)
    const int64_t len = (GRAN == QG_ROW) ? cols : (int64_t)group_size;
    const int64_t seg = (GRAN == QG_TENSOR) ? 0 : seg_shift >= 0 ? e >> seg_shift : e / len;
    const float s = scales[seg];
    // codes as offset-binary bytes (symmetric two's-complement fields xor their top bit), converted to float
    // by the byte conversions; q - z = u - (bias + z), exact in fp32
    const float zb = (SYM ? (float)(1 << (BITS - 1)) : 0.0f) + (SYM ? 0.0f : (float)zeros[seg]);
    float u[8];
    if (BITS == 4) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(codes)[c] ^ (SYM ? 0x88888888u : 0u);
        const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;  // codes 0, 2, 4, 6 and 1, 3, 5, 7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[2 * j] = (float)((ev >> (8 * j)) & 0xFFu);
            u[2 * j + 1] = (float)((od >> (8 * j)) & 0xFFu);
        }
    } else {
        const uint2 w = reinterpret_cast<const uint2 *>(codes)[c];
        const uint32_t w0 = w.x ^ (SYM ? 0x80808080u : 0u), w1 = w.y ^ (SYM ? 0x80808080u : 0u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] = (float)((w0 >> (8 * j)) & 0xFFu);
            u[j + 4] = (float)((w1 >> (8 * j)) & 0xFFu);
        }
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = s * (u[i] - zb);
    if (OUT_BF16) {
        uint4 o = make_uint4(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]), pack_bf16x2_rne(v[4], v[5]),
                             pack_bf16x2_rne(v[6], v[7]));
        reinterpret_cast<uint4 *>(out)[c] = o;
    } else {
        float4 *o = reinterpret_cast<float4 *>(out) + 2 * c;
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// INT4 groups with binary16 scales and packed zero points back to fp32 / bf16.
template <bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_dequant16(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales16,
                                                   const uint8_t *__restrict__ zeros4, int64_t n_chunks, int group_size,
                                                   void *__restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n_chunks)
        return;
    const int64_t seg = c * 8 / group_size;
    const float s = (float)__builtin_bit_cast(_Float16, scales16[seg]);
    const int z = SYM ? 0 : (int)((zeros4[seg / 2] >> (4 * (seg % 2))) & 0xFu);
    const uint32_t w = reinterpret_cast<const uint32_t *>(codes)[c];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int nib = (int)((w >> (4 * i)) & 0xFu);
        const int q = (SYM && nib >= 8) ? nib - 16 : nib;
        v[i] = s * (float)(q - z);
    }
    if (OUT_BF16) {
        reinterpret_cast<uint4 *>(out)[c] = make_uint4(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]),
                                                       pack_bf16x2_rne(v[4], v[5]), pack_bf16x2_rne(v[6], v[7]));
    } else {
        float4 *o = reinterpret_cast<float4 *>(out) + 2 * c;
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ------------------------------------------------------------------ host-side dispatch

namespace {

inline unsigned nblocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

template <typename XT, int BITS, bool SYM, int SMOOTH>
hipError_t quant_dispatch_gran(const QuantArgs &a, hipStream_t st)
{
    const int64_t n_chunks = a.rows * a.cols / 8;
    const XT *x = static_cast<const XT *>(a.x);
    if (a.granularity == QG_GROUP) {
        const unsigned nb = nblocks(n_chunks, 256);
        switch (a.group_size) {
        case 32:
            k_quant_group<XT, BITS, SYM, SMOOTH, 32><<<nb, 256, 0, st>>>(x, a.smooth, n_chunks, a.cols, a.codes,
                                                                         a.scales, a.zeros);
            break;
        case 64:
            k_quant_group<XT, BITS, SYM, SMOOTH, 64><<<nb, 256, 0, st>>>(x, a.smooth, n_chunks, a.cols, a.codes,
                                                                         a.scales, a.zeros);
            break;
        default:
            k_quant_group<XT, BITS, SYM, SMOOTH, 128><<<nb, 256, 0, st>>>(x, a.smooth, n_chunks, a.cols, a.codes,
                                                                          a.scales, a.zeros);
            break;
        }
    } else if (a.granularity == QG_ROW) {
        // threads per row: enough that each keeps at most kRowCache chunks in registers (four waves per row for
        // a 2048 x 4096 batch of tokens measured no faster than one)
        const int64_t nch = a.cols / 8;
        const unsigned grid = (unsigned)a.rows;
        if (nch <= 64 * 2)  // short rows (at most 1024 columns): two chunks per thread, fewer registers
            k_quant_row<XT, BITS, SYM, SMOOTH, 64, 2><<<grid, 64, 0, st>>>(x, a.smooth, a.cols, a.codes, a.scales,
                                                                          a.zeros);
        else if (nch <= 256 * kRowCache / 4)  // 64 threads
            k_quant_row<XT, BITS, SYM, SMOOTH, 64><<<grid, 64, 0, st>>>(x, a.smooth, a.cols, a.codes, a.scales,
                                                                       a.zeros);
        else if (nch <= 256 * kRowCache)
            k_quant_row<XT, BITS, SYM, SMOOTH, 256><<<grid, 256, 0, st>>>(x, a.smooth, a.cols, a.codes, a.scales,
                                                                         a.zeros);
        else
            k_quant_row<XT, BITS, SYM, SMOOTH, 1024><<<grid, 1024, 0, st>>>(x, a.smooth, a.cols, a.codes, a.scales,
                                                                           a.zeros);
    } else {
        float *ws = static_cast<float *>(a.workspace);
        const int nb = (int)std::min<int64_t>(kTensorBlocks, std::max<int64_t>(1, (n_chunks + 255) / 256));
        k_tensor_range<XT, SYM, SMOOTH><<<nb, 256, 0, st>>>(x, a.smooth, n_chunks, a.cols, ws);
        k_tensor_quant<XT, BITS, SYM, SMOOTH><<<nb, 256, 0, st>>>(x, a.smooth, n_chunks, a.cols, ws, nb, a.codes,
                                                                  a.scales, a.zeros);
    }
    return hipGetLastError();
}

template <typename XT, int BITS, bool SYM>
hipError_t quant_dispatch_smooth(const QuantArgs &a, hipStream_t st)
{
    switch (a.smooth_mode) {
    case SMOOTH_DIV:
        return quant_dispatch_gran<XT, BITS, SYM, SMOOTH_DIV>(a, st);
    case SMOOTH_MUL:
        return quant_dispatch_gran<XT, BITS, SYM, SMOOTH_MUL>(a, st);
    default:
        return quant_dispatch_gran<XT, BITS, SYM, SMOOTH_NONE>(a, st);
    }
}

template <typename XT>
hipError_t quant_dispatch_type(const QuantArgs &a, hipStream_t st)
{
    if (a.bits == 4)
        return a.symmetric ? quant_dispatch_smooth<XT, 4, true>(a, st) : quant_dispatch_smooth<XT, 4, false>(a, st);
    return a.symmetric ? quant_dispatch_smooth<XT, 8, true>(a, st) : quant_dispatch_smooth<XT, 8, false>(a, st);
}

// log2(n) when n is a power of two, else -1
inline int pow2_shift(int64_t n)
{
    if (n <= 0 || (n & (n - 1)) != 0)
        return -1;
    int k = 0;
    while ((int64_t(1) << k) < n)
        ++k;
    return k;
}

template <int BITS, bool SYM, int GRAN>
hipError_t dequant_out(const DequantArgs &a, hipStream_t st)
{
    const int64_t n_chunks = a.rows * a.cols / 8;
    const unsigned nb = nblocks(n_chunks, 256);
    const int shift = pow2_shift(GRAN == QG_ROW ? a.cols : (int64_t)a.group_size);
    if (a.out_bf16)
        k_dequant<BITS, SYM, GRAN, true><<<nb, 256, 0, st>>>(a.codes, a.scales, a.zeros, n_chunks, a.cols,
                                                             a.group_size, shift, a.out);
    else
        k_dequant<BITS, SYM, GRAN, false><<<nb, 256, 0, st>>>(a.codes, a.scales, a.zeros, n_chunks, a.cols,
                                                              a.group_size, shift, a.out);
    return hipGetLastError();
}

template <int BITS, bool SYM>
hipError_t dequant_gran(const DequantArgs &a, hipStream_t st)
{
    switch (a.granularity) {
    case QG_TENSOR:
        return dequant_out<BITS, SYM, QG_TENSOR>(a, st);
    case QG_ROW:
        return dequant_out<BITS, SYM, QG_ROW>(a, st);
    default:
        return dequant_out<BITS, SYM, QG_GROUP>(a, st);
    }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st)
{
    if (a.x_bf16)
        return quant_dispatch_type<uint16_t>(a, st);
    return quant_dispatch_type<float>(a, st);
}

size_t quantize_workspace_bytes(int32_t granularity)
{
    return granularity == QG_TENSOR ? (size_t)kTensorBlocks * 3 * sizeof(float) : 0;
}

template <typename XT, int BITS, bool SYM>
hipError_t static_launch(const StaticQuantArgs &a, hipStream_t st)
{
    const int64_t n_chunks = a.rows * a.cols / 8;
    const int64_t want = std::max<int64_t>((n_chunks + 256 * kStaticUnroll - 1) / (256 * kStaticUnroll),
                                           (a.rows + 255) / 256);
    const int64_t blocks = std::min<int64_t>(want, 4096);  // grid-stride beyond 16 blocks per CU
    k_quant_static<XT, BITS, SYM><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
        static_cast<const XT *>(a.x), n_chunks, a.scale, (float)a.zero, a.codes, a.row_scales, a.rows);
    return hipGetLastError();
}

template <typename XT>
hipError_t static_type(const StaticQuantArgs &a, hipStream_t st)
{
    if (a.bits == 4)
        return a.symmetric ? static_launch<XT, 4, true>(a, st) : static_launch<XT, 4, false>(a, st);
    return a.symmetric ? static_launch<XT, 8, true>(a, st) : static_launch<XT, 8, false>(a, st);
}

hipError_t launch_quantize_static(const StaticQuantArgs &a, hipStream_t st)
{
    return a.x_bf16 ? static_type<uint16_t>(a, st) : static_type<float>(a, st);
}

namespace {

template <typename XT, bool SYM>
hipError_t quant16_go(const Meta16Args &a, hipStream_t st)
{
    const int64_t n_chunks = a.rows * a.cols / 8;
    const unsigned nb = nblocks(n_chunks, 256);
    const XT *x = static_cast<const XT *>(a.x);
    switch (a.group_size) {
    case 32:
        k_quant_group16<XT, SYM, 32><<<nb, 256, 0, st>>>(x, n_chunks, a.codes, a.scales16, a.zeros4);
        break;
    case 64:
        k_quant_group16<XT, SYM, 64><<<nb, 256, 0, st>>>(x, n_chunks, a.codes, a.scales16, a.zeros4);
        break;
    default:
        k_quant_group16<XT, SYM, 128><<<nb, 256, 0, st>>>(x, n_chunks, a.codes, a.scales16, a.zeros4);
        break;
    }
    return hipGetLastError();
}

template <bool SYM>
hipError_t dequant16_go(const Meta16Args &a, void *out, bool out_bf16, hipStream_t st)
{
    const int64_t n_chunks = a.rows * a.cols / 8;
    const unsigned nb = nblocks(n_chunks, 256);
    if (out_bf16)
        k_dequant16<SYM, true><<<nb, 256, 0, st>>>(a.codes, a.scales16, a.zeros4, n_chunks, a.group_size, out);
    else
        k_dequant16<SYM, false><<<nb, 256, 0, st>>>(a.codes, a.scales16, a.zeros4, n_chunks, a.group_size, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_meta16(const Meta16Args &a, hipStream_t st)
{
    if (a.x_bf16)
        return a.symmetric ? quant16_go<uint16_t, true>(a, st) : quant16_go<uint16_t, false>(a, st);
    return a.symmetric ? quant16_go<float, true>(a, st) : quant16_go<float, false>(a, st);
}

hipError_t launch_dequantize_meta16(const Meta16Args &a, void *out, bool out_bf16, hipStream_t st)
{
    return a.symmetric ? dequant16_go<true>(a, out, out_bf16, st) : dequant16_go<false>(a, out, out_bf16, st);
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t st)
{
    if (a.bits == 4)
        return a.symmetric ? dequant_gran<4, true>(a, st) : dequant_gran<4, false>(a, st);
    return a.symmetric ? dequant_gran<8, true>(a, st) : dequant_gran<8, false>(a, st);
}

}  // namespace pqg
