// common.hpp -- device helpers shared by the gfx950 kernels of the quantized linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqg {

constexpr int kWave = 64;  // CDNA wavefront width

// ------------------------------------------------------------------ direct global -> LDS loads

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4] (7 = no wait), lgkmcnt
// [11:8] (15 = no wait)
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// One LDS block per (size, id): distinct objects, so the compiler keeps them apart in alias analysis (it
// would otherwise wait for every outstanding direct load into one block before reading another).
template <int BYTES, int ID>
__device__ __forceinline__ int8_t *lds_block()
{
    __shared__ __attribute__((aligned(16))) int8_t buf[BYTES];
    return buf;
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values as a packed bf16 pair (low half first) with one v_cvt_pk_bf16_f32: round to nearest even,
// the same bits as f32_to_bf16_bits on finite values (subnormals included) and on infinities.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2v_t));
}

// Load 8 consecutive elements (bf16 or fp32) as fp32. `p` must be 16-byte aligned.
template <typename XT>
__device__ __forceinline__ void load8(const XT *__restrict__ p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *__restrict__ p, float v[8])
{
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16_lo(u.x);
    v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y);
    v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z);
    v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w);
    v[7] = bf16_hi(u.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float *__restrict__ p, float v[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x;
    v[1] = a.y;
    v[2] = a.z;
    v[3] = a.w;
    v[4] = b.x;
    v[5] = b.y;
    v[6] = b.z;
    v[7] = b.w;
}

// ------------------------------------------------------------------ exact rounding of a quotient

// round-half-to-even of the correctly rounded fp32 quotient v / s, given r within one ulp of 1/s (the
// hardware reciprocal, or the correctly rounded one).
//
// Fast path: t = v * r differs from fl(v / s) by at most |v/s| * 2^-22 * (1 + 2^-23) (an ulp in r, one
// rounding in the product, one in the reference quotient). If t is farther than |t| * 2^-20 from the nearest
// half-integer, fl(v / s) lies strictly inside the same rounding interval as t and both round to the same
// integer. t - rint(t) and 0.5 - |.| are exact in that regime (Sterbenz), so the test itself is exact.
// Otherwise (a near-tie, or a non-finite t when s is subnormal) the correctly rounded division decides.
__device__ __forceinline__ float rne_quotient(float v, float s, float r)
{
    float t = v * r;
    float q = __builtin_rintf(t);
    float margin = 0.5f - __builtin_fabsf(t - q);
    if (!(margin > __builtin_fabsf(t) * 0x1p-20f))
        q = __builtin_rintf(v / s);
    return q;
}

// The margin test of rne_quotient as one fused operation: 0.5 - |t - q| is exact, so
// fma(-|t|, 2^-20, 0.5 - |t - q|) is the exact difference rounded once, whose sign is the sign of the exact
// difference (a nonzero difference of fp32 values is at least the smallest subnormal). True when t = v * r
// is safely away from a half-integer.
__device__ __forceinline__ bool rne_margin_ok(float t, float q)
{
    return __builtin_fmaf(-__builtin_fabsf(t), 0x1p-20f, 0.5f - __builtin_fabsf(t - q)) > 0.0f;
}

// rne_quotient for 8 values sharing s and r: the reciprocal products for all 8, and one branch, uniform over
// the wave and rarely taken, in which the lanes redo their near-ties with the correctly rounded division.
__device__ __forceinline__ void rne_quotient8(const float v[8], float s, float r, float q[8])
{
    uint64_t near = 0;  // lanes with a near-tie (ballots are lane masks in scalar registers)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = v[i] * r;
        q[i] = __builtin_rintf(t);
        near |= __builtin_amdgcn_ballot_w64(!rne_margin_ok(t, q[i]));
    }
    if (near) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!rne_margin_ok(v[i] * r, q[i]))
                q[i] = __builtin_rintf(v[i] / s);
    }
}

// 1/s to within one ulp (v_rcp_f32) for the reciprocal products above. Only for scales below 2^126 (then 1/s
// is a normal number) or infinite ones (r = 0, and v * 0 rounds as v / inf does); a subnormal s gives an
// infinite or inexact r whose products fail the margin test and take the division.
__device__ __forceinline__ float recip_scale(float s) { return __builtin_amdgcn_rcpf(s); }

// ------------------------------------------------------------------ segment parameters

// Scale / zero / code range of one segment from its range statistics. Mirrors the definition:
// symmetric: s = absmax / qmax; asymmetric: range widened to contain 0, s = (hi - lo) / (2^b - 1),
// z = rne(-lo / s) clamped. A step of 0 (all-zero or underflowing range) takes its codes with s = 1, z = 0
// (all 0, no division by zero) and stores the scale 0, so that s (q - z) is exactly 0 in every consumer.
struct SegParams {
    float s, r;  // step the codes are taken with and its correctly rounded reciprocal
    float st;    // the scale written out: s, or 0 when the step is 0
    float z;     // zero point (integer valued)
    float qmin, qmax;
};

template <int BITS, bool SYM>
__device__ __forceinline__ SegParams seg_params(float absmax, float lo, float hi)
{
    SegParams p;
    if (SYM) {
        constexpr int qm = (1 << (BITS - 1)) - 1;
        p.qmax = (float)qm;
        p.qmin = -(float)qm;
        p.z = 0.0f;
        p.s = absmax / (float)qm;
        p.st = p.s;
        if (!(p.s > 0.0f)) {
            p.s = 1.0f;
            p.st = 0.0f;
        }
    } else {
        constexpr int qm = (1 << BITS) - 1;
        p.qmax = (float)qm;
        p.qmin = 0.0f;
        lo = lo > 0.0f ? 0.0f : lo;
        hi = hi < 0.0f ? 0.0f : hi;
        p.s = (hi - lo) / (float)qm;
        p.st = p.s;
        if (!(p.s > 0.0f)) {
            p.s = 1.0f;
            p.st = 0.0f;
            p.z = 0.0f;
        } else {
            float z = __builtin_rintf(-lo / p.s);
            p.z = __builtin_fminf(__builtin_fmaxf(z, 0.0f), (float)qm);
        }
    }
    p.r = recip_scale(p.s);  // s < 2^126 here: at most FLT_MAX / 7 (symmetric), (2 FLT_MAX) / 15 or infinite
    return p;
}

// Integer code of one (smoothed) value: clamp(rne(v / s) + z, qmin, qmax).
__device__ __forceinline__ int code_of(float v, const SegParams &p)
{
    float q = rne_quotient(v, p.s, p.r) + p.z;
    q = __builtin_fminf(__builtin_fmaxf(q, p.qmin), p.qmax);
    return (int)q;
}

// ------------------------------------------------------------------ wave reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Max / min over aligned groups of WIDTH <= 16 lanes, every lane of a group receiving the result: a DPP
// butterfly inside the 16-lane rows (neighbours, pairs, mirrored half rows, mirrored rows), no LDS. Every lane
// of a group must be active.
template <int WIDTH>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(WIDTH >= 1 && WIDTH <= 16 && (WIDTH & (WIDTH - 1)) == 0, "groups inside one DPP row");
    if (WIDTH >= 2)
        v = __builtin_fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
    if (WIDTH >= 4)
        v = __builtin_fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
    if (WIDTH >= 8)
        v = __builtin_fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    if (WIDTH >= 16)
        v = __builtin_fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_min(float v)
{
    static_assert(WIDTH >= 1 && WIDTH <= 16 && (WIDTH & (WIDTH - 1)) == 0, "groups inside one DPP row");
    if (WIDTH >= 2)
        v = __builtin_fminf(v, dpp_f32<0xB1>(v));
    if (WIDTH >= 4)
        v = __builtin_fminf(v, dpp_f32<0x4E>(v));
    if (WIDTH >= 8)
        v = __builtin_fminf(v, dpp_f32<0x141>(v));
    if (WIDTH >= 16)
        v = __builtin_fminf(v, dpp_f32<0x140>(v));
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1)
        v = __builtin_fmaxf(v, __shfl_xor(v, off, WIDTH));
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1)
        v = __builtin_fminf(v, __shfl_xor(v, off, WIDTH));
    return v;
}

// Sum over a full wave; every lane receives the total. Order is fixed (butterfly), so the result is
// deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// Max / min over a full wave, returned as a wave-uniform value: the DPP butterfly of group_max / group_min
// inside each 16-lane row, then the four row results read out. Every lane must be active.
__device__ __forceinline__ float wave_max_uniform(float v)
{
    v = group_max<16>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_min_uniform(float v)
{
    v = group_min<16>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return __builtin_fminf(__builtin_fminf(r0, r1), __builtin_fminf(r2, r3));
}

// Sum over a full wave, returned as a wave-uniform value. Within each 16-lane row the sum is a
// butterfly of DPP moves (swap neighbours, swap pairs, mirror halves, mirror the row), so every lane of
// the row holds its row total; the four row totals are then read out and added in a fixed order.
// No LDS traffic, deterministic.
__device__ __forceinline__ float wave_sum_uniform(float v)
{
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

}  // namespace pqg
