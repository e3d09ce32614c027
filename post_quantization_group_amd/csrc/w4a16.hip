// w4a16.hip -- weight-only INT4 x bf16 linear layer on gfx950.
//
// y[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k] * (q[n, k] - z[n, g])
// ("第11章 模型量化与压缩" §11.1.6 step 5: dequantize and multiply with 16-bit activations; §11.10.1: at decode
// every weight is read once per step, so the layer is bound by the weight stream.)
//
// Design (small M, the decode case):
//   * A wave owns R output rows and a contiguous slice of K; each lane reads 16 bytes (32 codes) of each
//     of its R rows per iteration, so one wave instruction streams 1 KB of a row (fully coalesced 128-bit
//     loads). S waves of a block split K for the same R rows and are combined once, through LDS, in a
//     fixed order (deterministic).
//   * Dequantization stays in registers and costs about one VALU instruction per code: a nibble u is
//     moved into the top four mantissa bits of a bf16 whose exponent encodes 16, giving the exact value
//     16 + u; two codes (j, j+4) of a 32-bit word share one shift and one and-or. The activations are
//     re-paired to match with v_perm, once per chunk, shared by the R rows.
//   * The products use v_dot2_f32_bf16 (two bf16 products, fp32 accumulation). The code offset is removed
//     once per 32 codes: sum x (u - off) = sum x (16 + u) - (16 + off) sum x, with off = 8 for symmetric
//     codes (two's-complement nibbles are flipped to offset binary with one xor per word) and off = z for
//     asymmetric ones. The per-group scale multiplies each 32-code partial sum.
//   * No dequantized weight is ever written to memory.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// bf16 pair holding 16 + nibble for the two nibbles selected by the shift (low half, high half).
__device__ __forceinline__ uint32_t nib_pair_shl3(uint32_t w) { return ((w << 3) & 0x00780078u) | 0x41804180u; }
template <int SHR>
__device__ __forceinline__ uint32_t nib_pair_shr(uint32_t w)
{
    return ((w >> SHR) & 0x00780078u) | 0x41804180u;
}

constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr int kMaxWavesPerRow = 16;

// MT activation rows (1..4), R weight rows per block; S = blockDim.x / 64 waves split K.
template <int MT, int R, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(1024) void k_w4a16_gemv(const uint16_t *__restrict__ x, int64_t N, int64_t K,
                                                     const uint8_t *__restrict__ w, const float *__restrict__ scales,
                                                     const uint8_t *__restrict__ zeros, int group_size,
                                                     void *__restrict__ y, int64_t y_ld)
{
    __shared__ float red[kMaxWavesPerRow][R * MT];
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int S = blockDim.x / kWave;
    const int64_t row0 = (int64_t)blockIdx.x * R;
    const int64_t chunks = K / 32;                 // 32 codes = 16 bytes per lane
    const int64_t c_begin = chunks * wv / S;
    const int64_t c_end = chunks * (wv + 1) / S;
    const int64_t groups = K / group_size;
    const int64_t wrow_bytes = K / 2;

    // rows past N (last block) read row N-1 and are never stored
    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        rows[r] = row0 + r < N ? row0 + r : N - 1;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;

    for (int64_t c = c_begin + lane; c < c_end; c += kWave) {
        uint4 wq[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            wq[r] = *reinterpret_cast<const uint4 *>(w + rows[r] * wrow_bytes + c * 16);
        float sc[R], cf[R];
        const int64_t gi = (c * 32) / group_size;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sc[r] = scales[rows[r] * groups + gi];
            cf[r] = SYM ? 24.0f : 16.0f + (float)zeros[rows[r] * groups + gi];
        }
        // activations for this chunk, re-paired as (x_j, x_{j+4}) per 8-element block
        uint32_t xp[MT][16];
        float xsum[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 *xv = reinterpret_cast<const uint4 *>(x + (int64_t)m * K + c * 32);
            float s = 0.0f;
#pragma unroll
            for (int d2 = 0; d2 < 4; ++d2) {  // one 8-element block per 16-byte load
                const uint4 u = xv[d2];
                xp[m][4 * d2 + 0] = __builtin_amdgcn_perm(u.z, u.x, 0x05040100u);
                xp[m][4 * d2 + 1] = __builtin_amdgcn_perm(u.z, u.x, 0x07060302u);
                xp[m][4 * d2 + 2] = __builtin_amdgcn_perm(u.w, u.y, 0x05040100u);
                xp[m][4 * d2 + 3] = __builtin_amdgcn_perm(u.w, u.y, 0x07060302u);
                s = dot2(u.x, kBf16OnePair, s);
                s = dot2(u.y, kBf16OnePair, s);
                s = dot2(u.z, kBf16OnePair, s);
                s = dot2(u.w, kBf16OnePair, s);
            }
            xsum[m] = s;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t wd[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
            float part[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                part[m] = 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t word = SYM ? (wd[d] ^ 0x88888888u) : wd[d];
                const uint32_t b0 = nib_pair_shl3(word);
                const uint32_t b1 = nib_pair_shr<1>(word);
                const uint32_t b2 = nib_pair_shr<5>(word);
                const uint32_t b3 = nib_pair_shr<9>(word);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    part[m] = dot2(xp[m][4 * d + 0], b0, part[m]);
                    part[m] = dot2(xp[m][4 * d + 1], b1, part[m]);
                    part[m] = dot2(xp[m][4 * d + 2], b2, part[m]);
                    part[m] = dot2(xp[m][4 * d + 3], b3, part[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[r][m] = __builtin_fmaf(sc[r], __builtin_fmaf(-cf[r], xsum[m], part[m]), acc[r][m]);
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = wave_sum(acc[r][m]);

    if (S > 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    red[wv][r * MT + m] = acc[r][m];
        }
        __syncthreads();
        if (threadIdx.x < R * MT) {
            const int r = threadIdx.x / MT, m = threadIdx.x % MT;
            float t = red[0][threadIdx.x];
            for (int i = 1; i < S; ++i)
                t += red[i][threadIdx.x];
            if (row0 + r < N) {
                if (OUT_BF16)
                    reinterpret_cast<uint16_t *>(y)[m * y_ld + row0 + r] = (uint16_t)f32_to_bf16_bits(t);
                else
                    reinterpret_cast<float *>(y)[m * y_ld + row0 + r] = t;
            }
        }
    } else if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (row0 + r < N) {
                    if (OUT_BF16)
                        reinterpret_cast<uint16_t *>(y)[m * y_ld + row0 + r] = (uint16_t)f32_to_bf16_bits(acc[r][m]);
                    else
                        reinterpret_cast<float *>(y)[m * y_ld + row0 + r] = acc[r][m];
                }
    }
}

namespace {

template <int MT, int R, bool SYM>
hipError_t gemv_launch(const W4A16Args &a, const uint16_t *x, void *y, hipStream_t st)
{
    const int64_t rowblocks = (a.N + R - 1) / R;
    const int64_t chunks = a.K / 32;
    int S = 1;
    while (S < kMaxWavesPerRow && rowblocks * S < 4096 && chunks / (2 * S) >= kWave)
        S *= 2;
    const dim3 grid((unsigned)rowblocks), block(kWave * S);
    if (a.y_bf16)
        k_w4a16_gemv<MT, R, SYM, true><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales, a.zeros, a.group_size, y,
                                                               a.N);
    else
        k_w4a16_gemv<MT, R, SYM, false><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales, a.zeros, a.group_size,
                                                                y, a.N);
    return hipGetLastError();
}

template <bool SYM>
hipError_t gemv_mt(const W4A16Args &a, int mt, const uint16_t *x, void *y, hipStream_t st)
{
    switch (mt) {
    case 1:
        return gemv_launch<1, 4, SYM>(a, x, y, st);
    case 2:
        return gemv_launch<2, 4, SYM>(a, x, y, st);
    case 3:
        return gemv_launch<3, 2, SYM>(a, x, y, st);
    default:
        return gemv_launch<4, 2, SYM>(a, x, y, st);
    }
}

}  // namespace

hipError_t launch_w4a16(const W4A16Args &a, hipStream_t st)
{
    const size_t ysz = a.y_bf16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < a.M; m0 += 4) {
        const int mt = (int)std::min<int64_t>(4, a.M - m0);
        const uint16_t *x = a.x + m0 * a.K;
        void *y = static_cast<char *>(a.y) + (size_t)m0 * (size_t)a.N * ysz;
        hipError_t e = a.symmetric ? gemv_mt<true>(a, mt, x, y, st) : gemv_mt<false>(a, mt, x, y, st);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace pqg
