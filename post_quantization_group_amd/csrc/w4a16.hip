// w4a16.hip -- weight-only INT4 x bf16 linear layer on gfx950.
//
// y[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k] * (q[n, k] - z[n, g])
// ("第11章 模型量化与压缩" §11.1.6 step 5: dequantize and multiply with 16-bit activations; §11.10.1: at decode
// every weight is read once per step, so the layer is bound by the weight stream.)
//
// Design (small M, the decode case):
//   * A block owns R output rows; its S waves split K into contiguous slices. Each lane reads 16 bytes
//     (32 codes) of each of the R rows per iteration, so one wave instruction streams 1 KB of a row
//     (fully coalesced 128-bit loads, non-temporal: the weight stream is read once and should not evict
//     the activations from the caches). Row base pointers are uniform (scalar registers) and lanes add
//     32-bit offsets, so addressing costs almost no vector instructions. The S partial sums of a row are
//     combined once, through LDS, in a fixed order (deterministic).
//   * Two register stages alternate, so the next chunk's loads are in flight while the current one is
//     reduced. The loop has a uniform trip count and no branches: every iteration loads (addresses past
//     the slice are clamped to its last chunk) and computes, and chunks outside the slice get a zero
//     scale. Divergent branches around the loads would make the compiler drain all outstanding loads at
//     their joins.
//   * Dequantization stays in registers and costs one shift and one v_bitop3_b32 per pair of codes: the
//     nibble pair (j, j + 4) of a packed word is moved to bits [3, 7) of each 16-bit half and merged with
//     the bf16 pattern of 16.0, giving the exact value 16 + u (the bf16 mantissa step at 16 is 1/8, so the
//     nibble sits in the top four mantissa bits). For two's-complement codes the same instruction flips the
//     nibble's sign bit, turning q into its offset binary q + 8.
//   * The products use v_dot2_f32_bf16 (two bf16 products, fp32 accumulation). The code offset is removed
//     once per 32 codes: sum x (u - off) = sum x (16 + u) - (16 + off) sum x, with off = 8 (symmetric)
//     or z (asymmetric), then the group scale multiplies the 32-code partial sum. The fp32 sums run at
//     about (16 + off) sum |x|: with the value 128 + u (nibble at bits [0, 4), which saves the shift of the
//     first pair) they ran at (128 + off) sum |x|, and on groups whose codes sit near the zero point with a
//     wide range (a few outliers 100 x the rest) the fp32 output was off by up to 3.7e-5 normwise against
//     the binary64 result; the 16 + u form cancels about 6 x less.
//   * No dequantized weight is ever written to memory.
//
// The matrix-core variant below keeps ordinary (allocating) weight loads: with non-temporal ones it ran
// slower and left dirty lines in the last-level cache that slowed the kernels after it.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// A loop-invariant constant held in a VGPR. gfx9 VOP3 instructions take no literal and at most one scalar
// operand, so the three-input bit operation below needs its mask and magic in vector registers.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c)
{
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

// the 16 + u form (nibbles at bits [3, 7)), used by every kernel below
constexpr uint32_t kPairMask = 0x00780078u;
constexpr uint32_t kMagic16 = 0x41804180u;      // bf16 16.0 | 16.0
constexpr uint32_t kSignFlip = 0x00400040u;     // bit 6 of each half: the nibble's top bit
constexpr uint32_t kBf16OnePair = 0x3F803F80u;  // bf16 1.0 | 1.0
constexpr int kMaxWavesPerRow = 8;

__device__ __forceinline__ uint32_t pair_bits(uint32_t shifted, uint32_t mask, uint32_t magic)
{
    return __builtin_amdgcn_bitop3_b32(shifted, mask, magic, 0x6A);  // (a & b) ^ c
}

// Everything one lane loads for one 32-code chunk: R rows of packed codes, their scales and zero
// points, and MT rows of activations.
template <int MT, int R>
struct Stage {
    uint4 w[R];
    float s[R];
    float z[R];
    uint4 x[MT][4];
};

// Uniform (per block) base pointers of the R weight rows, their metadata and the MT activation rows. With
// 16-bit metadata s points at binary16 scales, z at the packed zero points and zr is the row's first group.
template <int MT, int R>
struct Bases {
    const uint8_t *w[R];
    const void *s[R];
    const uint8_t *z[R];
    int64_t zr[R];
    const uint16_t *x[MT];
};

template <int MT, int R, int G, bool SYM, bool M16>
__device__ __forceinline__ void stage_load(Stage<MT, R> &st, const Bases<MT, R> &b, uint32_t c)
{
    constexpr int kGroupShift = (G == 128) ? 2 : (G == 64) ? 1 : 0;  // chunk -> group index
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(b.w[r] + c * 16u));
        st.w[r] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const uint32_t gi = c >> kGroupShift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (M16) {
            st.s[r] = (float)static_cast<const _Float16 *>(b.s[r])[gi];
            const int64_t e = b.zr[r] + gi;
            st.z[r] = SYM ? 8.0f : (float)((b.z[r][e >> 1] >> (4 * (e & 1))) & 0xFu);
        } else {
            st.s[r] = static_cast<const float *>(b.s[r])[gi];
            st.z[r] = SYM ? 8.0f : (float)b.z[r][gi];
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint4 *xv = reinterpret_cast<const uint4 *>(b.x[m] + c * 32u);
#pragma unroll
        for (int d = 0; d < 4; ++d)
            st.x[m][d] = xv[d];
    }
}

template <int MT, int R>
__device__ __forceinline__ void stage_compute(const Stage<MT, R> &st, float acc[R][MT], uint32_t mask, uint32_t magic)
{
    // activations re-paired as (x_j, x_{j+4}) per 8-element block, and their sum
    uint32_t xp[MT][16];
    float xsum[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4 u = st.x[m][d];
            xp[m][4 * d + 0] = __builtin_amdgcn_perm(u.z, u.x, 0x05040100u);
            xp[m][4 * d + 1] = __builtin_amdgcn_perm(u.z, u.x, 0x07060302u);
            xp[m][4 * d + 2] = __builtin_amdgcn_perm(u.w, u.y, 0x05040100u);
            xp[m][4 * d + 3] = __builtin_amdgcn_perm(u.w, u.y, 0x07060302u);
            s = dot2(u.x, kBf16OnePair, s);
            s = dot2(u.y, kBf16OnePair, s);
            s = dot2(u.z, kBf16OnePair, s);
            s = dot2(u.w, kBf16OnePair, s);
        }
        xsum[m] = s;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t wd[4] = {st.w[r].x, st.w[r].y, st.w[r].z, st.w[r].w};
        float part[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            part[m] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t b0 = pair_bits(wd[d] << 3, mask, magic);
            const uint32_t b1 = pair_bits(wd[d] >> 1, mask, magic);
            const uint32_t b2 = pair_bits(wd[d] >> 5, mask, magic);
            const uint32_t b3 = pair_bits(wd[d] >> 9, mask, magic);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                part[m] = dot2(xp[m][4 * d + 0], b0, part[m]);
                part[m] = dot2(xp[m][4 * d + 1], b1, part[m]);
                part[m] = dot2(xp[m][4 * d + 2], b2, part[m]);
                part[m] = dot2(xp[m][4 * d + 3], b3, part[m]);
            }
        }
        // sum_k x (u - off) = sum_k x (16 + u) - (16 + off) sum_k x, then the group scale
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = __builtin_fmaf(st.s[r], __builtin_fmaf(-(16.0f + st.z[r]), xsum[m], part[m]), acc[r][m]);
    }
}

// One row block (rows rb * R .. rb * R + R - 1) of the decode product: MT activation rows (1..4), R weight rows,
// group size G; S = blockDim.x / 64 waves split K. `red` is the block's LDS for combining the S partial sums.
template <int MT, int R, int G, bool SYM, bool OUT_BF16, bool M16>
__device__ __forceinline__ void gemv_rowblock(const uint16_t *__restrict__ x, int64_t N, int64_t K,
                                              const uint8_t *__restrict__ w, const void *__restrict__ scales,
                                              const uint8_t *__restrict__ zeros, void *__restrict__ y, int64_t y_ld,
                                              int64_t rb, float (*red)[R * MT])
{
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar loop bounds
    const int S = blockDim.x / kWave;
    const int64_t row0 = rb * R;
    const int chunks = (int)(K / 32);  // 32 codes = 16 bytes per lane
    const int s_shift = __builtin_ctz(S);  // S is a power of two
    const int c_begin = (chunks * wv) >> s_shift;
    const int c_end = (chunks * (wv + 1)) >> s_shift;
    const int c_last = c_end - 1;
    const uint32_t mask = vreg_const(kPairMask);
    const uint32_t magic = vreg_const(SYM ? (kMagic16 ^ kSignFlip) : kMagic16);

    Bases<MT, R> bp;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r < N ? row0 + r : N - 1;  // rows past N read row N-1, never stored
        bp.w[r] = w + row * (K / 2);
        if (M16) {
            bp.s[r] = static_cast<const uint16_t *>(scales) + row * (K / G);
            bp.z[r] = zeros;
            bp.zr[r] = row * (K / G);
        } else {
            bp.s[r] = static_cast<const float *>(scales) + row * (K / G);
            bp.z[r] = SYM ? nullptr : zeros + row * (K / G);
            bp.zr[r] = 0;
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
        bp.x[m] = x + (int64_t)m * K;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;

    // two register stages: the loads of iteration it + 1 are in flight while iteration it is reduced
    const int iters = (c_end - c_begin + kWave - 1) / kWave;  // uniform
    Stage<MT, R> st[2];
    auto step = [&](int h, int it) {
        const int cn = c_begin + lane + kWave * (it + 1);
        stage_load<MT, R, G, SYM, M16>(st[h ^ 1], bp, (uint32_t)(cn < c_last ? cn : c_last));
        __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of this chunk's math
        const bool ok = c_begin + lane + kWave * it < c_end;
#pragma unroll
        for (int r = 0; r < R; ++r)
            st[h].s[r] = ok ? st[h].s[r] : 0.0f;
        stage_compute<MT, R>(st[h], acc, mask, magic);
        __builtin_amdgcn_sched_barrier(0);
    };
    {
        const int c = c_begin + lane;
        stage_load<MT, R, G, SYM, M16>(st[0], bp, (uint32_t)(c < c_last ? c : c_last));
    }
    int it = 0;
    for (; it + 2 <= iters; it += 2) {
        step(0, it);
        step(1, it + 1);
    }
    if (it < iters)  // odd trip count: one more chunk, in stage 0
        step(0, it);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = wave_sum_uniform(acc[r][m]);

    float *yf = reinterpret_cast<float *>(y);
    uint16_t *yh = reinterpret_cast<uint16_t *>(y);
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
                    yh[m * y_ld + row0 + r] = (uint16_t)f32_to_bf16_bits(t);
                else
                    yf[m * y_ld + row0 + r] = t;
            }
        }
    } else if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (row0 + r < N) {
                    if (OUT_BF16)
                        yh[m * y_ld + row0 + r] = (uint16_t)f32_to_bf16_bits(acc[r][m]);
                    else
                        yf[m * y_ld + row0 + r] = acc[r][m];
                }
    }
}

// MT activation rows (1..4), R weight rows per block, group size G; S = blockDim.x / 64 waves split K.
template <int MT, int R, int G, bool SYM, bool OUT_BF16, bool M16 = false>
__global__ __launch_bounds__(512) void k_w4a16_gemv(const uint16_t *__restrict__ x, int64_t N, int64_t K,
                                                    const uint8_t *__restrict__ w, const void *__restrict__ scales,
                                                    const uint8_t *__restrict__ zeros, void *__restrict__ y,
                                                    int64_t y_ld)
{
    __shared__ float red[kMaxWavesPerRow][R * MT];
    gemv_rowblock<MT, R, G, SYM, OUT_BF16, M16>(x, N, K, w, scales, zeros, y, y_ld, blockIdx.x, red);
}

// Several independent products in one launch: the grid is the concatenation of the problems' row blocks
// (problem p owns blocks [begin[p], begin[p + 1])); a block finds its problem with a uniform scan of the
// table, which lives in the kernel arguments.
template <int MT, int R, int G, bool SYM, bool OUT_BF16, bool M16 = false>
__global__ __launch_bounds__(512) void k_w4a16_gemv_grouped(const GroupedW4A16 table)
{
    __shared__ float red[kMaxWavesPerRow][R * MT];
    const int64_t b = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroupedProblems; ++i)
        p += (i < table.count && b >= table.begin[i]) ? 1 : 0;
    const GroupedW4A16::Problem &q = table.p[p];
    gemv_rowblock<MT, R, G, SYM, OUT_BF16, M16>(q.x, q.N, q.K, q.w, M16 ? q.scales16 : (const void *)q.scales, q.zeros,
                                               q.y, q.N, b - table.begin[p], red);
}

// ------------------------------------------------------------------ matrix-core variant (M >= 5 not taken by the
// staged kernel below: g = 32 / 64, or M > 32; up to 64 tokens per launch)
//
// v_mfma_f32_16x16x32_bf16 computes D[i][j] += sum_k A[i][k] B[k][j] on 16x32 / 32x16 bf16 tiles. Here
// A is the activation tile (i = token m) and B the dequantized weight tile (j = output row n), so lane
// l holds B for row n = l % 16 and k-block l / 16, and D for row n at tokens m = 4 (l / 16) + r: each lane
// owns one weight row, whose scale and zero point it loads itself.
//   * k-step = 128 codes. With g = 128 a lane loads 16 bytes (its quarter of the k-step) and word t feeds
//     MFMA t; all four MFMAs stay inside the one group. With g = 32 / 64 a lane loads the word of k-block
//     t for each MFMA t, so that each MFMA covers 32 consecutive codes of a single group.
//   * Weight words become B operands with the same nibble-pair dequantization as the vector kernel
//     (element 2j + h of the operand is code j + 4h of the word, value 16 + u); the activations are
//     re-paired to match with v_perm.
//   * Per group, one more MFMA against a B of ones gives sum_k x[m, k] for the lane's tokens; then
//     acc += s * (D - (16 + off) * xsum). Tokens past M reuse row M - 1 and are never stored.
//   * TT row tiles of 16 share each activation operand; MTILES tiles of 16 tokens share each weight
//     operand, so the weight stream is read once for up to 64 tokens. S waves of a block split K and are
//     combined through LDS in a fixed order.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// B operand (8 weights, value 16 + u each) from one packed word.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t wd, uint32_t mask, uint32_t magic)
{
    return as_bf16x8(pair_bits(wd << 3, mask, magic), pair_bits(wd >> 1, mask, magic), pair_bits(wd >> 5, mask, magic),
                     pair_bits(wd >> 9, mask, magic));
}

// A operand from 8 consecutive activations, re-paired as (x_j, x_{j+4}).
__device__ __forceinline__ bf16x8_t pair_x(uint4 u)
{
    return as_bf16x8(__builtin_amdgcn_perm(u.z, u.x, 0x05040100u), __builtin_amdgcn_perm(u.z, u.x, 0x07060302u),
                     __builtin_amdgcn_perm(u.w, u.y, 0x05040100u), __builtin_amdgcn_perm(u.w, u.y, 0x07060302u));
}

constexpr int kMfmaMaxWaves = 4;

template <int MTILES, int TT, int G>
struct MStage {
    static constexpr int GPS = G == 128 ? 1 : 128 / G;  // groups per k-step
    uint32_t w[TT][4];
    float s[TT][GPS];
    float z[TT][GPS];
    uint4 x[MTILES][4];
};

template <int MTILES, int TT, int G, bool SYM>
__device__ __forceinline__ void mstage_load(MStage<MTILES, TT, G> &st, const uint8_t *const wrow[TT],
                                            const float *const srow[TT], const uint8_t *const zrow[TT],
                                            const uint16_t *const xrow[MTILES], int kbase, int K, int kb)
{
    constexpr bool WIDE = (G == 128);
    constexpr int GPS = MStage<MTILES, TT, G>::GPS;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        if (WIDE) {
            const uint4 v = *reinterpret_cast<const uint4 *>(wrow[tt] + (kbase / 2 + 16 * kb));
            st.w[tt][0] = v.x;
            st.w[tt][1] = v.y;
            st.w[tt][2] = v.z;
            st.w[tt][3] = v.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                st.w[tt][t] = (kbase + 32 * t < K)
                                  ? *reinterpret_cast<const uint32_t *>(wrow[tt] + (kbase / 2 + 16 * t + 4 * kb))
                                  : 0u;
        }
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
            const int gi = (kbase + g * (128 / GPS)) / G;
            const bool ok = kbase + g * (128 / GPS) < K;
            st.s[tt][g] = ok ? srow[tt][gi] : 0.0f;
            st.z[tt][g] = SYM ? 8.0f : (ok ? (float)zrow[tt][gi] : 0.0f);
        }
    }
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = WIDE ? kbase + 32 * kb + 8 * t : kbase + 32 * t + 8 * kb;
            st.x[mt][t] = (k < K) ? *reinterpret_cast<const uint4 *>(xrow[mt] + k) : make_uint4(0, 0, 0, 0);
        }
}

template <int MTILES, int TT, int G>
__device__ __forceinline__ void mstage_compute(const MStage<MTILES, TT, G> &st, f32x4_t acc[TT][MTILES], uint32_t mask,
                                               uint32_t magic)
{
    constexpr int GPS = MStage<MTILES, TT, G>::GPS;
    constexpr int TPG = 4 / GPS;  // k-blocks (MFMAs) per group
    const bf16x8_t ones = as_bf16x8(kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair);
    bf16x8_t a[MTILES][4];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            a[mt][t] = pair_x(st.x[mt][t]);
    bf16x8_t b[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            b[tt][t] = dequant_word(st.w[tt][t], mask, magic);
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
        f32x4_t xs[MTILES];
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            xs[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = g * TPG; t < (g + 1) * TPG; ++t)
                xs[mt] = mfma_bf16(a[mt][t], ones, xs[mt]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const float cf = -(16.0f + st.z[tt][g]);
            const float sc = st.s[tt][g];
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) {
                f32x4_t d = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = g * TPG; t < (g + 1) * TPG; ++t)
                    d = mfma_bf16(a[mt][t], b[tt][t], d);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[tt][mt][r] = __builtin_fmaf(sc, __builtin_fmaf(cf, xs[mt][r], d[r]), acc[tt][mt][r]);
            }
        }
    }
}

template <int MTILES, int TT, int G, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_w4a16_mfma(const uint16_t *__restrict__ x, int64_t M, int64_t N, int64_t K,
                                                    const uint8_t *__restrict__ w, const float *__restrict__ scales,
                                                    const uint8_t *__restrict__ zeros, void *__restrict__ y)
{
    __shared__ float red[kMfmaMaxWaves - 1][TT * MTILES * 4][kWave];
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int S = blockDim.x / kWave;
    const int nl = lane % 16, kb = lane / 16;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * TT;
    const int ksteps = (int)((K + 127) / 128);
    const int ks_begin = ksteps * wv / S, ks_end = ksteps * (wv + 1) / S;
    const uint32_t mask = vreg_const(kPairMask);
    const uint32_t magic = vreg_const(SYM ? (kMagic16 ^ kSignFlip) : kMagic16);

    const uint8_t *wrow[TT];
    const float *srow[TT];
    const uint8_t *zrow[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t n = std::min<int64_t>(n0 + 16 * tt + nl, N - 1);
        wrow[tt] = w + n * (K / 2);
        srow[tt] = scales + n * (K / G);
        zrow[tt] = SYM ? nullptr : zeros + n * (K / G);
    }
    const uint16_t *xrow[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
        xrow[mt] = x + std::min<int64_t>(mt * 16 + nl, M - 1) * K;

    f32x4_t acc[TT][MTILES];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
            acc[tt][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    MStage<MTILES, TT, G> sa, sb;
    int ks = ks_begin;
    if (ks < ks_end)
        mstage_load<MTILES, TT, G, SYM>(sa, wrow, srow, zrow, xrow, ks * 128, (int)K, kb);
    while (ks < ks_end) {
        if (ks + 1 < ks_end)
            mstage_load<MTILES, TT, G, SYM>(sb, wrow, srow, zrow, xrow, (ks + 1) * 128, (int)K, kb);
        mstage_compute<MTILES, TT, G>(sa, acc, mask, magic);
        if (ks + 1 >= ks_end)
            break;
        if (ks + 2 < ks_end)
            mstage_load<MTILES, TT, G, SYM>(sa, wrow, srow, zrow, xrow, (ks + 2) * 128, (int)K, kb);
        mstage_compute<MTILES, TT, G>(sb, acc, mask, magic);
        ks += 2;
    }

    // combine the S K-slices in wave order, then store: lane holds rows n = n0 + 16 tt + nl at tokens
    // m = 16 mt + 4 kb + r
    if (S > 1) {
        if (wv > 0) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[wv - 1][(tt * MTILES + mt) * 4 + r][lane] = acc[tt][mt][r];
        }
        __syncthreads();
        if (wv > 0)
            return;
        for (int i = 1; i < S; ++i)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[tt][mt][r] += red[i - 1][(tt * MTILES + mt) * 4 + r][lane];
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t n = n0 + 16 * tt + nl;
        if (n >= N)
            continue;
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = mt * 16 + 4 * kb + r;
                if (m < M) {
                    if (OUT_BF16)
                        reinterpret_cast<uint16_t *>(y)[m * N + n] = (uint16_t)f32_to_bf16_bits(acc[tt][mt][r]);
                    else
                        reinterpret_cast<float *>(y)[m * N + n] = acc[tt][mt][r];
                }
            }
    }
}

// ------------------------------------------------------------------ matrix-core variant, M <= 32 per launch
//
// v_mfma_f32_32x32x16_bf16 (32 tokens x 32 rows x 16 codes; twice the rate of the 16x16x32 form on
// gfx950). Lane l holds A (activations) for token l % 32 and B (dequantized weights) for row l % 32, codes
// 8 (l / 32) .. + 8 of the 16; D holds row l % 32 at tokens 8 (r / 4) + 4 (l / 32) + r % 4.
//   * Loading operands straight into that layout makes every lane of a group of four read a different row
//     (or token), i.e. four cache lines per quad; the L1 then saturates on tag lookups long before HBM
//     does. So each wave stages 128 codes of its 32 rows (and the activations) at a time through a private
//     LDS region: its global loads read whole 64-byte row pieces (one line per quad), are written to LDS
//     with an XOR swizzle (no bank conflicts), and read back in operand order. LDS operations of one wave
//     execute in order, so no barrier is needed.
//   * g = 128: lane h of MFMA t works on codes 64 h + 8 t .. + 8 of the step. g = 32 / 64: every MFMA must
//     stay inside one group, so lane h of MFMA t takes codes 16 t + 8 h .. + 8; the even and odd 4-byte
//     words of each row go to separate halves of its LDS row, which lets each lane read its words with the
//     same two 16-byte reads.
//   * The activations are re-paired as (x_j, x_{j+4}) once, when they are written to LDS, to match the
//     nibble-pair dequantization.
//   * acc += s * (D - (16 + off) * xsum) per group, where xsum = sum_k x over the group for the lane's tokens.
//     Up to 8 tokens, xsum comes from the VALU: when a lane stages its 8 activations it adds them with dot2
//     against ones, a DPP butterfly over the lanes of its group finishes each token's sum, and the sums go
//     to LDS beside the activations. For more tokens one more MFMA against a B of ones computes it (the
//     VALU sums would then cost more issue slots than the MFMA).
//   * Only the accumulator registers that hold staged tokens are folded, reduced and stored (4 for up to
//     8 tokens, 8 for up to 16).
//   * Scales (and zero points) of four groups come with one load; they go through a buffer resource, so the
//     read past the last row's groups returns zero instead of touching memory.
//   * The next step's global loads are issued right after the current step's LDS stores, so they are in
//     flight during its MFMAs. S waves of a block split K and are combined through LDS (fixed order).
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_bf16_32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kStageMaxWaves = 8;
constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format, no swizzle

// LDS of one wave: 32 rows x 64 B of codes, 4 XI tokens x 256 B, and up to 8 tokens the GPS x 4 XI group sums
// of x.
template <int XI, int G>
constexpr int stage_region_bytes()
{
    return 2048 + XI * 1024 + (XI <= 2 ? (128 / G) * 4 * XI * 4 : 0);
}

// One row block (rows 32 rb .. 32 rb + 31) of the staged product: XI activation load instructions of 4 tokens
// each (M <= 4 XI); group size G in {32, 64, 128}; K % 128 == 0. `lds` holds kStageMaxWaves regions.
template <int XI, int G, bool SYM, bool OUT_BF16>
__device__ __forceinline__ void staged_rowblock(const uint16_t *__restrict__ x, int64_t M, int64_t N, int64_t K,
                                                const uint8_t *__restrict__ w, const float *__restrict__ scales,
                                                const uint8_t *__restrict__ zeros, void *__restrict__ y,
                                                int64_t rb, uint8_t *__restrict__ lds)
{
    constexpr int GPS = 128 / G;   // groups per 128-code step
    constexpr int TPG = 8 / GPS;   // MFMAs per group
    constexpr int SPM = 4 / GPS;   // steps per metadata load (four groups)
    constexpr int kTokens = 4 * XI;
    constexpr bool XV = XI <= 2;                // group sums of x on the VALU (else by MFMA)
    constexpr int NR = XI >= 8 ? 16 : 2 * XI;   // accumulator registers that hold staged tokens
    constexpr int kRegion = stage_region_bytes<XI, G>();
    static_assert(kRegion == 2048 + XI * 1024 + (XV ? GPS * kTokens * 4 : 0), "region layout");
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = blockDim.x / kWave;
    const int col = lane % 32, h = lane / 32;
    const int64_t n0 = rb * 32;
    const int steps = (int)(K / 128);
    const int groups = (int)(K / G);
    const int s_begin = steps * wv / S, s_end = steps * (wv + 1) / S;
    const int ns = s_end - s_begin;
    const int s_last = s_end > s_begin ? s_end - 1 : s_begin;
    const uint32_t mask = vreg_const(kPairMask);
    const uint32_t magic = vreg_const(SYM ? (kMagic16 ^ kSignFlip) : kMagic16);
    const bf16x8_t ones = as_bf16x8(kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair);
    uint8_t *const wl = lds + wv * kRegion;  // [32 rows][4 chunks of 16 B], chunk ^= (row / 4) % 4
    uint8_t *const xl = wl + 2048;           // [kTokens][16 pieces of 16 B], piece ^= token % 16
    float *const xsl = reinterpret_cast<float *>(xl + XI * 1024);  // [GPS][kTokens] (XV)

    // global -> LDS: weight instruction I covers rows 16 I + lane / 4 (piece lane % 4), activation
    // instruction I tokens 4 I + lane / 16 (piece lane % 16); tokens past M repeat token M - 1.
    // g = 128: piece e goes to chunk e. g < 128: its even words (2 of 4) to the row's first half, chunk
    // e / 2 + byte 8 (e % 2), its odd words to the same place in the second half.
    const uint8_t *wsrc[2];
    int wdst[2][2];
#pragma unroll
    for (int I = 0; I < 2; ++I) {
        const int r = 16 * I + lane / 4, e = lane % 4, swz = (r >> 2) & 3;
        wsrc[I] = w + std::min<int64_t>(n0 + r, N - 1) * (K / 2) + 16 * e;
        if (G == 128) {
            wdst[I][0] = r * 64 + 16 * (e ^ swz);
            wdst[I][1] = 0;
        } else {
            wdst[I][0] = r * 64 + 16 * ((e >> 1) ^ swz) + 8 * (e & 1);
            wdst[I][1] = r * 64 + 16 * ((2 + (e >> 1)) ^ swz) + 8 * (e & 1);
        }
    }
    const uint16_t *xsrc[XI];
    int xdst[XI];
#pragma unroll
    for (int I = 0; I < XI; ++I) {
        const int t = 4 * I + lane / 16, p = lane % 16;
        xsrc[I] = x + std::min<int64_t>(t, M - 1) * K + 8 * p;
        xdst[I] = t * 256 + 16 * (p ^ (t & 15));
    }
    // LDS -> operands: B lane (j, h) reads chunks 2h, 2h+1 of row j; A lane (i, h) of MFMA t reads piece
    // 8h + t (g = 128) or 2t + h (g < 128) of token i (tokens past the staged ones alias staged rows; their
    // outputs are never stored)
    int brd[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        brd[q] = col * 64 + 16 * ((2 * h + q) ^ ((col >> 2) & 3));
    const int ti = col & (kTokens - 1);
    const int64_t row = std::min<int64_t>(n0 + col, N - 1);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void *)scales, (short)0, (int)(N * groups * 4), kRawBufferWord3);
    const uint32_t soff = (uint32_t)(row * groups * 4);
    const uint32_t ztotal = SYM ? 0u : (uint32_t)(N * groups);  // zero-point bytes (>= 4 when asymmetric)
    const __amdgpu_buffer_rsrc_t zrs =  // unused (null, empty) when symmetric
        __builtin_amdgcn_make_buffer_rsrc((void *)zeros, (short)0, (int)ztotal, kRawBufferWord3);
    const uint32_t zoff = (uint32_t)(row * groups);

    u32x4_t wr[2], xr[XI];  // vector types, so that their LDS stores stay plain vector stores
    auto gload = [&](int i) __attribute__((always_inline)) {
        const int st = min(s_begin + i, s_last);
#pragma unroll
        for (int I = 0; I < 2; ++I)
            wr[I] = *reinterpret_cast<const u32x4_t *>(wsrc[I] + st * 64);
#pragma unroll
        for (int I = 0; I < XI; ++I)
            xr[I] = *reinterpret_cast<const u32x4_t *>(xsrc[I] + st * 128);
    };
    // metadata of the four groups that start with step s_begin + i: scales, and zero points as the four
    // bytes of one word
    struct Meta {
        u32x4_t s;
        uint32_t z;
    };
    auto mload = [&](Meta &md, int i) __attribute__((always_inline)) {
        const uint32_t g0 = (uint32_t)((s_begin + i) * GPS);
        md.s = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(srs, soff + 4 * g0, 0, 0));
        if (!SYM) {
            // a dword that crosses the end of the buffer reads as 0 as a whole, so the 4-byte window is
            // clamped to end inside the array (it holds at least 4 bytes) and shifted down afterwards
            const uint32_t zb = zoff + g0;
            const uint32_t zc = min(zb, ztotal - 4u);
            // (zb - zc <= 3 for every group a step uses; the prefetch past the slice may go further)
            md.z = __builtin_amdgcn_raw_buffer_load_b32(zrs, zc, 0, 0) >> (8u * min(zb - zc, 3u));
        }
    };

    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.0f;

    auto step = [&](int i, const Meta &md, int sj) __attribute__((always_inline)) {
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            if (G == 128) {
                *reinterpret_cast<u32x4_t *>(wl + wdst[I][0]) = wr[I];
            } else {
                *reinterpret_cast<uint2 *>(wl + wdst[I][0]) = make_uint2(wr[I].x, wr[I].z);
                *reinterpret_cast<uint2 *>(wl + wdst[I][1]) = make_uint2(wr[I].y, wr[I].w);
            }
        }
#pragma unroll
        for (int I = 0; I < XI; ++I) {
            const u32x4_t v = xr[I];
            *reinterpret_cast<u32x4_t *>(xl + xdst[I]) =
                u32x4_t{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                        __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
            if (XV) {
                // the lane's 8 activations, then the G / 8 lanes of its group (one token's 128 codes fill a
                // 16-lane row): quads, half rows, the whole row
                float sx = dot2(v.x, kBf16OnePair,
                                dot2(v.y, kBf16OnePair, dot2(v.z, kBf16OnePair, dot2(v.w, kBf16OnePair, 0.0f))));
                sx += dpp_f32<0xB1>(sx);
                sx += dpp_f32<0x4E>(sx);
                if (G >= 64)
                    sx += dpp_f32<0x141>(sx);
                if (G >= 128)
                    sx += dpp_f32<0x140>(sx);
                const int p = lane % 16, t = 4 * I + lane / 16;
                if (p % (G / 8) == 0)
                    xsl[(p / (G / 8)) * kTokens + t] = sx;
            }
        }
        gload(i + 1);  // the LDS stores above have read these registers
        __builtin_amdgcn_sched_barrier(0);
        uint4 b[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            b[q] = *reinterpret_cast<const uint4 *>(wl + brd[q]);
#pragma unroll
        for (int gq = 0; gq < GPS; ++gq) {
            f32x16_t xs, d;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                xs[r] = 0.0f;
                d[r] = 0.0f;
            }
            if (XV) {  // the sums of the lane's tokens 4 h .. 4 h + 3 (and 8 + 4 h .. with NR = 8)
#pragma unroll
                for (int q = 0; q < NR / 4; ++q) {
                    const float4 f = *reinterpret_cast<const float4 *>(xsl + gq * kTokens + 8 * q + 4 * h);
                    xs[4 * q] = f.x;
                    xs[4 * q + 1] = f.y;
                    xs[4 * q + 2] = f.z;
                    xs[4 * q + 3] = f.w;
                }
            }
#pragma unroll
            for (int t = gq * TPG; t < (gq + 1) * TPG; ++t) {
                const int piece = (G == 128) ? 8 * h + t : 2 * t + h;
                const bf16x8_t a = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(xl + ti * 256 + 16 * (piece ^ (ti & 15))));
                if (!XV)
                    xs = mfma_bf16_32(a, ones, xs);
                const uint4 wq = b[t / 4];
                const uint32_t wd = (t % 4 == 0) ? wq.x : (t % 4 == 1) ? wq.y : (t % 4 == 2) ? wq.z : wq.w;
                const bf16x8_t bw = dequant_word(wd, mask, magic);
                d = mfma_bf16_32(a, bw, d);
            }
            // the element goes through a scalar first: a bit_cast of a vector-element expression reads
            // element 0 with this compiler
            const int mi = sj * GPS + gq;  // group within the metadata word
            const uint32_t sbits = md.s[mi];
            const float sc = __uint_as_float(sbits);
            const float off = SYM ? 8.0f : (float)((md.z >> (8 * mi)) & 0xFFu);
            const float cf = -(16.0f + off);
#pragma unroll
            for (int r = 0; r < NR; ++r)
                acc[r] = __builtin_fmaf(sc, __builtin_fmaf(cf, xs[r], d[r]), acc[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    Meta cur, nxt;
    gload(0);
    mload(cur, 0);
    int i = 0;
    for (; i + SPM <= ns; i += SPM) {
        mload(nxt, i + SPM);
#pragma unroll
        for (int sj = 0; sj < SPM; ++sj)
            step(i + sj, cur, sj);
        cur = nxt;
    }
#pragma unroll
    for (int sj = 0; sj + 1 < SPM; ++sj)
        if (i + sj < ns)
            step(i + sj, cur, sj);

    // combine the S K-slices: halving tree over the staging area, fixed order
    float *red = reinterpret_cast<float *>(lds);  // [S / 2][16][64]
    for (int half = S / 2; half >= 1; half /= 2) {
        __syncthreads();
        if (wv >= half && wv < 2 * half)
#pragma unroll
            for (int r = 0; r < NR; ++r)
                red[((wv - half) * 16 + r) * kWave + lane] = acc[r];
        __syncthreads();
        if (wv < half)
#pragma unroll
            for (int r = 0; r < NR; ++r)
                acc[r] += red[(wv * 16 + r) * kWave + lane];
    }
    if (wv > 0)
        return;
    const int64_t n = n0 + col;
    if (n >= N)
        return;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t m = 8 * (r / 4) + 4 * h + r % 4;
        if (m < M) {
            if (OUT_BF16)
                reinterpret_cast<uint16_t *>(y)[m * N + n] = (uint16_t)f32_to_bf16_bits(acc[r]);
            else
                reinterpret_cast<float *>(y)[m * N + n] = acc[r];
        }
    }
}

template <int XI, int G, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(64 * kStageMaxWaves) void k_w4a16_mfma_lds(
    const uint16_t *__restrict__ x, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ w,
    const float *__restrict__ scales, const uint8_t *__restrict__ zeros, void *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStageMaxWaves * stage_region_bytes<XI, G>()];
    staged_rowblock<XI, G, SYM, OUT_BF16>(x, M, N, K, w, scales, zeros, y, blockIdx.x, lds);
}

// Several independent staged products with M tokens each in one launch: problem p owns row blocks
// [begin[p], begin[p + 1]) of the grid and a block finds its problem with a uniform scan of the table.
template <int XI, int G, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(64 * kStageMaxWaves) void k_w4a16_mfma_lds_grouped(const GroupedW4A16 table, int64_t M)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStageMaxWaves * stage_region_bytes<XI, G>()];
    const int64_t b = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroupedProblems; ++i)
        p += (i < table.count && b >= table.begin[i]) ? 1 : 0;
    const GroupedW4A16::Problem &q = table.p[p];
    staged_rowblock<XI, G, SYM, OUT_BF16>(q.x, M, q.N, q.K, q.w, q.scales, q.zeros, q.y, b - table.begin[p], lds);
}

// ------------------------------------------------------------------ shared activation tile, 17-32 tokens
//
// The staged kernel gives each wave its own K slice, so at 32 tokens every wave stages 8 KB of activations per
// 2 KB of weights. Here a block of 8 waves is R row waves (32 rows each) x S = 8 / R K groups: the R waves of a
// K group walk the same 128-code steps and share one activation tile per step, each loading 8 / R of its
// 8 instructions. The tile (with the per-token sums of the step, on the VALU as in the staged kernel at up to
// 8 tokens) is double-buffered in LDS with one block barrier per step; each wave stages its own 32 weight rows
// as in the staged kernel. g = 128, symmetric codes (one scale per row and step), K % 128 == 0. All K groups
// run the same number of steps (the longest slice); steps past a group's slice re-read its last step with a
// zero scale. Measured on the 70B projections at M = 32: q|k|v 28.1 us against 31.5 for the staged kernel,
// gate|up 89 against 97-100, the 28672-row gate 50.6 against 57; on 8192-row layers it loses (o 27.6 against
// 21.1), so it takes layers of more than 8192 rows.
template <int R, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_w4a16_mfma_shared(const uint16_t *__restrict__ x, int64_t M, int64_t N,
                                                           int64_t K, const uint8_t *__restrict__ w,
                                                           const float *__restrict__ scales, void *__restrict__ y)
{
    constexpr int XI = 8;                      // activation instructions of 4 tokens per step
    constexpr int S = 8 / R;                   // K groups
    constexpr int kTokens = 4 * XI;
    constexpr int NR = 16;                     // accumulator registers (32 tokens)
    constexpr int XL = XI / R;                 // activation load instructions per wave
    static_assert(XI % R == 0, "the row waves split the activation instructions");
    constexpr int kXB = XI * 1024 + kTokens * 4;  // one activation buffer: tile + per-token sums
    __shared__ __attribute__((aligned(16))) uint8_t wls[8 * 2048];
    __shared__ __attribute__((aligned(16))) uint8_t xls[S * 2 * kXB];
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rw = wv % R, kg = wv / R;
    const int col = lane % 32, h = lane / 32;
    const int64_t n0 = (int64_t)blockIdx.x * 32 * R + 32 * rw;
    const int steps = (int)(K / 128);
    const int nsmax = (steps + S - 1) / S;
    const int s_begin = steps * kg / S, s_end = steps * (kg + 1) / S;
    const int s_last = s_end > s_begin ? s_end - 1 : s_begin;  // s_begin < steps for every group
    const uint32_t mask = vreg_const(kPairMask);
    const uint32_t magic = vreg_const(kMagic16 ^ kSignFlip);
    uint8_t *const wl = wls + wv * 2048;
    uint8_t *const xb0 = xls + kg * 2 * kXB;

    // weights: instruction I covers rows 16 I + lane / 4, piece lane % 4 (chunk ^= (row / 4) % 4 in LDS)
    const uint8_t *wsrc[2];
    int wdst[2];
#pragma unroll
    for (int I = 0; I < 2; ++I) {
        const int r = 16 * I + lane / 4, e = lane % 4, swz = (r >> 2) & 3;
        wsrc[I] = w + std::min<int64_t>(n0 + r, N - 1) * (K / 2) + 16 * e;
        wdst[I] = r * 64 + 16 * (e ^ swz);
    }
    // activations: this wave's instructions J = rw XL + I cover tokens 4 J + lane / 16, piece lane % 16
    // (piece ^= token % 16 in LDS); tokens past M repeat token M - 1
    const uint16_t *xsrc[XL];
    int xdst[XL], xtok[XL];
#pragma unroll
    for (int I = 0; I < XL; ++I) {
        const int J = rw * XL + I;
        const int t = 4 * J + lane / 16, p = lane % 16;
        xsrc[I] = x + std::min<int64_t>(t, M - 1) * K + 8 * p;
        xdst[I] = t * 256 + 16 * (p ^ (t & 15));
        xtok[I] = t;
    }
    int brd[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        brd[q] = col * 64 + 16 * ((2 * h + q) ^ ((col >> 2) & 3));
    const float *ssrc = scales + std::min<int64_t>(n0 + col, N - 1) * steps;

    u32x4_t wr[2], xr[XL];
    float sr;
    auto wload = [&](int i) __attribute__((always_inline)) {
        const int st = min(s_begin + i, s_last);
#pragma unroll
        for (int I = 0; I < 2; ++I)
            wr[I] = *reinterpret_cast<const u32x4_t *>(wsrc[I] + st * 64);
        sr = (s_begin + i < s_end) ? ssrc[st] : 0.0f;  // steps past the slice add nothing
    };
    auto xload = [&](int i) __attribute__((always_inline)) {
        const int st = min(s_begin + i, s_last);
#pragma unroll
        for (int I = 0; I < XL; ++I)
            xr[I] = *reinterpret_cast<const u32x4_t *>(xsrc[I] + st * 128);
    };
    // activations re-paired as (x_j, x_{j+4}) into buffer buf, and each token's sum over the step (dot2 against
    // ones, then the 16 lanes of the token added by a DPP butterfly)
    auto xstore = [&](int buf) __attribute__((always_inline)) {
        uint8_t *const xl = xb0 + buf * kXB;
        float *const xsl = reinterpret_cast<float *>(xl + XI * 1024);
#pragma unroll
        for (int I = 0; I < XL; ++I) {
            const u32x4_t v = xr[I];
            *reinterpret_cast<u32x4_t *>(xl + xdst[I]) =
                u32x4_t{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                        __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
            float sx = dot2(v.x, kBf16OnePair, dot2(v.y, kBf16OnePair, dot2(v.z, kBf16OnePair,
                                                                             dot2(v.w, kBf16OnePair, 0.0f))));
            sx += dpp_f32<0xB1>(sx);   // quad: lanes 1 apart
            sx += dpp_f32<0x4E>(sx);   // quad: lanes 2 apart
            sx += dpp_f32<0x141>(sx);  // half-row mirror: the other quad of the 8
            sx += dpp_f32<0x140>(sx);  // row mirror: the other 8 of the 16
            if (lane % 16 == 0)
                xsl[xtok[I]] = sx;
        }
    };

    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        acc[r] = 0.0f;

    // step 0's activations into buffer 0, step 1's in registers, step 0's weights in registers
    xload(0);
    xstore(0);
    xload(1);
    wload(0);
    __syncthreads();
    for (int i = 0; i < nsmax; ++i) {
        const int cb = i & 1;
#pragma unroll
        for (int I = 0; I < 2; ++I)
            *reinterpret_cast<u32x4_t *>(wl + wdst[I]) = wr[I];
        const float sc = sr;
        wload(i + 1);
        xstore(cb ^ 1);  // step i + 1's activations into the other buffer
        xload(i + 2);
        uint8_t *const xl = xb0 + cb * kXB;
        const float *xsl = reinterpret_cast<const float *>(xl + XI * 1024);
        uint4 b[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            b[q] = *reinterpret_cast<const uint4 *>(wl + brd[q]);
        f32x16_t xs, d;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            xs[r] = 0.0f;
            d[r] = 0.0f;
        }
#pragma unroll
        for (int q = 0; q < NR / 4; ++q) {
            const float4 f = *reinterpret_cast<const float4 *>(xsl + 8 * q + 4 * h);
            xs[4 * q] = f.x;
            xs[4 * q + 1] = f.y;
            xs[4 * q + 2] = f.z;
            xs[4 * q + 3] = f.w;
        }
        // MFMA t: lane h holds codes 64 h + 8 t .. + 8 of the step for token (A) and row (B) col
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int piece = 8 * h + t;
            const bf16x8_t a = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4 *>(xl + col * 256 + 16 * (piece ^ (col & 15))));
            const uint4 wq = b[t / 4];
            const uint32_t wd = (t % 4 == 0) ? wq.x : (t % 4 == 1) ? wq.y : (t % 4 == 2) ? wq.z : wq.w;
            const bf16x8_t bw = dequant_word(wd, mask, magic);
            d = mfma_bf16_32(a, bw, d);
        }
        // sum_k x (u - 8) = sum_k x (16 + u) - 24 sum_k x, then the row's scale for this step
#pragma unroll
        for (int r = 0; r < NR; ++r)
            acc[r] = __builtin_fmaf(sc, __builtin_fmaf(-24.0f, xs[r], d[r]), acc[r]);
        __syncthreads();  // buffer cb is free for step i + 2; step i + 1's activations are visible
    }

    // K groups 1 .. S - 1 park their sums over the activation buffers, group 0 adds them in group order
    float *red = reinterpret_cast<float *>(xls);  // [S - 1][R][NR][64]
    static_assert((S - 1) * R * NR * kWave * 4 <= S * 2 * kXB, "partials fit");
    if (kg > 0)
#pragma unroll
        for (int r = 0; r < NR; ++r)
            red[(((kg - 1) * R + rw) * NR + r) * kWave + lane] = acc[r];
    __syncthreads();
    if (kg > 0)
        return;
    for (int g = 1; g < S; ++g)
#pragma unroll
        for (int r = 0; r < NR; ++r)
            acc[r] += red[(((g - 1) * R + rw) * NR + r) * kWave + lane];
    const int64_t n = n0 + col;
    if (n >= N)
        return;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t m = 8 * (r / 4) + 4 * h + r % 4;
        if (m < M) {
            if (OUT_BF16)
                reinterpret_cast<uint16_t *>(y)[m * N + n] = (uint16_t)f32_to_bf16_bits(acc[r]);
            else
                reinterpret_cast<float *>(y)[m * N + n] = acc[r];
        }
    }
}

namespace {

// Waves per block: split K until the grid holds about `target_waves` waves, keeping at least one full
// 2048-code iteration per wave.
inline int waves_per_row_block(int64_t rowblocks, int64_t K, int64_t target_waves)
{
    const int64_t chunks = K / 32;
    int S = 1;
    while (S < kMaxWavesPerRow && rowblocks * S < target_waves && chunks / (2 * S) >= kWave)
        S *= 2;
    return S;
}

template <int MT, int R, int G, bool SYM>
hipError_t gemv_launch(const W4A16Args &a, const uint16_t *x, void *y, hipStream_t st)
{
    const int64_t rowblocks = (a.N + R - 1) / R;
    const int S = waves_per_row_block(rowblocks, a.K, 4096);
    const dim3 grid((unsigned)rowblocks), block(kWave * S);
    if (a.meta16) {
        if (a.y_bf16)
            k_w4a16_gemv<MT, R, G, SYM, true, true><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales16, a.zeros, y,
                                                                           a.N);
        else
            k_w4a16_gemv<MT, R, G, SYM, false, true><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales16, a.zeros, y,
                                                                            a.N);
    } else if (a.y_bf16)
        k_w4a16_gemv<MT, R, G, SYM, true><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales, a.zeros, y, a.N);
    else
        k_w4a16_gemv<MT, R, G, SYM, false><<<grid, block, 0, st>>>(x, a.N, a.K, a.w, a.scales, a.zeros, y, a.N);
    return hipGetLastError();
}

template <int G, bool SYM>
hipError_t gemv_mt(const W4A16Args &a, int mt, const uint16_t *x, void *y, hipStream_t st)
{
    switch (mt) {
    case 1:
        return gemv_launch<1, 4, G, SYM>(a, x, y, st);
    case 2:
        return gemv_launch<2, 4, G, SYM>(a, x, y, st);
    case 3:
        return gemv_launch<3, 2, G, SYM>(a, x, y, st);
    default:
        return gemv_launch<4, 2, G, SYM>(a, x, y, st);
    }
}

// Matrix-core launch for up to 16 * MTILES tokens.
template <int MTILES, int TT, int G, bool SYM>
hipError_t mfma_launch(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    const int64_t blocks = (a.N + 16 * TT - 1) / (16 * TT);
    const int64_t ksteps = (a.K + 127) / 128;
    int S = 1;
    while (S < kMfmaMaxWaves && blocks * S < 4096 && ksteps / (2 * S) >= 4)
        S *= 2;
    const dim3 grid((unsigned)blocks), block(kWave * S);
    if (a.y_bf16)
        k_w4a16_mfma<MTILES, TT, G, SYM, true><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, a.zeros, y);
    else
        k_w4a16_mfma<MTILES, TT, G, SYM, false><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, a.zeros, y);
    return hipGetLastError();
}

// Staged matrix-core launch (M <= 4 XI tokens at x, output rows at y): 32 rows per block, S waves per block
// splitting K. A block of 8 waves fills a CU's register file (at 32 tokens) or most of it, so while the row
// blocks fit the CUs once, S = 8; beyond that S = 4, so that two blocks share a CU instead of the grid running
// a second, partial round; up to 8 tokens on layers of at least 768 row blocks S = 2 (longer K slices; the
// block's LDS is sized for 8 waves, so four such blocks share a CU). Every wave keeps at least two 128-code
// steps. Measured on the 70B projections
// (g = 128): the q|k|v launch (320 blocks) 21.7 us at S = 4 against 24.8 at 8, the 28672-row gate at M = 8
// 37.5 us at S = 2 against 43.0 at 4, the 57344-row gate|up at M = 16 80.3 us at S = 4 against 88.7 at 2.
constexpr int64_t kRowBlocksPerRound = 256;  // one 32-row block of 8 waves per CU

template <int XI, int G, bool SYM>
hipError_t lds_launch(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    const int64_t blocks = (a.N + 31) / 32;
    const int64_t steps = a.K / 128;
    int S = blocks <= kRowBlocksPerRound ? 8 : (XI == 2 && blocks >= 3 * kRowBlocksPerRound) ? 2 : 4;
    while (S > 1 && steps / S < 2)
        S /= 2;
    const dim3 grid((unsigned)blocks), block(kWave * S);
    if (a.y_bf16)
        k_w4a16_mfma_lds<XI, G, SYM, true><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, a.zeros, y);
    else
        k_w4a16_mfma_lds<XI, G, SYM, false><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, a.zeros, y);
    return hipGetLastError();
}

// Shared-activation launch (17-32 tokens): R row waves per block, the smallest of 2, 4, 8 that leaves at most
// 256 blocks (on the 70B layers: q|k|v 10240 rows at R = 2 28 us against 45 at R = 4; the 28672-row gate at
// R = 4 50.6 us against 55.6 at R = 2; gate|up at R = 4 or 8 89-90 us against 100 at R = 2).
template <int R>
hipError_t shared_launch(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    const dim3 grid((unsigned)((a.N + 32 * R - 1) / (32 * R))), block(kWave * 8);
    if (a.y_bf16)
        k_w4a16_mfma_shared<R, true><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, y);
    else
        k_w4a16_mfma_shared<R, false><<<grid, block, 0, st>>>(x, M, a.N, a.K, a.w, a.scales, y);
    return hipGetLastError();
}

// Layers of more than 8192 rows with at least two 128-code steps per K group of the shared kernel.
inline bool shared_fits(const W4A16Args &a, int64_t M)
{
    return M > 16 && M <= 32 && a.N > 32 * kRowBlocksPerRound && a.K / 128 >= 8;
}

template <int G, bool SYM>
hipError_t lds_mg(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    if (M <= 8)
        return lds_launch<2, G, SYM>(a, x, M, y, st);
    if (M <= 16)
        return lds_launch<4, G, SYM>(a, x, M, y, st);
    if (G == 128 && SYM && shared_fits(a, M)) {
        if (a.N <= 64 * kRowBlocksPerRound)
            return shared_launch<2>(a, x, M, y, st);
        if (a.N <= 128 * kRowBlocksPerRound)
            return shared_launch<4>(a, x, M, y, st);
        return shared_launch<8>(a, x, M, y, st);
    }
    return lds_launch<8, G, SYM>(a, x, M, y, st);
}

// Up to 32 tokens per launch.
template <bool SYM>
hipError_t lds_m(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return lds_mg<32, SYM>(a, x, M, y, st);
    case 64:
        return lds_mg<64, SYM>(a, x, M, y, st);
    default:
        return lds_mg<128, SYM>(a, x, M, y, st);
    }
}

template <int G, bool SYM>
hipError_t mfma_m(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    if (M <= 16)
        return mfma_launch<1, 2, G, SYM>(a, x, M, y, st);
    if (M <= 32)
        return mfma_launch<2, 2, G, SYM>(a, x, M, y, st);
    return mfma_launch<4, 2, G, SYM>(a, x, M, y, st);
}

template <bool SYM>
hipError_t mfma_g(const W4A16Args &a, const uint16_t *x, int64_t M, void *y, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return mfma_m<32, SYM>(a, x, M, y, st);
    case 64:
        return mfma_m<64, SYM>(a, x, M, y, st);
    default:
        return mfma_m<128, SYM>(a, x, M, y, st);
    }
}

template <bool SYM>
hipError_t gemv_g(const W4A16Args &a, int mt, const uint16_t *x, void *y, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return gemv_mt<32, SYM>(a, mt, x, y, st);
    case 64:
        return gemv_mt<64, SYM>(a, mt, x, y, st);
    default:
        return gemv_mt<128, SYM>(a, mt, x, y, st);
    }
}

}  // namespace

// Tokens at or above which the matrix-core kernels replace the vector kernel.
constexpr int64_t kMfmaMinTokens = 5;
// Up to this many tokens the staged kernel runs (in launches of 32 tokens, each re-reading the weights).
constexpr int64_t kStagedMaxTokens = 64;

namespace {

template <int MT, int R, int G, bool SYM>
hipError_t grouped_launch(const W4A16GroupedArgs &a, hipStream_t st)
{
    // problems with the most K first: their blocks run longest, so they are dispatched first
    int order[kMaxGroupedProblems];
    int n = 0;
    for (int i = 0; i < a.count; ++i)
        if (a.problems[i].N > 0)
            order[n++] = i;
    std::stable_sort(order, order + n, [&](int u, int v) { return a.problems[u].K > a.problems[v].K; });
    if (n == 0)
        return hipSuccess;
    GroupedW4A16 t = {};
    int64_t total = 0, kmin = a.problems[order[0]].K;
    for (int j = 0; j < n; ++j) {
        const W4A16Args &q = a.problems[order[j]];
        t.p[j] = {q.x, q.w, q.scales, nullptr, q.zeros, q.y, q.N, q.K};
        t.begin[j] = total;
        total += (q.N + R - 1) / R;
        kmin = std::min(kmin, q.K);
    }
    t.begin[n] = total;
    for (int j = n + 1; j <= kMaxGroupedProblems; ++j)
        t.begin[j] = total;
    t.count = n;
    const int S = waves_per_row_block(total, kmin, 4096);
    const dim3 grid((unsigned)total), block(kWave * S);
    if (a.y_bf16)
        k_w4a16_gemv_grouped<MT, R, G, SYM, true><<<grid, block, 0, st>>>(t);
    else
        k_w4a16_gemv_grouped<MT, R, G, SYM, false><<<grid, block, 0, st>>>(t);
    return hipGetLastError();
}

template <int G, bool SYM>
hipError_t grouped_mt(const W4A16GroupedArgs &a, hipStream_t st)
{
    switch (a.M) {
    case 1:
        return grouped_launch<1, 4, G, SYM>(a, st);
    case 2:
        return grouped_launch<2, 4, G, SYM>(a, st);
    case 3:
        return grouped_launch<3, 2, G, SYM>(a, st);
    default:
        return grouped_launch<4, 2, G, SYM>(a, st);
    }
}

template <bool SYM>
hipError_t grouped_g(const W4A16GroupedArgs &a, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return grouped_mt<32, SYM>(a, st);
    case 64:
        return grouped_mt<64, SYM>(a, st);
    default:
        return grouped_mt<128, SYM>(a, st);
    }
}

}  // namespace

namespace {

// The staged kernel works in 128-code steps and addresses scales through 32-bit buffer offsets (and, with zero
// points, reads them four bytes at a time from an array of at least four).
bool staged_fits(const W4A16Args &a)
{
    const int64_t groups = a.K / a.group_size;
    return a.K % 128 == 0 && a.N * groups * 4 < ((int64_t)1 << 31) && (a.symmetric || a.N * groups >= 4);
}

// Several staged products (5-32 tokens) in one launch: the problems' 32-row blocks as one grid (most K first),
// S waves per block from the whole grid and the shortest K.
template <int XI, int G, bool SYM>
hipError_t grouped_staged_launch(const W4A16GroupedArgs &a, hipStream_t st)
{
    int order[kMaxGroupedProblems];
    int n = 0;
    for (int i = 0; i < a.count; ++i)
        if (a.problems[i].N > 0)
            order[n++] = i;
    std::stable_sort(order, order + n, [&](int u, int v) { return a.problems[u].K > a.problems[v].K; });
    if (n == 0)
        return hipSuccess;
    GroupedW4A16 t = {};
    int64_t total = 0, kmin = a.problems[order[0]].K;
    for (int j = 0; j < n; ++j) {
        const W4A16Args &q = a.problems[order[j]];
        t.p[j] = {q.x, q.w, q.scales, nullptr, q.zeros, q.y, q.N, q.K};
        t.begin[j] = total;
        total += (q.N + 31) / 32;
        kmin = std::min(kmin, q.K);
    }
    for (int j = n; j <= kMaxGroupedProblems; ++j)
        t.begin[j] = total;
    t.count = n;
    // 8 waves while the blocks fit the CUs once, else 4 (the single launch's 2 for wide layers at up to 8 tokens
    // is slower here: the 70B layer's four products at M = 8 take 136 us with 2, 120 us with 4, 127 us with 8)
    int S = total <= kRowBlocksPerRound ? 8 : 4;
    while (S > 1 && (kmin / 128) / S < 2)
        S /= 2;
    const dim3 grid((unsigned)total), block(kWave * S);
    if (a.y_bf16)
        k_w4a16_mfma_lds_grouped<XI, G, SYM, true><<<grid, block, 0, st>>>(t, a.M);
    else
        k_w4a16_mfma_lds_grouped<XI, G, SYM, false><<<grid, block, 0, st>>>(t, a.M);
    return hipGetLastError();
}

template <int XI, bool SYM>
hipError_t grouped_staged_g(const W4A16GroupedArgs &a, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return grouped_staged_launch<XI, 32, SYM>(a, st);
    case 64:
        return grouped_staged_launch<XI, 64, SYM>(a, st);
    default:
        return grouped_staged_launch<XI, 128, SYM>(a, st);
    }
}

}  // namespace

hipError_t launch_w4a16_grouped(const W4A16GroupedArgs &a, hipStream_t st)
{
    if (a.M < 1 || a.count < 1 || a.count > kMaxGroupedProblems)
        return hipErrorInvalidValue;
    if (a.M <= 4)
        return a.symmetric ? grouped_g<true>(a, st) : grouped_g<false>(a, st);
    // 5-32 tokens: one staged launch when every problem fits the staged kernel (on the 70B layer, one launch over
    // q|k|v, o, gate|up and down streams 3.5-3.7 TB/s at M = 8 against 3.3 in four launches, and 2.47 at M = 32
    // against 2.29 with the shared-activation kernel on the wide products); otherwise, and above 32 tokens, each
    // problem as its own product
    bool staged = a.M <= 32;
    for (int i = 0; i < a.count; ++i)
        staged = staged && (a.problems[i].N == 0 || staged_fits(a.problems[i]));
    if (staged) {
        if (a.M <= 8)
            return a.symmetric ? grouped_staged_g<2, true>(a, st) : grouped_staged_g<2, false>(a, st);
        if (a.M <= 16)
            return a.symmetric ? grouped_staged_g<4, true>(a, st) : grouped_staged_g<4, false>(a, st);
        return a.symmetric ? grouped_staged_g<8, true>(a, st) : grouped_staged_g<8, false>(a, st);
    }
    for (int i = 0; i < a.count; ++i)
        if (a.problems[i].N > 0)
            if (hipError_t e = launch_w4a16(a.problems[i], st))
                return e;
    return hipSuccess;
}

hipError_t launch_w4a16(const W4A16Args &a, hipStream_t st)
{
    const size_t ysz = a.y_bf16 ? 2 : 4;
    if (a.meta16 && a.M >= kMfmaMinTokens)
        return hipErrorInvalidValue;  // 16-bit metadata: the vector (decode) kernel only
    if (a.M >= kMfmaMinTokens && a.M <= kStagedMaxTokens && staged_fits(a)) {
        for (int64_t m0 = 0; m0 < a.M; m0 += 32) {
            const int64_t mc = std::min<int64_t>(32, a.M - m0);
            const uint16_t *x = a.x + m0 * a.K;
            void *y = static_cast<char *>(a.y) + (size_t)m0 * (size_t)a.N * ysz;
            hipError_t e = a.symmetric ? lds_m<true>(a, x, mc, y, st) : lds_m<false>(a, x, mc, y, st);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    if (a.M >= kMfmaMinTokens) {
        for (int64_t m0 = 0; m0 < a.M; m0 += 64) {
            const int64_t mc = std::min<int64_t>(64, a.M - m0);
            const uint16_t *x = a.x + m0 * a.K;
            void *y = static_cast<char *>(a.y) + (size_t)m0 * (size_t)a.N * ysz;
            hipError_t e = a.symmetric ? mfma_g<true>(a, x, mc, y, st) : mfma_g<false>(a, x, mc, y, st);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    for (int64_t m0 = 0; m0 < a.M; m0 += 4) {
        const int mt = (int)std::min<int64_t>(4, a.M - m0);
        const uint16_t *x = a.x + m0 * a.K;
        void *y = static_cast<char *>(a.y) + (size_t)m0 * (size_t)a.N * ysz;
        hipError_t e = a.symmetric ? gemv_g<true>(a, mt, x, y, st) : gemv_g<false>(a, mt, x, y, st);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace pqg
