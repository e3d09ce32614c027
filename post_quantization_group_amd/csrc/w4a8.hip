// w4a8.hip -- INT4 per-group weights x INT8 per-token activations on gfx950 int8 matrix cores.
//
// y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] * (q_w[n, k] - z[n, g])
// ("第11章 模型量化与压缩" §11.4.5 and §11.10.2: W4A8 is the INT4 group weights of weight-only quantization
// stacked on the INT8 per-token activations of SmoothQuant; the two are independent, so each keeps its own
// scales: one per weight group, one per token. The integer sums run per group, exactly; the group scales
// then weight them in fp32.)
//
// Operands. v_mfma_i32_32x32x32_i8 with the activation tile as A (rows = tokens) and the weight tile as B
// (columns = output channels): lane l holds output channel n = l % 32 and, in register r, token
// m = 8 (r / 4) + 4 (l / 32) + r % 4. A lane therefore needs one weight scale and one zero point per group
// and tile, whatever r.
//   * Weight codes are staged packed (two per byte) and unpacked when read: 8 bytes (16 codes) of row n give
//     one B operand. Per 4-byte word (8 codes): the low and the high nibbles are masked into bytes, biased by
//     0x80 (and, for two's-complement codes, their sign bit flipped, which turns q into q + 8), put back in
//     code order with v_perm, and the zero point (8 for symmetric codes) is subtracted from all four bytes
//     at once: each byte is >= 0x80 > z, so no borrow crosses a byte. Removing the bias leaves the signed
//     byte q - z in [-15, 15].
//   * Which codes one MFMA sums is free as long as A and B agree; what matters is that every MFMA lies inside
//     one group. A step's 128 codes are taken as two pairs of 64 codes, each pair as two MFMAs. For g = 64
//     and 128 a pair lies inside one group, and lane half h takes the pair's codes 32 h .. 32 h + 31 (one
//     16-byte read of packed codes, 16 codes per MFMA). For g = 32 each MFMA must be one group of 32
//     consecutive codes, so lane half h takes its codes 16 h .. 16 h + 15 (an 8-byte read per MFMA). The
//     int32 accumulator of a group is started from zero, and after the group's last MFMA it is added into
//     fp32 accumulators with its scale s_w[n, g].
// Tiling: 128 (m) x 128 (n) block tile, four waves of 64 x 64 (2 x 2 MFMA tiles; 128 x 64 and 64 x 32 for
// g = 32 and 64), K steps of 128 codes
// (activation rows 128 bytes, weight rows 64 bytes), two LDS stages filled from registers while the other
// is multiplied, as in the register-staged INT8 kernel. XCD-aware tile order as there.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kW8Xcds = 8;
constexpr int kBM = 128, kWM = 64, kBK = 128;  // kBK in codes
constexpr int kThreads = 256;
constexpr int kXRow = kBK, kWRow = kBK / 2;    // bytes per staged row
constexpr int kXLoads = kBM * kXRow / 16 / kThreads;  // 4
static_assert(kXLoads * 16 * kThreads == kBM * kXRow, "whole loads");

// Output channels per wave: 64 (two MFMA tiles) for g = 128, 32 for g = 32 and 64, whose per-step group
// metadata and more frequent folds would otherwise not fit the 256 registers of two waves per SIMD.
template <int G>
struct W4A8Tile {
    static constexpr int WN = G == 128 ? 64 : 32, BN = 2 * WN;
    static constexpr int WLOADS = BN * kWRow / 16 / kThreads;
    static_assert(WLOADS * 16 * kThreads == BN * kWRow, "whole loads");
};

// LDS offset of 16-byte piece c of a staged row r: rows of 128 bytes (activations) and 64 bytes (packed
// weights). The piece index is xor-ed with row bits so that the 16 rows read together by one half of a
// wave fall into different bank quads.
__device__ __forceinline__ int xoff(int r, int c) { return r * kXRow + 16 * (c ^ (((r >> 1) & 3) | ((r >> 2) & 4))); }
__device__ __forceinline__ int woff(int r, int c) { return r * kWRow + 16 * (c ^ (((r >> 2) & 1) | ((r >> 3) & 2))); }

// One B operand (16 signed codes q - z) from 8 bytes of packed codes, with the zero point z replicated in zz.
__device__ __forceinline__ v4i unpack8(uint32_t w0, uint32_t w1, uint32_t mask, uint32_t bias, uint32_t zz)
{
    const uint32_t w[2] = {w0, w1};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t ev = __builtin_amdgcn_bitop3_b32(w[i], mask, bias, 0x6A);       // codes 0,2,4,6: (a & b) ^ c
        const uint32_t od = __builtin_amdgcn_bitop3_b32(w[i] >> 4, mask, bias, 0x6A);  // codes 1,3,5,7
        // back in code order (bytes c0 c1 c2 c3 and c4 c5 c6 c7), then minus z in every byte, bias removed
        o[2 * i] = (__builtin_amdgcn_perm(od, ev, 0x05010400u) - zz) ^ 0x80808080u;
        o[2 * i + 1] = (__builtin_amdgcn_perm(od, ev, 0x07030602u) - zz) ^ 0x80808080u;
    }
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

// A loop-invariant constant in a VGPR (v_bitop3_b32 takes no literal).
__device__ __forceinline__ uint32_t vconst(uint32_t c)
{
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

template <int G, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void k_w4a8(const int8_t *__restrict__ xq, const float *__restrict__ sx,
                                                     int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ wp,
                                                     const float *__restrict__ sw, const uint8_t *__restrict__ zw,
                                                     void *__restrict__ y, int tiles)
{
    constexpr int kWN = W4A8Tile<G>::WN, kBN = W4A8Tile<G>::BN, kWLoads = W4A8Tile<G>::WLOADS;
    constexpr int TM = kWM / 32, TN = kWN / 32;
    constexpr int DPG = G / 32;   // MFMA depths per group (1, 2 or 4: a divisor of the 4 depths of a step)
    constexpr int GPS = kBK / G;  // groups per step
    __shared__ __attribute__((aligned(16))) int8_t sX[2][kBM * kXRow];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kBN * kWRow];

    const int per = (tiles + kW8Xcds - 1) / kW8Xcds;  // XCD x takes tiles [x per, (x + 1) per)
    const int t = (int)(blockIdx.x % kW8Xcds) * per + (int)(blockIdx.x / kW8Xcds);
    if (t >= tiles)
        return;
    const int m_tiles = (int)((M + kBM - 1) / kBM);
    const int64_t n0 = (int64_t)(t / m_tiles) * kBN;
    const int64_t m0 = (int64_t)(t % m_tiles) * kBM;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = w % (kBM / kWM), wn = w / (kBM / kWM);
    const int col = lane % 32, h = lane / 32;
    const int64_t groups = K / G;

    // global -> register -> LDS: piece p = tid + 256 i -> staged row p / pieces-per-row, piece p % that.
    // 32-bit offsets from the tile's first rows (a [128, K] activation slice and a [BN, K / 2] weight slice).
    const int8_t *xbase = xq + m0 * K;
    const uint8_t *wbase = wp + n0 * (K / 2);
    uint32_t xoffs[kXLoads], woffs[kWLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int p = tid + kThreads * i;
        xoffs[i] = (uint32_t)(std::min<int64_t>(p / 8, M - 1 - m0) * K + 16 * (p % 8));
    }
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
        const int p = tid + kThreads * i;
        woffs[i] = (uint32_t)(std::min<int64_t>(p / 4, N - 1 - n0) * (K / 2) + 16 * (p % 4));
    }
    // staging registers as clang vectors: arrays of HIP's uint4 struct stayed in scratch memory here
    v4i rx[kXLoads], rw[kWLoads];
    auto load = [&](int step) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            rx[i] = *reinterpret_cast<const v4i *>(xbase + (xoffs[i] + (uint32_t)step * kBK));
#pragma unroll
        for (int i = 0; i < kWLoads; ++i)
            rw[i] = *reinterpret_cast<const v4i *>(wbase + (woffs[i] + (uint32_t)step * (kBK / 2)));
    };
    auto store = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int p = tid + kThreads * i;
            *reinterpret_cast<v4i *>(&sX[st][xoff(p / 8, p % 8)]) = rx[i];
        }
#pragma unroll
        for (int i = 0; i < kWLoads; ++i) {
            const int p = tid + kThreads * i;
            *reinterpret_cast<v4i *>(&sW[st][woff(p / 4, p % 4)]) = rw[i];
        }
    };

    // per-lane weight rows of the TN tiles (clamped: rows past N are computed, never stored)
    int64_t nrow[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i)
        nrow[i] = std::min<int64_t>(n0 + wn * kWN + i * 32 + col, N - 1);
    // scales and replicated zero points of the step's GPS groups, loaded one step ahead like the tiles
    struct Meta {
        float s[TN][GPS];
        uint32_t zz[TN][GPS];
    };
    auto load_meta = [&](Meta &md, int step) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const int64_t idx = nrow[i] * groups + (int64_t)step * GPS + gi;
                md.s[i][gi] = sw[idx];
                md.zz[i][gi] = (SYM ? 8u : (uint32_t)zw[idx]) * 0x01010101u;
            }
    };

    const uint32_t mask = vconst(0x0F0F0F0Fu);
    const uint32_t bias = vconst(SYM ? 0x88888888u : 0x80808080u);
    v16i acc[TN][TM];
    float facc[TN][TM][16];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                acc[i][j][e] = 0;
                facc[i][j][e] = 0.0f;
            }
    // add a finished group (index gi within the step) into the fp32 accumulators, restart the integer ones
    auto fold = [&](const Meta &md, int gi) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const float sc = md.s[i][gi];
#pragma unroll
            for (int j = 0; j < TM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    facc[i][j][e] = __builtin_fmaf(sc, (float)acc[i][j][e], facc[i][j][e]);
                    acc[i][j][e] = 0;
                }
        }
    };

    const int nsteps = (int)(K / kBK);
    Meta mcur, mnxt;
    load(0);
    load_meta(mcur, 0);
    store(0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps) {
            load(step + 1);
            load_meta(mnxt, step + 1);
        }
        // two pairs of MFMA depths per step; pair q covers codes 64 q .. 64 q + 63 of the step
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            v4i fb[TN][2];
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int row = wn * kWN + i * 32 + col;
                if constexpr (G == 32) {
                    // MFMA e is group 2 q + e: packed piece 2 q + e, its half h
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const uint2 pc = *reinterpret_cast<const uint2 *>(&sW[cur][woff(row, 2 * q + e) + 8 * h]);
                        fb[i][e] = unpack8(pc.x, pc.y, mask, bias, mcur.zz[i][2 * q + e]);
                    }
                } else {
                    // the pair is inside group (2 q) / DPG: packed piece 2 q + h, MFMA e its half e
                    const uint4 pc = *reinterpret_cast<const uint4 *>(&sW[cur][woff(row, 2 * q + h)]);
                    const uint32_t zz = mcur.zz[i][(2 * q) / DPG];
                    fb[i][0] = unpack8(pc.x, pc.y, mask, bias, zz);
                    fb[i][1] = unpack8(pc.z, pc.w, mask, bias, zz);
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                // the activation piece holding the same 16 codes as fb[.][e]
                const int xp = G == 32 ? 4 * q + 2 * e + h : 4 * q + 2 * h + e;
                v4i fa[TM];
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    fa[j] = *reinterpret_cast<const v4i *>(&sX[cur][xoff(wm * kWM + j * 32 + col, xp)]);
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[j], fb[i][e], acc[i][j], 0, 0, 0);
                // depth 2 q + e of the step ends its group when (2 q + e + 1) % DPG == 0 (DPG divides 4)
                if ((2 * q + e + 1) % DPG == 0)
                    fold(mcur, (2 * q + e) / DPG);
            }
        }
        if (step + 1 < nsteps) {
            store(cur ^ 1);
            mcur = mnxt;
        }
        __syncthreads();
    }

    // epilogue: token scale and store; lane holds channel n, registers r the tokens 8 (r / 4) + 4 h + r % 4.
    // For one r the 32 lanes of a half write 32 consecutive channels of one output row.
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int64_t n = n0 + wn * kWN + i * 32 + col;
        if (n >= N)
            continue;
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * kWM + j * 32 + 8 * (r / 4) + 4 * h + r % 4;
                if (m < M) {
                    const float v = facc[i][j][r] * sx[m];
                    if (OUT_BF16)
                        reinterpret_cast<uint16_t *>(y)[m * N + n] = (uint16_t)f32_to_bf16_bits(v);
                    else
                        reinterpret_cast<float *>(y)[m * N + n] = v;
                }
            }
    }
}

template <int G, bool SYM>
hipError_t w4a8_go(const W4A8Args &a, hipStream_t st)
{
    constexpr int kBN = W4A8Tile<G>::BN;
    const int64_t tiles = ((a.N + kBN - 1) / kBN) * ((a.M + kBM - 1) / kBM);
    const int64_t per = (tiles + kW8Xcds - 1) / kW8Xcds;
    const dim3 grid((unsigned)(per * kW8Xcds)), block(kThreads);
    if (a.y_bf16)
        k_w4a8<G, SYM, true><<<grid, block, 0, st>>>(a.x_q, a.x_scales, a.M, a.N, a.K, a.w, a.w_scales, a.w_zeros,
                                                     a.y, (int)tiles);
    else
        k_w4a8<G, SYM, false><<<grid, block, 0, st>>>(a.x_q, a.x_scales, a.M, a.N, a.K, a.w, a.w_scales, a.w_zeros,
                                                      a.y, (int)tiles);
    return hipGetLastError();
}

template <bool SYM>
hipError_t w4a8_sym(const W4A8Args &a, hipStream_t st)
{
    switch (a.group_size) {
    case 32:
        return w4a8_go<32, SYM>(a, st);
    case 64:
        return w4a8_go<64, SYM>(a, st);
    default:
        return w4a8_go<128, SYM>(a, st);
    }
}

}  // namespace

hipError_t launch_w4a8(const W4A8Args &a, hipStream_t st)
{
    return a.symmetric ? w4a8_sym<true>(a, st) : w4a8_sym<false>(a, st);
}

}  // namespace pqg
