// gemm_i8.hip -- INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, with the W8A8 epilogue.
//
// acc[m, n] = sum_k a[m, k] * b[n, k]  (exact integer accumulation), then optionally
// y[m, n] = float(acc) * (s_x[m] * s_w[n])   ("第11章 模型量化与压缩" §11.4.5 step 6: INT8 GEMM, INT32
// accumulation, dequantized output; "模型压缩：量化、ZeroQuant、LLM.int8() 与 SmoothQuant" §11: one scale per
// row of the left operand and one per column of the right operand).
//
// Tiling. v_mfma_i32_16x16x64_i8 multiplies a 16x64 by a 64x16 int8 tile. The weight tile is fed as the
// MFMA "A" operand and the activation tile as "B", so the 16x16 result lands with each lane holding four
// consecutive output channels n of one token m: the epilogue writes 16 bytes (int32) or 8 bytes (bf16)
// per lane, contiguous along the output row.
//   block: 256 threads = 4 waves in a 2 (n) x 2 (m) arrangement; block tile 128 (n) x 128 (m), K step 64
//   wave : 64 (n) x 64 (m) = 4 x 4 MFMA tiles, 16 int32 accumulators of 4 registers
//   LDS  : two stages of [128][64 + 16 pad] bytes for each operand; global -> register -> LDS staging with
//          the next K step's loads in flight while the current one is multiplied.
// Both operands are read from LDS with one 16-byte read per lane per 16x64 fragment: lane l takes row
// l % 16 and bytes [16 (l / 16), 16 (l / 16) + 16) of the 64-byte K slice. A and B use the same
// lane-to-k assignment, so the products pair up whatever k order the instruction uses internally.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBN = 128;           // output channels per block (MFMA A side)
constexpr int kBM = 128;           // tokens per block (MFMA B side)
constexpr int kBK = 64;            // K bytes per step
constexpr int kLdsStride = kBK + 16;  // padded row stride (bytes)

template <int MODE>  // 0: raw int32, 1: bf16 epilogue, 2: fp32 epilogue
__global__ __launch_bounds__(256) void k_gemm_i8(const int8_t *__restrict__ a, const int8_t *__restrict__ b,
                                                 int64_t M, int64_t N, int64_t K, const float *__restrict__ sa,
                                                 const float *__restrict__ sb, void *__restrict__ c)
{
    __shared__ __attribute__((aligned(16))) int8_t sW[2][kBN * kLdsStride];
    __shared__ __attribute__((aligned(16))) int8_t sX[2][kBM * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int wn = wv % 2, wm = wv / 2;
    const int64_t n_tiles = (N + kBN - 1) / kBN;
    const int64_t n0 = (int64_t)(blockIdx.x % n_tiles) * kBN;
    const int64_t m0 = (int64_t)(blockIdx.x / n_tiles) * kBM;

    // global -> LDS assignment: each operand tile is 128 rows x 4 pieces of 16 bytes = 512 pieces,
    // two per thread: piece p = tid + 256 i -> row p / 4, piece p % 4.
    int ldr[2], ldp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i;
        ldr[i] = p / 4;
        ldp[i] = p % 4;
    }
    auto load_tiles = [&](int64_t k0, uint4 rw[2], uint4 rx[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t kk = k0 + ldp[i] * 16;
            const int64_t nr = n0 + ldr[i], mr = m0 + ldr[i];
            rw[i] = (nr < N && kk < K) ? *reinterpret_cast<const uint4 *>(b + nr * K + kk) : make_uint4(0, 0, 0, 0);
            rx[i] = (mr < M && kk < K) ? *reinterpret_cast<const uint4 *>(a + mr * K + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tiles = [&](int st, const uint4 rw[2], const uint4 rx[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<uint4 *>(&sW[st][ldr[i] * kLdsStride + ldp[i] * 16]) = rw[i];
            *reinterpret_cast<uint4 *>(&sX[st][ldr[i] * kLdsStride + ldp[i] * 16]) = rx[i];
        }
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};

    uint4 rw[2], rx[2];
    load_tiles(0, rw, rx);
    store_tiles(0, rw, rx);
    __syncthreads();

    const int frow = lane % 16;
    const int fcol = (lane / 16) * 16;
    const int nsteps = (int)((K + kBK - 1) / kBK);
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps)
            load_tiles((int64_t)(step + 1) * kBK, rw, rx);
        v4i fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fa[i] = *reinterpret_cast<const v4i *>(&sW[cur][(wn * 64 + i * 16 + frow) * kLdsStride + fcol]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const v4i *>(&sX[cur][(wm * 64 + j * 16 + frow) * kLdsStride + fcol]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if (step + 1 < nsteps)
            store_tiles(cur ^ 1, rw, rx);
        __syncthreads();
    }

    // epilogue: lane holds acc rows n = 4 (lane / 16) + r (r = 0..3) of each 16x16 tile, column m = lane % 16
    // vector stores need every row start 16-byte (int32 / fp32) or 8-byte (bf16) aligned
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(c) % (MODE == 1 ? 8 : 16)) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 64 + j * 16 + (lane % 16);
        if (m >= M)
            continue;
        const float sxm = (MODE == 0) ? 0.0f : sa[m];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t nb = n0 + wn * 64 + i * 16 + 4 * (lane / 16);
            const v4i v = acc[i][j];
            if (MODE == 0) {
                int32_t *out = static_cast<int32_t *>(c) + m * N + nb;
                if (vec_ok && nb + 3 < N) {
                    *reinterpret_cast<v4i *>(out) = v;
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (nb + r < N)
                            out[r] = v[r];
                }
            } else {
                float f[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float swn = (nb + r < N) ? sb[nb + r] : 0.0f;
                    f[r] = (float)v[r] * (sxm * swn);
                }
                if (MODE == 1) {
                    uint16_t *out = static_cast<uint16_t *>(c) + m * N + nb;
                    if (vec_ok && nb + 3 < N) {
                        *reinterpret_cast<uint2 *>(out) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
                    } else {
                        for (int r = 0; r < 4; ++r)
                            if (nb + r < N)
                                out[r] = (uint16_t)f32_to_bf16_bits(f[r]);
                    }
                } else {
                    float *out = static_cast<float *>(c) + m * N + nb;
                    if (vec_ok && nb + 3 < N) {
                        *reinterpret_cast<float4 *>(out) = make_float4(f[0], f[1], f[2], f[3]);
                    } else {
                        for (int r = 0; r < 4; ++r)
                            if (nb + r < N)
                                out[r] = f[r];
                    }
                }
            }
        }
    }
}

hipError_t launch_gemm_i8(const GemmI8Args &g, hipStream_t st)
{
    const int64_t tiles = ((g.N + kBN - 1) / kBN) * ((g.M + kBM - 1) / kBM);
    const dim3 grid((unsigned)tiles), block(256);
    if (g.sa == nullptr)
        k_gemm_i8<0><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, nullptr, nullptr, g.c);
    else if (g.c_bf16)
        k_gemm_i8<1><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c);
    else
        k_gemm_i8<2><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c);
    return hipGetLastError();
}

}  // namespace pqg
