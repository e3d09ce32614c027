// smooth.hip -- SmoothQuant smoothing factor on gfx950.
//
// s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)  ("量化、蒸馏与模型压缩" §2.3 eq. (1); "第11章 模型量化与压缩" §11.4.3).
// Two column reductions (activations X [T, K] over tokens, weights W [N, K] over output rows) and one
// elementwise pass. Max is exact and order independent, so the slicing below cannot change a bit.
//
// k_colabsmax: one launch for both tensors. A block of four waves owns 512 consecutive columns (8 per lane, one
// 16-byte piece per row for bf16, two for fp32) and a slice of kSliceRows rows; wave w reduces rows
// 16 w .. 16 w + 15 of the slice with all sixteen rows' loads issued before the first maximum, the four
// waves' maxima meet in LDS, and the block writes the slice maxima to ws[slice][K]. Row slices of X come
// first in the grid's y dimension, then those of W.
// k_smooth_factor: a block of 256 threads owns 16 columns; thread group q reduces slices q, q + 16, ... of
// both tensors, the sixteen partial maxima meet in LDS, and the first group evaluates the factor.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

constexpr int kSliceRows = 64;      // rows per block, one workspace row per block
constexpr int kWaveRows = 16;       // rows per wave, all in flight together
constexpr int kColsPerBlock = 512;  // 64 lanes x 8 columns
constexpr int kColThreads = 256;
static_assert(kSliceRows == kWaveRows * (kColThreads / kWave), "the waves of a block cover its slice");

__host__ __device__ inline int64_t slices_for(int64_t rows)
{
    return rows < kSliceRows ? 1 : (rows + kSliceRows - 1) / kSliceRows;
}

// Column maxima of |x| over rows r0 .. r0 + kWaveRows - 1 (those below `rows`) for the 8 columns of chunk ch.
// Rows past the end re-read the last row, which leaves a maximum unchanged; no load sits under a branch.
template <typename XT>
__device__ __forceinline__ void colabsmax_rows(const XT *__restrict__ x, int64_t rows, int64_t cols, int64_t ch,
                                               int64_t r0, float m[8])
{
    constexpr int XW = sizeof(XT) * 8 / 16;  // 16-byte pieces per chunk: 1 (bf16) or 2 (fp32)
    uint4 raw[kWaveRows][XW];
#pragma unroll
    for (int u = 0; u < kWaveRows; ++u) {
        const int64_t r = std::min<int64_t>(r0 + u, rows - 1);
        const uint4 *p = reinterpret_cast<const uint4 *>(x + r * cols + ch * 8);
#pragma unroll
        for (int q = 0; q < XW; ++q)
            raw[u][q] = p[q];
    }
#pragma unroll
    for (int u = 0; u < kWaveRows; ++u) {
        float v[8];
        if (XW == 1) {
            v[0] = bf16_lo(raw[u][0].x);
            v[1] = bf16_hi(raw[u][0].x);
            v[2] = bf16_lo(raw[u][0].y);
            v[3] = bf16_hi(raw[u][0].y);
            v[4] = bf16_lo(raw[u][0].z);
            v[5] = bf16_hi(raw[u][0].z);
            v[6] = bf16_lo(raw[u][0].w);
            v[7] = bf16_hi(raw[u][0].w);
        } else {
#pragma unroll
            for (int q = 0; q < XW; ++q) {
                v[4 * q + 0] = __uint_as_float(raw[u][q].x);
                v[4 * q + 1] = __uint_as_float(raw[u][q].y);
                v[4 * q + 2] = __uint_as_float(raw[u][q].z);
                v[4 * q + 3] = __uint_as_float(raw[u][q].w);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[i]));
    }
}

template <typename XT, typename WT>
__global__ __launch_bounds__(kColThreads) void k_colabsmax(const XT *__restrict__ x, int64_t tokens,
                                                           const WT *__restrict__ w, int64_t out_features,
                                                           int64_t cols, int64_t px, float *__restrict__ wsx,
                                                           float *__restrict__ wsw)
{
    __shared__ __attribute__((aligned(16))) float red[kColThreads / kWave][kColsPerBlock];
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t nch = cols / 8;
    const int64_t ch = std::min<int64_t>((int64_t)blockIdx.x * kWave + lane, nch - 1);
    const bool is_x = blockIdx.y < px;
    const int64_t slice = is_x ? blockIdx.y : blockIdx.y - px;
    const int64_t r0 = slice * kSliceRows + (int64_t)wv * kWaveRows;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (is_x) {
        if (r0 < tokens)
            colabsmax_rows<XT>(x, tokens, cols, ch, r0, m);
    } else {
        if (r0 < out_features)
            colabsmax_rows<WT>(w, out_features, cols, ch, r0, m);
    }
    float4 *mine = reinterpret_cast<float4 *>(&red[wv][lane * 8]);
    mine[0] = make_float4(m[0], m[1], m[2], m[3]);
    mine[1] = make_float4(m[4], m[5], m[6], m[7]);
    __syncthreads();
    // thread t combines columns 2 t, 2 t + 1 of the block over the four waves
    const int c2 = 2 * (int)threadIdx.x;
    float2 r = *reinterpret_cast<const float2 *>(&red[0][c2]);
#pragma unroll
    for (int i = 1; i < kColThreads / kWave; ++i) {
        const float2 o = *reinterpret_cast<const float2 *>(&red[i][c2]);
        r.x = __builtin_fmaxf(r.x, o.x);
        r.y = __builtin_fmaxf(r.y, o.y);
    }
    const int64_t col = (int64_t)blockIdx.x * kColsPerBlock + c2;
    if (col < cols)
        *reinterpret_cast<float2 *>((is_x ? wsx : wsw) + slice * cols + col) = r;
}

// Maximum over slices q, q + Q, q + 2Q, ... of column j (four loads in flight).
template <int Q>
__device__ __forceinline__ float slices_max(const float *__restrict__ ws, int64_t slices, int64_t cols, int64_t j,
                                            int q)
{
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t p = q;
    for (; p + 3 * Q < slices; p += 4 * Q) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            a[u] = __builtin_fmaxf(a[u], ws[(p + Q * u) * cols + j]);
    }
    for (; p < slices; p += Q)
        a[0] = __builtin_fmaxf(a[0], ws[p * cols + j]);
    return __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), __builtin_fmaxf(a[2], a[3]));
}

constexpr int kFactorCols = 16;                  // columns per block
constexpr int kFactorSplit = 256 / kFactorCols;  // slice groups per column

__global__ __launch_bounds__(256) void k_smooth_factor(const float *__restrict__ wsx, int64_t px,
                                                       const float *__restrict__ wsw, int64_t pw, int64_t cols,
                                                       double alpha, float *__restrict__ s)
{
    __shared__ float part[2][kFactorSplit][kFactorCols];
    const int c = threadIdx.x % kFactorCols, q = threadIdx.x / kFactorCols;
    const int64_t j = (int64_t)blockIdx.x * kFactorCols + c;
    const int64_t jj = j < cols ? j : cols - 1;
    part[0][q][c] = slices_max<kFactorSplit>(wsx, px, cols, jj, q);
    part[1][q][c] = slices_max<kFactorSplit>(wsw, pw, cols, jj, q);
    __syncthreads();
    if (q != 0 || j >= cols)
        return;
    float ax = part[0][0][c], aw = part[1][0][c];
    for (int i = 1; i < kFactorSplit; ++i) {
        ax = __builtin_fmaxf(ax, part[0][i][c]);
        aw = __builtin_fmaxf(aw, part[1][i][c]);
    }
    float r;
    if (ax == 0.0f || aw == 0.0f)
        r = 1.0f;  // undefined factor: leave the channel unscaled
    else if (alpha == 0.5)
        r = __builtin_sqrtf(ax) / __builtin_sqrtf(aw);
    else if (alpha == 1.0)
        r = ax;
    else if (alpha == 0.0)
        r = 1.0f / aw;
    else
        r = (float)(pow((double)ax, alpha) / pow((double)aw, 1.0 - alpha));
    s[j] = r;
}

size_t smooth_workspace_bytes(int64_t tokens, int64_t out_features, int64_t in_features)
{
    return (size_t)(slices_for(tokens) + slices_for(out_features)) * (size_t)in_features * sizeof(float);
}

hipError_t launch_smooth(const SmoothArgs &a, hipStream_t st)
{
    const int64_t px = slices_for(a.tokens), pw = slices_for(a.out_features);
    float *wsx = static_cast<float *>(a.workspace);
    float *wsw = wsx + px * a.in_features;
    if (px + pw > 65535)  // the row slices of both tensors span the grid's y dimension
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((a.in_features + kColsPerBlock - 1) / kColsPerBlock), (unsigned)(px + pw));
    if (a.x_bf16 && a.w_bf16)
        k_colabsmax<uint16_t, uint16_t><<<grid, kColThreads, 0, st>>>(static_cast<const uint16_t *>(a.x), a.tokens,
                                                                      static_cast<const uint16_t *>(a.w),
                                                                      a.out_features, a.in_features, px, wsx, wsw);
    else if (a.x_bf16)
        k_colabsmax<uint16_t, float><<<grid, kColThreads, 0, st>>>(static_cast<const uint16_t *>(a.x), a.tokens,
                                                                   static_cast<const float *>(a.w), a.out_features,
                                                                   a.in_features, px, wsx, wsw);
    else if (a.w_bf16)
        k_colabsmax<float, uint16_t><<<grid, kColThreads, 0, st>>>(static_cast<const float *>(a.x), a.tokens,
                                                                   static_cast<const uint16_t *>(a.w),
                                                                   a.out_features, a.in_features, px, wsx, wsw);
    else
        k_colabsmax<float, float><<<grid, kColThreads, 0, st>>>(static_cast<const float *>(a.x), a.tokens,
                                                                static_cast<const float *>(a.w), a.out_features,
                                                                a.in_features, px, wsx, wsw);
    k_smooth_factor<<<(unsigned)((a.in_features + kFactorCols - 1) / kFactorCols), 256, 0, st>>>(
        wsx, px, wsw, pw, a.in_features, a.alpha, a.s);
    return hipGetLastError();
}

}  // namespace pqg
