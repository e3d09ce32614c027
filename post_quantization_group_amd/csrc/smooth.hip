// smooth.hip -- SmoothQuant smoothing factor on gfx950.
//
// s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)  ("量化、蒸馏与模型压缩" §2.3 eq. (1); "第11章 模型量化与压缩" §11.4.3).
// Two column reductions (activations X [T, K] over tokens, weights W [N, K] over output rows) and one
// elementwise pass. Max is exact and order independent, so the slicing below cannot change a bit.
//
// k_colabsmax: one launch for both tensors (blockIdx.z). A block is one wave of 64 threads owning 512
// consecutive columns (8 per thread, one 16-byte load per row) and a slice of kRowsPerSlice rows; it writes
// the slice maxima to ws[slice][K]. Eight rows are loaded before they are reduced, so each lane keeps
// eight 16-byte loads in flight.
// k_smooth_factor: a block of 256 threads owns 16 columns; thread group q reduces slices q, q + 16, ... of
// both tensors, the sixteen partial maxima meet in LDS, and the first group evaluates the factor.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

constexpr int kRowsPerSlice = 32;
constexpr int kColsPerBlock = 512;
constexpr int kRowUnroll = 8;

__host__ __device__ inline int64_t slices_for(int64_t rows)
{
    return rows < kRowsPerSlice ? 1 : (rows + kRowsPerSlice - 1) / kRowsPerSlice;
}

template <typename XT>
__device__ __forceinline__ void colabsmax_slice(const XT *__restrict__ x, int64_t rows, int64_t cols, int64_t ch,
                                                int64_t slice, float *__restrict__ ws)
{
    const int64_t r0 = slice * kRowsPerSlice;
    const int nr = (int)std::min<int64_t>(rows - r0, kRowsPerSlice);
    const XT *p = x + r0 * cols + ch * 8;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int r = 0;
    for (; r + kRowUnroll <= nr; r += kRowUnroll) {
        float v[kRowUnroll][8];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u)
            load8<XT>(p + (int64_t)(r + u) * cols, v[u]);
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[u][i]));
    }
    for (; r < nr; ++r) {
        float v[8];
        load8<XT>(p + (int64_t)r * cols, v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[i]));
    }
    float4 *o = reinterpret_cast<float4 *>(ws + slice * cols + ch * 8);
    o[0] = make_float4(m[0], m[1], m[2], m[3]);
    o[1] = make_float4(m[4], m[5], m[6], m[7]);
}

template <typename XT, typename WT>
__global__ __launch_bounds__(64) void k_colabsmax(const XT *__restrict__ x, int64_t tokens, const WT *__restrict__ w,
                                                  int64_t out_features, int64_t cols, float *__restrict__ wsx,
                                                  float *__restrict__ wsw)
{
    const int64_t ch = (int64_t)blockIdx.x * 64 + threadIdx.x;  // chunk of 8 columns
    if (ch * 8 >= cols)
        return;
    const int64_t slice = blockIdx.y;
    if (blockIdx.z == 0) {
        if (slice < slices_for(tokens))
            colabsmax_slice<XT>(x, tokens, cols, ch, slice, wsx);
    } else {
        if (slice < slices_for(out_features))
            colabsmax_slice<WT>(w, out_features, cols, ch, slice, wsw);
    }
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
    const dim3 grid((unsigned)((a.in_features + kColsPerBlock - 1) / kColsPerBlock), (unsigned)std::max(px, pw), 2);
    if (a.x_bf16 && a.w_bf16)
        k_colabsmax<uint16_t, uint16_t><<<grid, 64, 0, st>>>(static_cast<const uint16_t *>(a.x), a.tokens,
                                                             static_cast<const uint16_t *>(a.w), a.out_features,
                                                             a.in_features, wsx, wsw);
    else if (a.x_bf16)
        k_colabsmax<uint16_t, float><<<grid, 64, 0, st>>>(static_cast<const uint16_t *>(a.x), a.tokens,
                                                          static_cast<const float *>(a.w), a.out_features,
                                                          a.in_features, wsx, wsw);
    else if (a.w_bf16)
        k_colabsmax<float, uint16_t><<<grid, 64, 0, st>>>(static_cast<const float *>(a.x), a.tokens,
                                                          static_cast<const uint16_t *>(a.w), a.out_features,
                                                          a.in_features, wsx, wsw);
    else
        k_colabsmax<float, float><<<grid, 64, 0, st>>>(static_cast<const float *>(a.x), a.tokens,
                                                       static_cast<const float *>(a.w), a.out_features,
                                                       a.in_features, wsx, wsw);
    k_smooth_factor<<<(unsigned)((a.in_features + kFactorCols - 1) / kFactorCols), 256, 0, st>>>(
        wsx, px, wsw, pw, a.in_features, a.alpha, a.s);
    return hipGetLastError();
}

}  // namespace pqg
