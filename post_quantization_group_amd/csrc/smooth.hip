// smooth.hip -- SmoothQuant smoothing factor on gfx950.
//
// s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)  ("量化、蒸馏与模型压缩" §2.3 eq. (1); "第11章 模型量化与压缩" §11.4.3).
// Two column reductions (activations X [T, K] over tokens, weights W [N, K] over output rows) and one
// elementwise pass. Max is exact and order independent, so the slicing below cannot change a bit.
//
// k_colabsmax: block (256 threads) x = 2048 consecutive columns (8 per thread, one 16-byte load per row),
// block y = a slice of rows; writes the slice maxima to ws[slice][K]. k_smooth_factor reduces the slices.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

constexpr int kColSlices = 64;  // row slices per tensor (at most)

template <typename XT>
__global__ __launch_bounds__(256) void k_colabsmax(const XT *__restrict__ x, int64_t rows, int64_t cols,
                                                   int64_t rows_per_slice, float *__restrict__ ws)
{
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk of 8 columns
    if (ch * 8 >= cols)
        return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_slice;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rows_per_slice);
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t r = r0; r < r1; ++r) {
        float v[8];
        load8<XT>(x + r * cols + ch * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[i]));
    }
    float4 *o = reinterpret_cast<float4 *>(ws + (int64_t)blockIdx.y * cols + ch * 8);
    o[0] = make_float4(m[0], m[1], m[2], m[3]);
    o[1] = make_float4(m[4], m[5], m[6], m[7]);
}

__global__ __launch_bounds__(256) void k_smooth_factor(const float *__restrict__ wsx, int px,
                                                       const float *__restrict__ wsw, int pw, int64_t cols,
                                                       double alpha, float *__restrict__ s)
{
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= cols)
        return;
    float ax = 0.0f, aw = 0.0f;
    for (int p = 0; p < px; ++p)
        ax = __builtin_fmaxf(ax, wsx[(int64_t)p * cols + j]);
    for (int p = 0; p < pw; ++p)
        aw = __builtin_fmaxf(aw, wsw[(int64_t)p * cols + j]);
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

namespace {
inline int slices_for(int64_t rows) { return (int)std::max<int64_t>(1, std::min<int64_t>(kColSlices, rows)); }
}  // namespace

size_t smooth_workspace_bytes(int64_t tokens, int64_t out_features, int64_t in_features)
{
    return (size_t)(slices_for(tokens) + slices_for(out_features)) * (size_t)in_features * sizeof(float);
}

hipError_t launch_smooth(const SmoothArgs &a, hipStream_t st)
{
    const int px = slices_for(a.tokens), pw = slices_for(a.out_features);
    float *wsx = static_cast<float *>(a.workspace);
    float *wsw = wsx + (int64_t)px * a.in_features;
    const unsigned gx = (unsigned)((a.in_features / 8 + 255) / 256);
    const int64_t rpx = (a.tokens + px - 1) / px, rpw = (a.out_features + pw - 1) / pw;
    if (a.x_bf16)
        k_colabsmax<uint16_t><<<dim3(gx, px), 256, 0, st>>>(static_cast<const uint16_t *>(a.x), a.tokens,
                                                             a.in_features, rpx, wsx);
    else
        k_colabsmax<float><<<dim3(gx, px), 256, 0, st>>>(static_cast<const float *>(a.x), a.tokens, a.in_features,
                                                          rpx, wsx);
    if (a.w_bf16)
        k_colabsmax<uint16_t><<<dim3(gx, pw), 256, 0, st>>>(static_cast<const uint16_t *>(a.w), a.out_features,
                                                             a.in_features, rpw, wsw);
    else
        k_colabsmax<float><<<dim3(gx, pw), 256, 0, st>>>(static_cast<const float *>(a.w), a.out_features,
                                                          a.in_features, rpw, wsw);
    k_smooth_factor<<<(unsigned)((a.in_features + 255) / 256), 256, 0, st>>>(wsx, px, wsw, pw, a.in_features,
                                                                             a.alpha, a.s);
    return hipGetLastError();
}

}  // namespace pqg
