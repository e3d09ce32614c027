// kernels.hpp -- launch interface between the C ABI (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace pqg {

enum { QG_TENSOR = 0, QG_ROW = 1, QG_GROUP = 2 };
enum { SMOOTH_NONE = 0, SMOOTH_DIV = 1, SMOOTH_MUL = 2 };

struct QuantArgs {
    const void *x;
    bool x_bf16;
    int64_t rows, cols;
    const float *smooth;
    int smooth_mode;
    int bits;
    bool symmetric;
    int granularity;
    int group_size;
    void *codes;
    float *scales;
    uint8_t *zeros;
    void *workspace;
};

// Static per-tensor quantization: fixed, caller-given (scale, zero); row_scales (optional) filled with scale.
struct StaticQuantArgs {
    const void *x;
    bool x_bf16;
    int64_t rows, cols;
    int bits;
    bool symmetric;
    float scale;
    int zero;
    void *codes;
    float *row_scales;
};

struct DequantArgs {
    const void *codes;
    const float *scales;
    const uint8_t *zeros;
    int64_t rows, cols;
    int bits;
    bool symmetric;
    int granularity;
    int group_size;
    void *out;
    bool out_bf16;
};

struct SmoothArgs {
    const void *x;
    bool x_bf16;
    int64_t tokens;
    const void *w;
    bool w_bf16;
    int64_t out_features, in_features;
    double alpha;
    float *s;
    void *workspace;
};

struct W4A16Args {
    const uint16_t *x;  // bf16 [M, K]
    int64_t M, N, K;
    const uint8_t *w;   // [N, K/2]
    const float *scales;
    const uint8_t *zeros;
    int group_size;
    bool symmetric;
    void *y;
    bool y_bf16;
};

struct GemmI8Args {
    const int8_t *a;  // [M, K]  (activation codes)
    const int8_t *b;  // [N, K]  (weight codes)
    int64_t M, N, K;
    // epilogue: raw int32 when sa == nullptr, else y = float(acc) * (sa[m] * sb[n])
    const float *sa;
    const float *sb;
    void *c;
    bool c_bf16;  // epilogue output type (ignored for raw int32)
};

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st);
size_t quantize_workspace_bytes(int32_t granularity);
hipError_t launch_quantize_static(const StaticQuantArgs &a, hipStream_t st);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t st);

size_t smooth_workspace_bytes(int64_t tokens, int64_t out_features, int64_t in_features);
hipError_t launch_smooth(const SmoothArgs &a, hipStream_t st);

hipError_t launch_w4a16(const W4A16Args &a, hipStream_t st);

hipError_t launch_gemm_i8(const GemmI8Args &a, hipStream_t st);

// W4A8: INT8 per-token activation codes x INT4 per-group weight codes.
struct W4A8Args {
    const int8_t *x_q;       // [M, K]
    const float *x_scales;   // [M]
    int64_t M, N, K;
    const uint8_t *w;        // packed INT4 [N, K/2]
    const float *w_scales;   // [N, K/g]
    const uint8_t *w_zeros;  // [N, K/g], NULL iff symmetric
    int group_size;
    bool symmetric;
    void *y;                 // [M, N]
    bool y_bf16;
};

hipError_t launch_w4a8(const W4A8Args &a, hipStream_t st);

}  // namespace pqg
