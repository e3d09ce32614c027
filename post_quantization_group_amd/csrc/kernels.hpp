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
    bool meta16 = false;                // 16-bit metadata (decode path only): binary16 scales in scales16,
    const uint16_t *scales16 = nullptr;  // [N, K/g]; zeros then packed two per byte (flattened group index)
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

// Several independent decode products (M <= 4 tokens each, one group size / symmetry / output type) in one
// launch; the table travels in the kernel arguments.
constexpr int kMaxGroupedProblems = 8;
struct GroupedW4A16 {
    struct Problem {
        const uint16_t *x;  // bf16 [M, K]
        const uint8_t *w;   // [N, K/2]
        const float *scales;
        const uint16_t *scales16;  // unused here (fp32 scales); kept so the row-block code takes either
        const uint8_t *zeros;
        void *y;            // [M, N]
        int64_t N, K;
    } p[kMaxGroupedProblems];
    int64_t begin[kMaxGroupedProblems + 1];  // first row block of each problem, begin[count] = total
    int count;
};

struct W4A16GroupedArgs {
    const W4A16Args *problems;  // host array: x, N, K, w, scales, zeros, y of each problem
    int count;
    int64_t M;
    int group_size;
    bool symmetric;
    bool y_bf16;
};

hipError_t launch_w4a16_grouped(const W4A16GroupedArgs &a, hipStream_t st);

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

// INT4 groups with 16-bit metadata: binary16 scales, zero points two per byte (flattened group index).
struct Meta16Args {
    const void *x;  // quantize input [rows, cols] (bf16 or fp32)
    bool x_bf16;
    int64_t rows, cols;
    bool symmetric;
    int group_size;
    uint8_t *codes;      // packed [rows, cols / 2]
    uint16_t *scales16;  // [rows * cols / g] binary16
    uint8_t *zeros4;     // [(rows * cols / g + 1) / 2], NULL iff symmetric
};

hipError_t launch_quantize_meta16(const Meta16Args &a, hipStream_t st);
hipError_t launch_dequantize_meta16(const Meta16Args &a, void *out, bool out_bf16, hipStream_t st);

// KV cache: keys per channel over groups of block_tokens tokens (and their dequantization).
struct KvKeysArgs {
    const void *x;  // [tokens, channels] bf16 or fp32 (quantize only)
    bool x_bf16;
    int64_t tokens, channels;
    int block_tokens;
    bool symmetric;
    void *codes;     // int8 (symmetric) / uint8 [tokens, channels]
    float *scales;   // [tokens / T, channels]
    uint8_t *zeros;  // [tokens / T, channels], NULL iff symmetric
};

hipError_t launch_kv_keys(const KvKeysArgs &a, hipStream_t st);
hipError_t launch_kv_dequant_keys(const KvKeysArgs &a, void *out, bool out_bf16, hipStream_t st);

// KV cache: one online append step for a batch of sequences.
struct KvAppendArgs {
    const void *k_new, *v_new;  // [batch, channels], bf16 or fp32
    bool x_bf16;
    int64_t batch, channels;
    const int64_t *positions;  // [batch]
    int64_t max_tokens;
    int block_tokens, v_group_size;
    bool symmetric;
    void *k_res;                       // [batch, T, channels], the input dtype
    void *k_codes;                     // [batch, max_tokens, channels]
    float *k_scales;                   // [batch, max_tokens / T, channels]
    uint8_t *k_zeros;                  // same, NULL iff symmetric
    void *v_codes;                     // [batch, max_tokens, channels]
    float *v_scales;                   // [batch, max_tokens, channels / v_group_size or 1]
    uint8_t *v_zeros;                  // same, NULL iff symmetric
};

hipError_t launch_kv_append(const KvAppendArgs &a, hipStream_t st);

// One streaming read of `bytes` (a multiple of 16) at 16-byte aligned `src`; `sink` receives at most one word.
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_mfma_i8(int64_t blocks, int32_t iters, uint32_t *sink, hipStream_t st);

}  // namespace pqg
