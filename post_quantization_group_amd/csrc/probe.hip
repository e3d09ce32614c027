// probe.hip -- two measurement utilities, no step of the method.
//
// k_stream_read: one streaming read of a device buffer, to measure the device's achievable read rate beside
// the rates of the library's kernels. Every byte is read once with 16-byte non-temporal loads, four per lane
// in flight (grid-stride); the loaded words are folded by xor into one word, which reaches `sink` only under a
// condition on the data (so the loads cannot be dropped); the sink's contents carry no meaning.
//
// k_mfma_i8: the int8 matrix-core rate the device sustains with no memory traffic at all, to set the INT8
// GEMM's rate beside. Blocks of 8 waves (two per SIMD, as the GEMM runs) issue v_mfma_i32_32x32x32_i8 on twelve
// independent accumulators per wave (the GEMM wave's 4 x 3 tiles, in VGPRs as there) from register operands; the clock the chip holds under this load is the
// one the GEMM sees, so the ratio of the two rates isolates the GEMM's schedule from the chip's power limit.
// The accumulators are folded into one word that reaches `sink` only under a condition on it.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

typedef unsigned probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_stream_read(const probe_u32x4 *__restrict__ src, int64_t n16,
                                                     uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    probe_u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + stride < n16; i += 2 * stride) {
        const probe_u32x4 a = __builtin_nontemporal_load(src + i);
        const probe_u32x4 b = __builtin_nontemporal_load(src + i + stride);
        acc ^= a ^ b;
    }
    for (; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9E3779B9u)
        sink[0] = r;
}

typedef int probe_v4i __attribute__((ext_vector_type(4)));
typedef int probe_v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void k_mfma_i8(int iters, uint32_t *__restrict__ sink)
{
    const int t = (int)threadIdx.x + (int)blockIdx.x * 512;
    probe_v4i fa[4], fb[3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        fa[i] = probe_v4i{t + i, t * 3 + i, t * 5 + 2 * i, t * 7 + 3 * i};
#pragma unroll
    for (int j = 0; j < 3; ++j)
        fb[j] = probe_v4i{t ^ (0x55 + j), t * 11 + j, t * 13 + 2 * j, t * 17 + 3 * j};
    probe_v16i acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            acc[i][j] = probe_v16i{};
    for (int k = 0; k < iters; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                r ^= (uint32_t)acc[i][j][e];
    if (r == 0x9E3779B9u)
        sink[0] = r;
}

hipError_t launch_mfma_i8(int64_t blocks, int32_t iters, uint32_t *sink, hipStream_t st)
{
    if (blocks == 0 || iters == 0)
        return hipSuccess;
    k_mfma_i8<<<(unsigned)blocks, 512, 0, st>>>(iters, sink);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st)
{
    const int64_t n16 = bytes / 16;
    const int64_t blocks = std::min<int64_t>((n16 + 1023) / 1024, 65536);  // about 4 loads per lane
    if (blocks == 0)
        return hipSuccess;
    k_stream_read<<<(unsigned)blocks, 256, 0, st>>>(static_cast<const probe_u32x4 *>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace pqg
