// kv.hip -- INT8 KV cache: keys per channel over token groups, values per token, appended online.
//
// ("第11章 模型量化与压缩" §11.6.2-§11.6.5: the cache is produced during decoding, so it is quantized online;
// per-token scales suit V, per-channel scales suit K, whose outliers sit in a few channels; KIVI keeps the most
// recent keys at full precision and quantizes them per channel once a group of tokens is complete.)
//
// Layout: one layer's keys (or values) token-major, [tokens, channels] with channels = KV heads x head_dim.
// Key codes [tokens, channels] with scales (and zero points) [tokens / T, channels]; value codes
// [tokens, channels] with one scale per token or per group of channels. Codes and scales are those of the
// quantize kernels: s from the segment's range, q = clamp(rne(x / s) + z).
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

namespace {

// 8 codes of an INT8 segment -> 8 bytes.
__device__ __forceinline__ uint2 codes8(const float v[8], const SegParams *p)
{
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        w[j / 4] |= ((uint32_t)code_of(v[j], p[j]) & 0xFFu) << (8 * (j % 4));
    return make_uint2(w[0], w[1]);
}

template <bool SYM>
__device__ __forceinline__ void stats_init(float *am, float *lo, float *hi, const float v[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        am[j] = __builtin_fabsf(v[j]);
        lo[j] = v[j];
        hi[j] = v[j];
    }
}

template <bool SYM>
__device__ __forceinline__ void stats_add(float *am, float *lo, float *hi, const float v[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        am[j] = __builtin_fmaxf(am[j], __builtin_fabsf(v[j]));
        lo[j] = __builtin_fminf(lo[j], v[j]);
        hi[j] = __builtin_fmaxf(hi[j], v[j]);
    }
}

// ------------------------------------------------------------------ keys, per channel over token groups
//
// Block (group b, 64 channels): 256 threads as 32 token rows x 8 lanes of 8 channels; a thread keeps its T / 32
// rows of 8 values in registers, so the group is read once. Channel ranges: within a wave over its 8 rows by
// xor shuffles, then over the four waves through LDS (max and min are exact in any order).
constexpr int kKvCols = 64, kKvThreads = 256, kKvRows = kKvThreads / 8;

// Per-channel parameters of a tile of rows x CW channels held by 256 threads as 256 / LR row lanes x LR = CW / 8
// channel lanes (thread tid: channels 8 (tid % LR) .. + 7): the thread's partial ranges are combined over the
// wave's row lanes by xor shuffles, then over the four waves through `red` (max and min are exact in any order).
template <bool SYM, int CW = kKvCols>
__device__ __forceinline__ void tile_params(float *am, float *lo, float *hi, float (*red)[kKvThreads / kWave][CW],
                                            SegParams *p)
{
    constexpr int LR = CW / 8;
    const int tid = threadIdx.x, lr = tid % LR;
#pragma unroll
    for (int off = LR; off < kWave; off <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            am[j] = __builtin_fmaxf(am[j], __shfl_xor(am[j], off, kWave));
            lo[j] = __builtin_fminf(lo[j], __shfl_xor(lo[j], off, kWave));
            hi[j] = __builtin_fmaxf(hi[j], __shfl_xor(hi[j], off, kWave));
        }
    const int wv = tid / kWave;
    if (tid % kWave < LR)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            red[0][wv][lr * 8 + j] = am[j];
            red[1][wv][lr * 8 + j] = lo[j];
            red[2][wv][lr * 8 + j] = hi[j];
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float a = red[0][0][lr * 8 + j], l = red[1][0][lr * 8 + j], h = red[2][0][lr * 8 + j];
#pragma unroll
        for (int w = 1; w < kKvThreads / kWave; ++w) {
            a = __builtin_fmaxf(a, red[0][w][lr * 8 + j]);
            l = __builtin_fminf(l, red[1][w][lr * 8 + j]);
            h = __builtin_fmaxf(h, red[2][w][lr * 8 + j]);
        }
        p[j] = seg_params<8, SYM>(a, l, h);
    }
}

// Keys are read once and their codes written once: non-temporal loads and stores keep them out of the way of
// the caches (3 % faster than ordinary ones at T = 128).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));

template <typename XT>
__device__ __forceinline__ void load8_nt(const XT *__restrict__ p, float v[8])
{
    if constexpr (sizeof(XT) == 2) {
        const u32x4_nt u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const u32x4_nt a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
        const u32x4_nt b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p) + 1);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = __uint_as_float(w[i]);
    }
}

// Block (group b, CW channels): a thread keeps its rows of 8 values in registers, so the group is read once and
// written once. With CW = 128 a row's 16 lanes read 256 bytes (bf16) and write whole 128-byte lines of codes.
template <typename XT, bool SYM, int T, int CW>
__global__ __launch_bounds__(kKvThreads) void k_kv_keys(const XT *__restrict__ x, int64_t channels,
                                                        void *__restrict__ codes, float *__restrict__ scales,
                                                        uint8_t *__restrict__ zeros)
{
    constexpr int LR = CW / 8, ROWS = kKvThreads / LR, RP = T / ROWS;  // lanes per row, rows per pass, per thread
    static_assert(RP >= 1 && RP * ROWS == T, "whole rows per thread");
    __shared__ float red[3][kKvThreads / kWave][CW];
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x, lr = tid % LR, r0 = tid / LR;
    const int64_t c0 = (int64_t)blockIdx.y * CW + lr * 8;
    float v[RP][8];
#pragma unroll
    for (int i = 0; i < RP; ++i)
        load8_nt<XT>(x + (b * T + r0 + ROWS * i) * channels + c0, v[i]);
    float am[8], lo[8], hi[8];
    stats_init<SYM>(am, lo, hi, v[0]);
#pragma unroll
    for (int i = 1; i < RP; ++i)
        stats_add<SYM>(am, lo, hi, v[i]);
    SegParams p[8];
    tile_params<SYM, CW>(am, lo, hi, red, p);
    if (r0 == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            scales[b * channels + c0 + j] = p[j].st;
            if (!SYM)
                zeros[b * channels + c0 + j] = (uint8_t)p[j].z;
        }
    }
#pragma unroll
    for (int i = 0; i < RP; ++i)
    {
        const uint2 cw = codes8(v[i], p);
        __builtin_nontemporal_store(
            u32x2_nt{cw.x, cw.y},
            reinterpret_cast<u32x2_nt *>(static_cast<int8_t *>(codes) + (b * T + r0 + ROWS * i) * channels + c0));
    }
}

template <typename XT, bool SYM, int CW>
hipError_t keys_cw(const KvKeysArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)(a.tokens / a.block_tokens), (unsigned)(a.channels / CW)), block(kKvThreads);
    const XT *x = static_cast<const XT *>(a.x);
    switch (a.block_tokens) {
    case 32:
        k_kv_keys<XT, SYM, 32, CW><<<grid, block, 0, st>>>(x, a.channels, a.codes, a.scales, a.zeros);
        break;
    case 64:
        k_kv_keys<XT, SYM, 64, CW><<<grid, block, 0, st>>>(x, a.channels, a.codes, a.scales, a.zeros);
        break;
    case 128:
        k_kv_keys<XT, SYM, 128, CW><<<grid, block, 0, st>>>(x, a.channels, a.codes, a.scales, a.zeros);
        break;
    default:
        k_kv_keys<XT, SYM, 256, CW><<<grid, block, 0, st>>>(x, a.channels, a.codes, a.scales, a.zeros);
        break;
    }
    return hipGetLastError();
}

// 128-channel tiles when the channels allow it (whole 128-byte lines of codes per row), else 64.
template <typename XT, bool SYM>
hipError_t keys_go(const KvKeysArgs &a, hipStream_t st)
{
    if (a.channels % 128 == 0)
        return keys_cw<XT, SYM, 128>(a, st);
    return keys_cw<XT, SYM, 64>(a, st);
}

// ------------------------------------------------------------------ keys back

// x_hat[t, c] = s[t / T, c] (q[t, c] - z[t / T, c]): one thread per 8 elements, grid-stride.
template <bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_kv_dequant_keys(const void *__restrict__ codes, const float *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros, int64_t tokens,
                                                         int64_t channels, int64_t block_tokens, void *__restrict__ out)
{
    const int64_t n8 = tokens * channels / 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i * 8, t = e / channels, c = e % channels;
        const int64_t sb = t / block_tokens * channels + c;
        const uint2 q = *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(codes) + e);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t byte = ((j < 4 ? q.x : q.y) >> (8 * (j % 4))) & 0xFFu;
            const int qi = SYM ? (int)(int8_t)byte : (int)byte - (int)zeros[sb + j];
            v[j] = scales[sb + j] * (float)qi;
        }
        if (OUT_BF16)
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + e) =
                make_uint4(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]), pack_bf16x2_rne(v[4], v[5]),
                           pack_bf16x2_rne(v[6], v[7]));
        else {
            float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + e);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

// ------------------------------------------------------------------ online append

constexpr int kAppThreads = 256;
constexpr int kAppChunks = 4;  // 8-channel chunks per thread: channels <= 256 * 4 * 8 = 8192

// Range of a whole row over the block (per-token value scales): wave shuffles, then the four waves via LDS.
template <bool SYM>
__device__ __forceinline__ void block_range8(float &am, float &lo, float &hi, float (*red)[kAppThreads / kWave])
{
    am = wave_max<kWave>(am);
    lo = wave_min<kWave>(lo);
    hi = wave_max<kWave>(hi);
    const int wv = threadIdx.x / kWave;
    __syncthreads();  // red may still be read from an earlier use
    if (threadIdx.x % kWave == 0) {
        red[0][wv] = am;
        red[1][wv] = lo;
        red[2][wv] = hi;
    }
    __syncthreads();
    am = red[0][0];
    lo = red[1][0];
    hi = red[2][0];
#pragma unroll
    for (int w = 1; w < kAppThreads / kWave; ++w) {
        am = __builtin_fmaxf(am, red[0][w]);
        lo = __builtin_fminf(lo, red[1][w]);
        hi = __builtin_fmaxf(hi, red[2][w]);
    }
}

// Block (sequence b, 64-channel slice y). Values: every block of the sequence quantizes the whole new value row
// (a few KB) per token (VG = 0) or per group of VG channels and writes its slice of row p. Keys: the block copies
// its slice of the new key to residual slot p % T; when p % T == T - 1 the group of tokens is complete and the
// block quantizes its T x 64 tile per channel (the new row read from the input) into rows p - T + 1 .. p.
template <typename XT, bool SYM, int VG>
__global__ __launch_bounds__(kAppThreads) void k_kv_append(const XT *__restrict__ k_new, const XT *__restrict__ v_new,
                                                           int64_t channels, const int64_t *__restrict__ positions,
                                                           int64_t max_tokens, int T, XT *__restrict__ k_res,
                                                           int8_t *__restrict__ k_codes, float *__restrict__ k_scales,
                                                           uint8_t *__restrict__ k_zeros, int8_t *__restrict__ v_codes,
                                                           float *__restrict__ v_scales, uint8_t *__restrict__ v_zeros)
{
    static_assert(kAppThreads == kKvThreads, "the key tile uses the bulk kernel's thread layout");
    __shared__ float red[3][kAppThreads / kWave];
    __shared__ float tred[3][kKvThreads / kWave][kKvCols];
    const int64_t b = blockIdx.x;
    const int y = blockIdx.y;  // channels 64 y .. 64 y + 63 = chunks 8 y .. 8 y + 7
    const int64_t p = positions[b];
    if (p < 0 || p >= max_tokens)
        return;  // uniform over the block
    const int tid = threadIdx.x;
    const int64_t nchunk = channels / 8;
    const XT *kn = k_new + b * channels;
    const XT *vn = v_new + b * channels;
    auto in_slice = [&](int64_t ci) { return ci >= 8 * (int64_t)y && ci < 8 * (int64_t)y + 8; };

    // values
    float v[kAppChunks][8];
#pragma unroll
    for (int u = 0; u < kAppChunks; ++u) {
        const int64_t ci = tid + (int64_t)kAppThreads * u;
        if (ci < nchunk)
            load8<XT>(vn + ci * 8, v[u]);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[u][j] = 0.0f;  // outside the row: 0 leaves max |x| and the widened range unchanged
    }
    const int64_t vrow = b * max_tokens + p;
    if (VG == 0) {
        float am = 0.0f, lo = 0.0f, hi = 0.0f;  // the range is widened to contain 0 anyway (asymmetric)
#pragma unroll
        for (int u = 0; u < kAppChunks; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                am = __builtin_fmaxf(am, __builtin_fabsf(v[u][j]));
                lo = __builtin_fminf(lo, v[u][j]);
                hi = __builtin_fmaxf(hi, v[u][j]);
            }
        block_range8<SYM>(am, lo, hi, red);
        const SegParams sp = seg_params<8, SYM>(am, lo, hi);
        const SegParams ps[8] = {sp, sp, sp, sp, sp, sp, sp, sp};
#pragma unroll
        for (int u = 0; u < kAppChunks; ++u) {
            const int64_t ci = tid + (int64_t)kAppThreads * u;
            if (ci < nchunk && in_slice(ci))
                *reinterpret_cast<uint2 *>(v_codes + vrow * channels + ci * 8) = codes8(v[u], ps);
        }
        if (y == 0 && tid == 0) {
            v_scales[vrow] = sp.st;
            if (!SYM)
                v_zeros[vrow] = (uint8_t)sp.z;
        }
    } else {
        // a group is VG / 8 consecutive chunks = consecutive lanes of one pass (256 is a multiple of VG / 8)
        constexpr int GL = VG / 8;
        const int64_t ngroups = channels / VG;
#pragma unroll
        for (int u = 0; u < kAppChunks; ++u) {
            const int64_t ci = tid + (int64_t)kAppThreads * u;
            if ((int64_t)kAppThreads * u >= nchunk)
                break;  // uniform: no chunk of this pass is in the row
            float am = 0.0f, lo = v[u][0], hi = v[u][0];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                am = __builtin_fmaxf(am, __builtin_fabsf(v[u][j]));
                lo = __builtin_fminf(lo, v[u][j]);
                hi = __builtin_fmaxf(hi, v[u][j]);
            }
            am = wave_max<GL>(am);
            lo = wave_min<GL>(lo);
            hi = wave_max<GL>(hi);
            const SegParams sp = seg_params<8, SYM>(am, lo, hi);
            const SegParams ps[8] = {sp, sp, sp, sp, sp, sp, sp, sp};
            if (ci < nchunk && in_slice(ci)) {
                *reinterpret_cast<uint2 *>(v_codes + vrow * channels + ci * 8) = codes8(v[u], ps);
                if (ci % GL == 0) {  // the group's first chunk lies in exactly one slice
                    v_scales[vrow * ngroups + ci / GL] = sp.st;
                    if (!SYM)
                        v_zeros[vrow * ngroups + ci / GL] = (uint8_t)sp.z;
                }
            }
        }
    }

    // keys: this slice of the residual slot
    const int slot = (int)(p % T);
    XT *res = k_res + b * (int64_t)T * channels;
    const int64_t c0 = (int64_t)y * kKvCols;
    if (tid < 8) {
        const int64_t c = c0 + tid * 8;
        if (sizeof(XT) == 2)
            *reinterpret_cast<uint4 *>(res + slot * channels + c) = *reinterpret_cast<const uint4 *>(kn + c);
        else {
            reinterpret_cast<float4 *>(res + slot * channels + c)[0] = reinterpret_cast<const float4 *>(kn + c)[0];
            reinterpret_cast<float4 *>(res + slot * channels + c)[1] = reinterpret_cast<const float4 *>(kn + c)[1];
        }
    }
    if (slot != T - 1)
        return;  // uniform
    // the complete group, as the bulk kernel: rows r0 + 32 i (i < T / 32) of channels c0 + 8 lr .. + 7
    const int lr = tid % 8, r0 = tid / 8, rp = T / kKvRows;
    const int64_t c = c0 + lr * 8;
    float w[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < rp) {
            const int r = r0 + kKvRows * i;
            load8<XT>(r == T - 1 ? kn + c : res + r * channels + c, w[i]);  // row T - 1 is the new key
        }
    float am[8], lo[8], hi[8];
    stats_init<SYM>(am, lo, hi, w[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        if (i < rp)
            stats_add<SYM>(am, lo, hi, w[i]);
    SegParams ps[8];
    tile_params<SYM, kKvCols>(am, lo, hi, tred, ps);
    const int64_t kb = b * (max_tokens / T) + p / T;
    if (r0 == 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            k_scales[kb * channels + c + j] = ps[j].st;
            if (!SYM)
                k_zeros[kb * channels + c + j] = (uint8_t)ps[j].z;
        }
    const int64_t first = p - (T - 1);  // the group's first token
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < rp)
            *reinterpret_cast<uint2 *>(k_codes + ((b * max_tokens + first + r0 + kKvRows * i) * channels + c)) =
                codes8(w[i], ps);
}

template <typename XT, bool SYM, int VG>
hipError_t append_go(const KvAppendArgs &a, hipStream_t st)
{
    k_kv_append<XT, SYM, VG><<<dim3((unsigned)a.batch, (unsigned)(a.channels / kKvCols)), dim3(kAppThreads), 0, st>>>(
        static_cast<const XT *>(a.k_new), static_cast<const XT *>(a.v_new), a.channels, a.positions, a.max_tokens,
        a.block_tokens, static_cast<XT *>(a.k_res), static_cast<int8_t *>(a.k_codes), a.k_scales, a.k_zeros,
        static_cast<int8_t *>(a.v_codes), a.v_scales, a.v_zeros);
    return hipGetLastError();
}

template <typename XT, bool SYM>
hipError_t append_vg(const KvAppendArgs &a, hipStream_t st)
{
    switch (a.v_group_size) {
    case 32:
        return append_go<XT, SYM, 32>(a, st);
    case 64:
        return append_go<XT, SYM, 64>(a, st);
    case 128:
        return append_go<XT, SYM, 128>(a, st);
    default:
        return append_go<XT, SYM, 0>(a, st);
    }
}

}  // namespace

hipError_t launch_kv_keys(const KvKeysArgs &a, hipStream_t st)
{
    if (a.x_bf16)
        return a.symmetric ? keys_go<uint16_t, true>(a, st) : keys_go<uint16_t, false>(a, st);
    return a.symmetric ? keys_go<float, true>(a, st) : keys_go<float, false>(a, st);
}

hipError_t launch_kv_dequant_keys(const KvKeysArgs &a, void *out, bool out_bf16, hipStream_t st)
{
    const int64_t n8 = a.tokens * a.channels / 8;
    const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 8192);
    const dim3 grid((unsigned)blocks), block(256);
    if (a.symmetric) {
        if (out_bf16)
            k_kv_dequant_keys<true, true><<<grid, block, 0, st>>>(a.codes, a.scales, a.zeros, a.tokens, a.channels,
                                                                  a.block_tokens, out);
        else
            k_kv_dequant_keys<true, false><<<grid, block, 0, st>>>(a.codes, a.scales, a.zeros, a.tokens, a.channels,
                                                                   a.block_tokens, out);
    } else {
        if (out_bf16)
            k_kv_dequant_keys<false, true><<<grid, block, 0, st>>>(a.codes, a.scales, a.zeros, a.tokens, a.channels,
                                                                   a.block_tokens, out);
        else
            k_kv_dequant_keys<false, false><<<grid, block, 0, st>>>(a.codes, a.scales, a.zeros, a.tokens, a.channels,
                                                                    a.block_tokens, out);
    }
    return hipGetLastError();
}

hipError_t launch_kv_append(const KvAppendArgs &a, hipStream_t st)
{
    if (a.x_bf16)
        return a.symmetric ? append_vg<uint16_t, true>(a, st) : append_vg<uint16_t, false>(a, st);
    return a.symmetric ? append_vg<float, true>(a, st) : append_vg<float, false>(a, st);
}

}  // namespace pqg
