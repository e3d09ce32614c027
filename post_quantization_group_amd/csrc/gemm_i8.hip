// gemm_i8.hip -- INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, with the W8A8 epilogue.
//
// acc[m, n] = sum_k a[m, k] * b[n, k]  (exact integer accumulation), then optionally
// y[m, n] = float(acc) * (s_x[m] * s_w[n])   ("第11章 模型量化与压缩" §11.4.5 step 6: INT8 GEMM, INT32
// accumulation, dequantized output; "模型压缩：量化、ZeroQuant、LLM.int8() 与 SmoothQuant" §11: one scale per
// row of the left operand and one per column of the right operand).
//
// Instruction. v_mfma_i32_32x32x32_i8 (32x32 output, 32 deep) sustains about twice the int8 rate of the
// 16x16x64 form on gfx950, so it is the building block. The weight tile is the MFMA "A" operand and the
// activation tile "B": lane l holds output column m = l % 32 and, in accumulator register r, output row
// n = 8 (r / 4) + 4 (l / 32) + r % 4, i.e. four consecutive output channels per group of four registers.
// The bf16 epilogue (when output rows are whole 16-byte chunks) stages the scaled tile in LDS and writes it back
// as 16-byte stores along output rows: the whole tile at once in the 128 x 128 and ring kernels, each wave's
// 32-row slices in the wide kernel; otherwise each group of four registers is one 16-byte (int32 / fp32) or
// 8-byte (bf16) store.
// Three kernels share this layout. With K % 64 == 0, the wide kernel at the end (256 x 384 tiles, one block
// of eight waves per CU) takes shapes whose tiles fill three quarters to all of the CUs in one round, and the
// ring kernel (256 x 128 tiles) other shapes with M >= 256; both load their operands straight into a
// three-stage LDS ring. The register-staged 128 x 128 kernel described next takes every other shape.
// Tiling.
//   block: BN (n) x BM (m) output tile, split into waves of WN x WM; K step of BK bytes (BK / 32 MFMA
//          depths; 64 or 128).
//   wave : (WN/32) x (WM/32) MFMA tiles; per K step 2 (WN/32 + WM/32) 16-byte fragment reads from LDS.
//   LDS  : two stages of [BN][BK] (weights) and [BM][BK] (activations) bytes, swizzled; the next K step's
//          global loads are in flight (in registers) while the current one is multiplied.
// A fragment of depth 32 at sub-step s is row l % 32, 16-byte piece 2 s + l / 32 of the 64-byte K slice
// for both operands, so the products pair up whatever k order the instruction uses internally.
// Blocks are dispatched round-robin over the 8 XCDs; block b is remapped so that each XCD walks a
// contiguous range of tiles, token tiles fastest, and its L2 keeps reusing the same weight tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;

// LDS offset of 16-byte piece c of tile row r, for rows of BK bytes (64 or 128). gfx950 LDS serves a
// 128-bit access over 64 banks of 4 bytes, 16 lanes per cycle: writes take 16 consecutive lanes (whole
// rows of consecutive pieces); reads take lanes 0-7 with 16-23, 8-15 with 24-31, and so on, which for a
// 32-row fragment means 16 rows r .. r + 7, r + 16 .. r + 23 reading the same piece. An xor of the piece
// index with bits of the row spreads those rows over all 16 bank quads:
//   64-byte rows (4 pieces, 4 rows share a bank pattern mod 256 B): row bits 2 and 4;
//   128-byte rows (8 pieces, 2 rows per 256 B): row bits 1, 2 and 4.
template <int BK>
__device__ __forceinline__ int lds_off(int r, int c)
{
    if (BK == 64)
        return r * BK + 16 * (c ^ (((r >> 2) & 1) | ((r >> 3) & 2)));
    return r * BK + 16 * (c ^ (((r >> 1) & 3) | ((r >> 2) & 4)));
}

// Epilogue for four consecutive output channels nb .. nb + 3 at token m, with their weight scales sw[0..3]
// (unused for MODE 0).
template <int MODE>
__device__ __forceinline__ void store4s(const int v[4], int64_t m, int64_t nb, int64_t M, int64_t N, float sxm,
                                        const float sw[4], void *__restrict__ c, bool vec_ok)
{
    if (m >= M)
        return;
    if (MODE == 0) {
        int32_t *out = static_cast<int32_t *>(c) + m * N + nb;
        if (vec_ok && nb + 3 < N) {
            *reinterpret_cast<v4i *>(out) = v4i{v[0], v[1], v[2], v[3]};
        } else {
            for (int r = 0; r < 4; ++r)
                if (nb + r < N)
                    out[r] = v[r];
        }
        return;
    }
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        f[r] = (float)v[r] * (sxm * sw[r]);
    if (MODE == 1) {
        uint16_t *out = static_cast<uint16_t *>(c) + m * N + nb;
        if (vec_ok && nb + 3 < N) {
            *reinterpret_cast<uint2 *>(out) = make_uint2(pack_bf16x2_rne(f[0], f[1]), pack_bf16x2_rne(f[2], f[3]));
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

// The same with the weight scales read from sb (zero past N).
template <int MODE>
__device__ __forceinline__ void store4(const int v[4], int64_t m, int64_t nb, int64_t M, int64_t N, float sxm,
                                       const float *__restrict__ sb, void *__restrict__ c, bool vec_ok)
{
    float sw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (MODE != 0)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sw[r] = (nb + r < N) ? sb[nb + r] : 0.0f;
    store4s<MODE>(v, m, nb, M, N, sxm, sw, c, vec_ok);
}

template <int BN, int BM, int WN, int WM, int BK, int MODE>  // MODE 0: raw int32, 1: bf16, 2: fp32 epilogue
__global__ __launch_bounds__((BN / WN) * (BM / WM) * 64) void k_gemm_i8(
    const int8_t *__restrict__ a, const int8_t *__restrict__ b, int64_t M, int64_t N, int64_t K,
    const float *__restrict__ sa, const float *__restrict__ sb, void *__restrict__ c, int tiles)
{
    constexpr int NT = (BN / WN) * (BM / WM) * 64;  // threads
    constexpr int TN = WN / 32, TM = WM / 32;
    constexpr int NP = BK / 16;                          // 16-byte pieces per tile row
    constexpr int WP = BN * NP, XP = BM * NP;            // pieces per K step
    constexpr int WLOADS = (WP + NT - 1) / NT;            // per thread
    constexpr int XLOADS = (XP + NT - 1) / NT;
    // operand stages; after the main loop the same memory stages the bf16 output tile
    constexpr int kSmem = 2 * (BN + BM) * BK;
    static_assert(kSmem >= BM * BN * 2, "the output tile must fit in the operand stages");
    __shared__ __attribute__((aligned(16))) int8_t smem[kSmem];
    int8_t(*sW)[BN * BK] = reinterpret_cast<int8_t(*)[BN * BK]>(smem);
    int8_t(*sX)[BM * BK] = reinterpret_cast<int8_t(*)[BM * BK]>(smem + 2 * BN * BK);

    // XCD-aware tile order: XCD x = blockIdx % 8 takes tiles [x * per, (x + 1) * per)
    const int per = (tiles + kXcds - 1) / kXcds;
    const int t = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (t >= tiles)
        return;
    const int m_tiles = (int)((M + BM - 1) / BM);
    const int64_t n0 = (int64_t)(t / m_tiles) * BN;
    const int64_t m0 = (int64_t)(t % m_tiles) * BM;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int wn = wv % (BN / WN), wm = wv / (BN / WN);

    // global -> LDS assignment: piece p = tid + NT i -> row p / NP, 16-byte piece p % NP of the K slice
    auto load_tiles = [&](int64_t k0, uint4 rw[WLOADS], uint4 rx[XLOADS]) {
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const int p = tid + NT * i;
            const int64_t nr = n0 + p / NP, kk = k0 + (p % NP) * 16;
            rw[i] = (p < WP && nr < N && kk < K) ? *reinterpret_cast<const uint4 *>(b + nr * K + kk)
                                                 : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            const int p = tid + NT * i;
            const int64_t mr = m0 + p / NP, kk = k0 + (p % NP) * 16;
            rx[i] = (p < XP && mr < M && kk < K) ? *reinterpret_cast<const uint4 *>(a + mr * K + kk)
                                                 : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tiles = [&](int st, const uint4 rw[WLOADS], const uint4 rx[XLOADS]) {
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const int p = tid + NT * i;
            if (p < WP)
                *reinterpret_cast<uint4 *>(&sW[st][lds_off<BK>(p / NP, p % NP)]) = rw[i];
        }
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            const int p = tid + NT * i;
            if (p < XP)
                *reinterpret_cast<uint4 *>(&sX[st][lds_off<BK>(p / NP, p % NP)]) = rx[i];
        }
    };

    v16i acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    uint4 rw[WLOADS], rx[XLOADS];
    load_tiles(0, rw, rx);
    store_tiles(0, rw, rx);
    __syncthreads();

    const int frow = lane % 32;
    const int fhalf = lane / 32;
    const int nsteps = (int)((K + BK - 1) / BK);
    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        if (step + 1 < nsteps)
            load_tiles((int64_t)(step + 1) * BK, rw, rx);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            v4i fb[TM];
#pragma unroll
            for (int j = 0; j < TM; ++j)
                fb[j] = *reinterpret_cast<const v4i *>(&sX[cur][lds_off<BK>(wm * WM + j * 32 + frow, 2 * s + fhalf)]);
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const v4i fa =
                    *reinterpret_cast<const v4i *>(&sW[cur][lds_off<BK>(wn * WN + i * 32 + frow, 2 * s + fhalf)]);
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[j], acc[i][j], 0, 0, 0);
            }
        }
        if (step + 1 < nsteps)
            store_tiles(cur ^ 1, rw, rx);
        __syncthreads();
    }

    // epilogue: register group g (4 registers) of a 32x32 tile holds rows 8 g + 4 (lane / 32) + 0..3 at
    // token column lane % 32.
    // bf16 output with 16-byte aligned rows: the scaled tile goes through LDS ([token][channel], 16-byte
    // chunks xor-swizzled by the token's low four bits) and leaves as 16-byte stores, four full 256-byte
    // rows per wave instruction. Written directly, each store would cover 16 bytes in each of 32 rows.
    if (MODE == 1 && (N % 8) == 0 && (reinterpret_cast<uintptr_t>(c) % 16) == 0) {
        constexpr int ROWB = BN * 2;  // bytes of one staged token row
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int ml = wm * WM + j * 32 + frow;
            const int64_t m = m0 + ml;
            const float sxm = m < M ? sa[m] : 0.0f;
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * WN + i * 32 + 8 * g + 4 * fhalf;
                    const int64_t nb = n0 + nl;
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float swn = (nb + r < N) ? sb[nb + r] : 0.0f;
                        f[r] = (float)acc[i][j][4 * g + r] * (sxm * swn);
                    }
                    const int chunk = (nl * 2 / 16) ^ (ml & 15);
                    *reinterpret_cast<uint2 *>(smem + ml * ROWB + chunk * 16 + (nl * 2) % 16) =
                        make_uint2(pack_bf16x2_rne(f[0], f[1]), pack_bf16x2_rne(f[2], f[3]));
                }
        }
        __syncthreads();
        constexpr int CHUNKS = BM * ROWB / 16;  // 16-byte chunks of the tile
        uint16_t *y = static_cast<uint16_t *>(c);
#pragma unroll
        for (int q = tid; q < CHUNKS; q += NT) {
            const int ml = q / (ROWB / 16), cl = q % (ROWB / 16);
            const int64_t m = m0 + ml, nb = n0 + cl * 8;
            if (m < M && nb < N) {
                const uint4 v = *reinterpret_cast<const uint4 *>(smem + ml * ROWB + ((cl ^ (ml & 15)) * 16));
                *reinterpret_cast<uint4 *>(y + m * N + nb) = v;  // N % 8 == 0: a chunk never crosses N
            }
        }
        return;
    }
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(c) % (MODE == 1 ? 8 : 16)) == 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int64_t m = m0 + wm * WM + j * 32 + frow;
        const float sxm = (MODE == 0 || m >= M) ? 0.0f : sa[m];
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                const int64_t nb = n0 + wn * WN + i * 32 + 8 * g + 4 * fhalf;
                store4<MODE>(v, m, nb, M, N, sxm, sb, c, vec_ok);
            }
    }
}

template <int BN, int BM, int WN, int WM, int BK = 64>
hipError_t gemm_launch(const GemmI8Args &g, hipStream_t st)
{
    constexpr int NT = (BN / WN) * (BM / WM) * 64;
    const int64_t tiles = ((g.N + BN - 1) / BN) * ((g.M + BM - 1) / BM);
    const int64_t per = (tiles + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per * kXcds)), block(NT);
    if (g.sa == nullptr)
        k_gemm_i8<BN, BM, WN, WM, BK, 0><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, nullptr, nullptr, g.c, (int)tiles);
    else if (g.c_bf16)
        k_gemm_i8<BN, BM, WN, WM, BK, 1><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    else
        k_gemm_i8<BN, BM, WN, WM, BK, 2><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    return hipGetLastError();
}

// ------------------------------------------------------------------ ring kernel (K % 64 == 0, M >= 256)
//
// 256 (m) x 128 (n) block tile, four waves of 128 (m) x 64 (n), 64-byte K steps. Operands go global -> LDS
// with direct loads (global_load_lds_dwordx4: no registers, no LDS store instructions) into a ring of three
// stages. At step k the block issues the loads of step k + 2, multiplies stage k, and then waits only for
// the loads of step k + 1 (issued one step earlier) before the barrier, so a barrier never drains the loads
// of the step after next. The three stages are separate LDS arrays, which lets the compiler see that the
// direct loads into one stage cannot alias the fragment reads of another (it would otherwise wait for
// every outstanding direct load before each read).
//   * A direct load writes lane l's 16 bytes to LDS at (base + 16 l): each instruction fills 64 consecutive
//     16-byte slots. The xor swizzle of the LDS layout is applied on the source side: slot (row, physical
//     piece p) is filled from logical piece p ^ swizzle(row) of that row.
//   * The larger tile halves the LDS bytes read per MFMA against 128 x 128 tiles with 32 x 64 wave tiles,
//     and 2048 x 11008 gives 688 tiles (2.7 rounds on 256 CUs). Two blocks fit per CU (72 KB of LDS each).
//   * bf16 output goes through the idle stages like the 128 x 128 kernel's epilogue.
constexpr int kRingBM = 256, kRingBN = 128, kRingWM = 128, kRingWN = 64, kRingBK = 64;
constexpr int kRingWaves = (kRingBM / kRingWM) * (kRingBN / kRingWN);
constexpr int kRingThreads = kRingWaves * kWave;
constexpr int kRingStage = (kRingBM + kRingBN) * kRingBK;    // bytes: [BM][64] activations, [BN][64] weights
constexpr int kRingLoads = kRingStage / 16 / kRingThreads;    // direct loads per thread per step
static_assert(kRingStage % (16 * kRingThreads) == 0, "each thread issues whole loads");


template <int MODE>
__global__ __launch_bounds__(kRingThreads, 2) void k_gemm_i8_ring(const int8_t *__restrict__ a,
                                                                 const int8_t *__restrict__ b, int64_t M,
                                                                 int64_t N, int64_t K, const float *__restrict__ sa,
                                                                 const float *__restrict__ sb, void *__restrict__ c,
                                                                 int tiles)
{
    constexpr int BM = kRingBM, BN = kRingBN, BK = kRingBK, WM = kRingWM, WN = kRingWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int XBYTES = BM * BK;
    __shared__ __attribute__((aligned(16))) int8_t s0[kRingStage];
    __shared__ __attribute__((aligned(16))) int8_t s1[kRingStage];
    __shared__ __attribute__((aligned(16))) int8_t s2[kRingStage];

    const int per = (tiles + kXcds - 1) / kXcds;  // XCD x takes tiles [x per, (x + 1) per)
    const int t = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (t >= tiles)
        return;
    const int m_tiles = (int)((M + BM - 1) / BM);
    const int64_t n0 = (int64_t)(t / m_tiles) * BN;
    const int64_t m0 = (int64_t)(t % m_tiles) * BM;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = w % (BM / WM), wn = w / (BM / WM);
    const int fr = lane % 32, fh = lane / 32;

    // direct-load sources: instruction i of wave w fills slots (i * waves + w) * 64 + lane of a stage; slot
    // P holds row P / 4 (activation rows first, then weight rows), physical piece P % 4
    const int8_t *src[kRingLoads];
    int lofs[kRingLoads];
#pragma unroll
    for (int i = 0; i < kRingLoads; ++i) {
        const int S0 = (i * kRingWaves + w) * kWave;
        const int P = S0 + lane;
        const bool isx = P < BM * 4;
        const int q = isx ? P : P - BM * 4;
        const int r = q >> 2;
        const int logical = (q & 3) ^ (((r >> 2) & 1) | ((r >> 3) & 2));  // inverse of lds_off<64>'s swizzle
        if (isx)
            src[i] = a + std::min<int64_t>(m0 + r, M - 1) * K + 16 * logical;
        else
            src[i] = b + std::min<int64_t>(n0 + r, N - 1) * K + 16 * logical;
        lofs[i] = S0 * 16;
    }
    const int nsteps = (int)(K / BK);
    auto issue = [&](int8_t *stage, int k) {
        const int64_t kk = (int64_t)(k < nsteps ? k : nsteps - 1) * BK;  // past the end: reload the last step
#pragma unroll
        for (int i = 0; i < kRingLoads; ++i)
            __builtin_amdgcn_global_load_lds((global_void_t *)(src[i] + kk), (lds_void_t *)(stage + lofs[i]), 16, 0, 0);
    };

    v16i acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    auto multiply = [&](const int8_t *xs) {
        const int8_t *ws = xs + XBYTES;
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            v4i fx[TM], fw[TN];
#pragma unroll
            for (int j = 0; j < TM; ++j)
                fx[j] = *reinterpret_cast<const v4i *>(xs + lds_off<64>(wm * WM + j * 32 + fr, 2 * s + fh));
#pragma unroll
            for (int i = 0; i < TN; ++i)
                fw[i] = *reinterpret_cast<const v4i *>(ws + lds_off<64>(wn * WN + i * 32 + fr, 2 * s + fh));
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i], fx[j], acc[i][j], 0, 0, 0);
        }
    };
    auto step = [&](int8_t *cur, int8_t *after_next, int k) {
        issue(after_next, k + 2);
        multiply(cur);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kRingLoads, 0));  // step k + 1 landed, fragment reads done
        __builtin_amdgcn_s_barrier();
    };

    issue(s0, 0);
    issue(s1, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kRingLoads, 15));
    __builtin_amdgcn_s_barrier();
    int k = 0;
    for (; k + 3 <= nsteps; k += 3) {
        step(s0, s2, k);
        step(s1, s0, k + 1);
        step(s2, s1, k + 2);
    }
    if (k < nsteps)
        step(s0, s2, k);
    if (k + 1 < nsteps)
        step(s1, s0, k + 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // no direct load may land in the stages reused below

    if (MODE == 1 && (N % 8) == 0 && (reinterpret_cast<uintptr_t>(c) % 16) == 0) {
        // bf16 tile staged as [token][channel] rows of 256 bytes over the three stages (96 rows each)
        constexpr int ROWB = BN * 2, RPS = kRingStage / ROWB;
        static_assert(3 * RPS >= BM, "the output tile fits in the stages");
        auto rowp = [&](int ml) -> int8_t * {
            return ml < RPS ? s0 + ml * ROWB : ml < 2 * RPS ? s1 + (ml - RPS) * ROWB : s2 + (ml - 2 * RPS) * ROWB;
        };
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int ml = wm * WM + j * 32 + fr;
            const int64_t m = m0 + ml;
            const float sxm = m < M ? sa[m] : 0.0f;
            int8_t *rp = rowp(ml);
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * WN + i * 32 + 8 * g + 4 * fh;
                    const int64_t nb = n0 + nl;
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float swn = (nb + r < N) ? sb[nb + r] : 0.0f;
                        f[r] = (float)acc[i][j][4 * g + r] * (sxm * swn);
                    }
                    const int chunk = (nl * 2 / 16) ^ (ml & 15);
                    *reinterpret_cast<uint2 *>(rp + chunk * 16 + (nl * 2) % 16) =
                        make_uint2(pack_bf16x2_rne(f[0], f[1]), pack_bf16x2_rne(f[2], f[3]));
                }
        }
        __syncthreads();
        constexpr int CPR = ROWB / 16;
        uint16_t *y = static_cast<uint16_t *>(c);
        for (int q = tid; q < BM * CPR; q += kRingThreads) {
            const int ml = q / CPR, cl = q % CPR;
            const int64_t m = m0 + ml, nb = n0 + cl * 8;
            if (m < M && nb < N)  // N % 8 == 0: a chunk never crosses N
                *reinterpret_cast<uint4 *>(y + m * N + nb) =
                    *reinterpret_cast<const uint4 *>(rowp(ml) + ((cl ^ (ml & 15)) * 16));
        }
        return;
    }
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(c) % (MODE == 1 ? 8 : 16)) == 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int64_t m = m0 + wm * WM + j * 32 + fr;
        const float sxm = (MODE == 0 || m >= M) ? 0.0f : sa[m];
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                store4<MODE>(v, m, n0 + wn * WN + i * 32 + 8 * g + 4 * fh, M, N, sxm, sb, c, vec_ok);
            }
    }
}

hipError_t ring_launch(const GemmI8Args &g, hipStream_t st)
{
    const int64_t tiles = ((g.N + kRingBN - 1) / kRingBN) * ((g.M + kRingBM - 1) / kRingBM);
    const int64_t per = (tiles + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per * kXcds)), block(kRingThreads);
    if (g.sa == nullptr)
        k_gemm_i8_ring<0><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, nullptr, nullptr, g.c, (int)tiles);
    else if (g.c_bf16)
        k_gemm_i8_ring<1><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    else
        k_gemm_i8_ring<2><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    return hipGetLastError();
}

// ------------------------------------------------------------------ wide kernel (one round of 256 x 384 tiles)
//
// Measured on the ring kernel: with its 256 x 128 tile a CU must bring in 384 bytes per K byte for 32K
// multiply-adds, about 47 B/clk at the int8 matrix-core rate, and it gets 20-27 B/clk from L2 under full
// load; the same ring with all blocks reading one L2-resident tile was hardly faster, so the limit is the
// per-CU path (direct loads into LDS plus the fragment reads out of it), not DRAM or L2 misses.
//   * A 256 (m) x 384 (n) tile loads 640 bytes per K byte for 96K multiply-adds (about 27 B/clk at full
//     rate), and 2048 x 11008 becomes 8 x 29 = 232 tiles: one round on 256 CUs instead of the ring
//     kernel's 688 tiles on 512 block slots.
//   * One block of eight waves per CU, each wave 128 (m) x 96 (n) = 4 x 3 MFMA tiles (192 accumulator
//     registers; four waves of 128 x 192 would need 384 and the compiler spills them).
//   * 64-byte K steps in a three-stage direct-to-LDS ring (3 x 40 KB), loads two steps ahead, as in the
//     ring kernel. Stages are separate LDS blocks so that the compiler can tell a direct load into one
//     stage from the fragment reads of another.
//   * Ping-pong schedule. Waves w and w + 4 share a SIMD; waves 0-3 form group 0 and waves 4-7 group 1,
//     and group 1 runs one barrier behind group 0. Each 32-deep sub-step is a memory phase (the direct
//     loads two steps ahead at the first sub-step of a step, the wave's seven 16-byte fragment reads, and
//     the wait for them) and a compute phase (its 12 MFMAs), each ended by a block barrier. So while one
//     group's MFMAs run, the other group's fragment reads are in flight, and every SIMD always has a wave
//     with operands in registers. With the epilogue below, the compiler's own interleaving of reads and
//     MFMAs took 89.5-94 us on the 2048 x 11008 x 4096 layer, the ping-pong 87-90 us; with both groups in
//     step (the same phases, no offset) it took 116 us (stores straight from the accumulators). Raising the
//     compute phase's wave priority made no difference. A memory phase moves 28 KB of fragments
//     through the LDS for 384 cycles of MFMA per SIMD, so it is as long as the compute phase: the loop runs
//     about 1.25 x the time of its MFMAs alone.
//   * The tile's 384 weight and 256 token scales are loaded straight into LDS (640 floats) before the ring
//     starts, so the epilogue reads each group of four weight scales with one LDS read.
//   * bf16 epilogue: each wave passes every 32-row slice of its 128 x 96 tile through a wave-private LDS
//     buffer (the ring stages, free by then) and writes it back as 16-byte stores along rows, 192-byte runs
//     per row. The store phase of the one round is exposed (nothing else runs then): 45 MB of bf16 output
//     took 15-17 us as 8-byte stores straight from the accumulators (16-byte pieces of 32 rows per
//     instruction) and takes 6 us this way (2048 x 11008 x 4096: 98-100 us -> 87-90 us, bit-identical).
//     int32 and fp32 outputs, and bf16 outputs whose rows are not whole 16-byte chunks, keep the stores
//     straight from the accumulators.
//   * Operand loads carry the sc0 cache-policy bit (3 % faster with the compiler-interleaved loop, no
//     difference with the ping-pong; sc1 or both were slower).
// Taken when its tiles fill between three quarters and all of the CUs in a single round; otherwise the
// ring kernel (more, smaller tiles) balances better.
constexpr int kWideBM = 256, kWideBN = 384, kWideWM = 128, kWideWN = 96, kWideBK = 64;
constexpr int kLoadSc0 = 1;  // cache-policy bits of the wide kernel's direct operand loads: sc0
constexpr int kWideWaves = (kWideBM / kWideWM) * (kWideBN / kWideWN);
constexpr int kWideThreads = kWideWaves * kWave;
constexpr int kWideStage = (kWideBM + kWideBN) * kWideBK;         // 40960 bytes
constexpr int kWideLoads = kWideStage / 16 / kWideThreads;         // 5 direct loads per thread per step
constexpr int kWideALoads = kWideBM * kWideBK / 16 / kWideThreads;  // the first 2 fill activation rows
constexpr int kWideStagePitch = 208;  // bytes per row of a wave's 32 x 96 bf16 epilogue slice (192 + 16)
static_assert(kWideStage % (16 * kWideThreads) == 0 && (kWideBM * kWideBK) % (16 * kWideThreads) == 0,
              "each load instruction fills whole rows of one operand");
static_assert(kWideWaves == 8, "the ping-pong schedule pairs waves w and w + 4");
static_assert(6 * 32 * kWideStagePitch <= kWideStage && 2 * 32 * kWideStagePitch <= kWideStage,
              "six waves' epilogue slices fit in stage 0, two in stage 1");


template <int MODE>
__global__ __launch_bounds__(kWideThreads, 1) void k_gemm_i8_wide(const int8_t *__restrict__ a,
                                                                 const int8_t *__restrict__ b, int64_t M,
                                                                 int64_t N, int64_t K, const float *__restrict__ sa,
                                                                 const float *__restrict__ sb, void *__restrict__ c,
                                                                 int tiles)
{
    constexpr int BM = kWideBM, BN = kWideBN, WM = kWideWM, WN = kWideWN, BK = kWideBK;
    constexpr int TM = WM / 32, TN = WN / 32, PPR = BK / 16;
    int8_t *const s0 = lds_block<kWideStage, 0>();
    int8_t *const s1 = lds_block<kWideStage, 1>();
    int8_t *const s2 = lds_block<kWideStage, 2>();

    const int per = (tiles + kXcds - 1) / kXcds;  // XCD x takes tiles [x per, (x + 1) per)
    const int t = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (t >= tiles)
        return;
    const int m_tiles = (int)((M + BM - 1) / BM);
    const int64_t n0 = (int64_t)(t / m_tiles) * BN;
    const int64_t m0 = (int64_t)(t % m_tiles) * BM;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int grp = w / 4;  // ping-pong group
    const int wm = w % (BM / WM), wn = w / (BM / WM);
    const int fr = lane % 32, fh = lane / 32;

    // direct-load sources as 32-bit offsets from the tile's first rows: instruction i of wave w fills slots
    // (i * waves + w) * 64 + lane; slot P holds row P / 4 (activation rows first), physical piece P % 4
    const int8_t *abase = a + m0 * K;
    const int8_t *bbase = b + n0 * K;
    uint32_t off[kWideLoads];
#pragma unroll
    for (int i = 0; i < kWideLoads; ++i) {
        const int P = (i * kWideWaves + w) * kWave + lane;
        const bool isx = i < kWideALoads;
        const int q = isx ? P : P - BM * PPR;
        const int r = q / PPR;
        const int logical = (q % PPR) ^ (((r >> 2) & 1) | ((r >> 3) & 2));  // inverse of lds_off<64>'s swizzle
        const int64_t rr = isx ? std::min<int64_t>(r, M - 1 - m0) : std::min<int64_t>(r, N - 1 - n0);
        off[i] = (uint32_t)(rr * K + 16 * logical);
    }
    const int nsteps = (int)(K / BK);
    auto issue = [&](int8_t *stage, int k) __attribute__((always_inline)) {
        const uint32_t kk = (uint32_t)(k < nsteps ? k : nsteps - 1) * BK;  // past the end: reload the last step
#pragma unroll
        for (int i = 0; i < kWideLoads; ++i)
            __builtin_amdgcn_global_load_lds((global_void_t *)((i < kWideALoads ? abase : bbase) + (off[i] + kk)),
                                             (lds_void_t *)(stage + (i * kWideWaves + w) * kWave * 16), 16, 0,
                                             kLoadSc0);
    };

    v16i acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // A block barrier that no instruction is scheduled across (the phases must stay where they are written).
    auto phase_end = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Sub-step s of step k on stage xs. Hazards of the ring, with every wave passing the same barriers:
    //   * the loads for step k + 2 overwrite the stage of step k - 1, whose last fragment reads (sub-step 1
    //     of step k - 1) every wave finished (its lgkmcnt wait) before a barrier that precedes this issue;
    //   * step k + 1's stage is read from the first sub-step of step k + 1 on; each wave waits for its own
    //     loads of step k + 1 (all but the 5 just issued) in this memory phase, before two more barriers.
    auto substep = [&](const int8_t *xs, int8_t *after_next, int k, int s) __attribute__((always_inline)) {
        const int8_t *ws = xs + BM * BK;
        if (s == 0)
            issue(after_next, k + 2);
        v4i fx[TM], fw[TN];
#pragma unroll
        for (int j = 0; j < TM; ++j)
            fx[j] = *reinterpret_cast<const v4i *>(xs + lds_off<64>(wm * WM + j * 32 + fr, 2 * s + fh));
#pragma unroll
        for (int i = 0; i < TN; ++i)
            fw[i] = *reinterpret_cast<const v4i *>(ws + lds_off<64>(wn * WN + i * 32 + fr, 2 * s + fh));
        if (s == 0)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(kWideLoads, 0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        phase_end();
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i], fx[j], acc[i][j], 0, 0, 0);
        phase_end();
    };
    auto step = [&](int8_t *cur, int8_t *after_next, int k) __attribute__((always_inline)) {
        substep(cur, after_next, k, 0);
        substep(cur, after_next, k, 1);
    };

    // The tile's scales, straight into LDS before the ring starts: BN weight scales, then BM token scales (rows
    // past N or M repeat the last one; their outputs are never stored). They land long before the epilogue.
    float *const lsc = reinterpret_cast<float *>(lds_block<(BN + BM) * 4, 3>());
    if (MODE != 0) {
        for (int base = w * kWave; base < BN + BM; base += kWideThreads) {
            const int idx = base + lane;
            const float *src = idx < BN ? sb + std::min<int64_t>(n0 + idx, N - 1)
                                        : sa + std::min<int64_t>(m0 + (idx - BN), M - 1);
            if (idx < BN + BM)
                __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)(lsc + base), 4, 0, 0);
        }
    }
    issue(s0, 0);
    issue(s1, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kWideLoads, 15));
    __builtin_amdgcn_s_barrier();
    // group 1 starts one barrier late and group 0 ends with one more, so both pass the same number
    if (grp == 1)
        phase_end();
    int k = 0;
    for (; k + 3 <= nsteps; k += 3) {
        step(s0, s2, k);
        step(s1, s0, k + 1);
        step(s2, s1, k + 2);
    }
    if (k < nsteps)
        step(s0, s2, k);
    if (k + 1 < nsteps)
        step(s1, s0, k + 1);
    if (grp == 0)
        phase_end();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // no direct load may land in the stages reused below

    __syncthreads();  // every wave's scale loads have landed (each waited for its own above)
    if (MODE == 1 && (N % 8) == 0 && (reinterpret_cast<uintptr_t>(c) % 16) == 0) {
        int8_t *const wbuf = w < 6 ? s0 + w * 32 * kWideStagePitch : s1 + (w - 6) * 32 * kWideStagePitch;
        uint16_t *const y = static_cast<uint16_t *>(c);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int ml = wm * WM + j * 32 + fr;
            const float sxm = lsc[BN + ml];
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int cl = i * 32 + 8 * g + 4 * fh;  // column within the wave's 96
                    const float4 s4 = *reinterpret_cast<const float4 *>(lsc + wn * WN + cl);
                    const float f0 = (float)acc[i][j][4 * g] * (sxm * s4.x);
                    const float f1 = (float)acc[i][j][4 * g + 1] * (sxm * s4.y);
                    const float f2 = (float)acc[i][j][4 * g + 2] * (sxm * s4.z);
                    const float f3 = (float)acc[i][j][4 * g + 3] * (sxm * s4.w);
                    *reinterpret_cast<uint2 *>(wbuf + fr * kWideStagePitch + cl * 2) =
                        make_uint2(pack_bf16x2_rne(f0, f1), pack_bf16x2_rne(f2, f3));
                }
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            // 32 rows x 12 chunks of 16 bytes; N % 8 == 0, so a chunk is wholly inside or outside N
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int q = lane + kWave * u, row = q / 12, ch = q % 12;
                const v4i v = *reinterpret_cast<const v4i *>(wbuf + row * kWideStagePitch + ch * 16);
                const int64_t m = m0 + wm * WM + j * 32 + row, n = n0 + wn * WN + ch * 8;
                if (m < M && n < N)
                    *reinterpret_cast<v4i *>(y + m * N + n) = v;
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // the slice is read out before the next overwrites it
        }
        return;
    }
    const bool vec_ok = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(c) % (MODE == 1 ? 8 : 16)) == 0;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int ml = wm * WM + j * 32 + fr;
        const float sxm = MODE == 0 ? 0.0f : lsc[BN + ml];
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * WN + i * 32 + 8 * g + 4 * fh;
                float sw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (MODE != 0) {
                    const float4 s4 = *reinterpret_cast<const float4 *>(lsc + nl);
                    sw[0] = s4.x;
                    sw[1] = s4.y;
                    sw[2] = s4.z;
                    sw[3] = s4.w;
                }
                const int v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                store4s<MODE>(v, m0 + ml, n0 + nl, M, N, sxm, sw, c, vec_ok);
            }
    }
}

inline int64_t wide_tiles(const GemmI8Args &g)
{
    return ((g.N + kWideBN - 1) / kWideBN) * ((g.M + kWideBM - 1) / kWideBM);
}

hipError_t wide_launch(const GemmI8Args &g, hipStream_t st)
{
    const int64_t tiles = wide_tiles(g);
    const int64_t per = (tiles + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per * kXcds)), block(kWideThreads);
    if (g.sa == nullptr)
        k_gemm_i8_wide<0><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, nullptr, nullptr, g.c, (int)tiles);
    else if (g.c_bf16)
        k_gemm_i8_wide<1><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    else
        k_gemm_i8_wide<2><<<grid, block, 0, st>>>(g.a, g.b, g.M, g.N, g.K, g.sa, g.sb, g.c, (int)tiles);
    return hipGetLastError();
}

// Both direct-load kernels need whole 64-byte K steps. The wide kernel is taken when its 256 x 384 tiles
// fill at least three quarters of the CUs in one round; the ring kernel once there are full 256-token tiles.
constexpr int kCus = 256;

hipError_t launch_gemm_i8(const GemmI8Args &g, hipStream_t st)
{
    if (g.K % kWideBK == 0) {
        const int64_t wt = wide_tiles(g);
        if (wt >= kCus * 3 / 4 && wt <= kCus)
            return wide_launch(g, st);
    }
    if (g.K % kRingBK == 0 && g.M >= kRingBM)
        return ring_launch(g, st);
    return gemm_launch<128, 128, 32, 64, 64>(g, st);
}

}  // namespace pqg
