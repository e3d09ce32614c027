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
// m = 8 (r / 4) + 4 (l / 32) + r % 4. A lane therefore needs one weight scale (and zero point) per group,
// whatever r.
//
// What bounds it. Every group ends in a fold: each int32 accumulator is converted to fp32 and added with its
// group scale, two VALU instructions per accumulator per group. At g = 128 that is as many VALU cycles as
// the group's MFMA cycles (a wave64 VALU instruction takes 4 cycles, an int8 32x32x32 MFMA 32), so the
// kernel is built to spend as little VALU as possible elsewhere:
//   * Symmetric codes (two's complement nibbles) are unpacked by moving each nibble to the top of its byte:
//     the byte then reads as 16 q, so the MFMA sums 16x the exact integer, and the factor 1/16 is applied
//     with the token scale at the end (a power of two: the fp32 results are those of unscaled sums). Per
//     4-byte word (8 codes): one shift, two v_perm, two masks.
//   * Asymmetric codes: the nibbles are masked into bytes biased by 0x80, put in code order with v_perm, and
//     the zero point is subtracted from all four bytes at once (each byte is >= 0x80 > z, so no borrow
//     crosses a byte); removing the bias leaves the signed byte q - z in [-15, 15].
//   * A wave computes 128 tokens x 32 channels (four MFMA tiles share each unpacked weight operand).
//   * The folds are software-pipelined against the MFMAs (see multiply below), so that the VALU converts
//     one tile while the matrix core multiplies another, instead of each fold waiting for its MFMAs.
// Which codes one MFMA sums is free as long as A and B agree; what matters is that every MFMA lies inside one
// group. A step's 128 codes are two pairs of 64 codes, each pair two MFMAs. For g = 64 and 128 a pair lies
// inside one group and lane half h takes the pair's codes 32 h .. 32 h + 31 (one 16-byte read of packed
// codes, 16 codes per MFMA); for g = 32 each MFMA must be one group of 32 consecutive codes, so lane half h
// takes its codes 16 h .. 16 h + 15 (an 8-byte read per MFMA). The int32 accumulators of a group start from
// zero (the MFMA's C operand) and are folded after the group's last MFMA.
// Tiling and feed: 128 (m) x 128 (n) block tile, four waves side by side along n, K steps of 128 codes; tiles are
// taken in groups of four token tiles (below).
// Operands go global -> LDS with direct loads (no registers, no LDS store instructions) into a ring of three
// stages, as in the INT8 GEMM's ring kernel: step k issues the loads of step k + 2, multiplies stage k and
// waits only for the loads of step k + 1. The group scales of step k + 1 are loaded into registers just
// before those direct loads, so waiting for all but the last six loads also covers them. The epilogue stages
// the unscaled fp32 tile in the idle stages and writes 16-byte chunks of output rows with the token scale.
#include "common.hpp"
#include "kernels.hpp"

namespace pqg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kW8Xcds = 8;
constexpr int kBM = 128, kBN = 128, kBK = 128;  // tokens x channels per block, codes per K step
constexpr int kWaves = 4, kThreads = kWaves * kWave;
constexpr int kWN = kBN / kWaves;                // 32 channels per wave
constexpr int kTM = kBM / 32;                    // 4 token tiles per wave
constexpr int kXRow = kBK, kWRow = kBK / 2;      // bytes per staged row
constexpr int kXBytes = kBM * kXRow;             // 16384
constexpr int kStage = kXBytes + kBN * kWRow;    // 24576
constexpr int kLoads = kStage / 16 / kThreads;   // 6 direct loads per thread per step
constexpr int kXLoads = kXBytes / 16 / kThreads; // the first 4 fill activation rows
static_assert(kLoads * 16 * kThreads == kStage && kXLoads * 16 * kThreads == kXBytes, "whole loads");
static_assert(kWN == 32, "one MFMA tile of channels per wave");

// LDS offset of 16-byte piece c of a staged row r: rows of 128 bytes (activations) and 64 bytes (packed
// weights). The piece index is xor-ed with row bits so that the 16 rows read together by one half of a
// wave fall into different bank quads. Both swizzles are their own inverse.
__device__ __forceinline__ int xsw(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }
__device__ __forceinline__ int wsw(int r) { return ((r >> 2) & 1) | ((r >> 3) & 2); }
__device__ __forceinline__ int xoff(int r, int c) { return r * kXRow + 16 * (c ^ xsw(r)); }
__device__ __forceinline__ int woff(int r, int c) { return r * kWRow + 16 * (c ^ wsw(r)); }

// One B operand from 8 bytes of symmetric packed codes: 16 bytes 16 q, in code order.
__device__ __forceinline__ v4i unpack_sym(uint32_t w0, uint32_t w1)
{
    const uint32_t w[2] = {w0, w1};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t s = w[i] << 4;  // byte j: low nibble of byte j on top
        // bytes (s0 w0 s1 w1) and (s2 w2 s3 w3): codes 0..3 and 4..7 on top of their bytes
        o[2 * i] = __builtin_amdgcn_perm(w[i], s, 0x05010400u) & 0xF0F0F0F0u;
        o[2 * i + 1] = __builtin_amdgcn_perm(w[i], s, 0x07030602u) & 0xF0F0F0F0u;
    }
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

// One B operand from 8 bytes of asymmetric packed codes: 16 signed bytes q - z, with z replicated in zz.
__device__ __forceinline__ v4i unpack_asym(uint32_t w0, uint32_t w1, uint32_t zz)
{
    const uint32_t w[2] = {w0, w1};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t ev = (w[i] & 0x0F0F0F0Fu) | 0x80808080u;         // codes 0,2,4,6 + 0x80
        const uint32_t od = ((w[i] >> 4) & 0x0F0F0F0Fu) | 0x80808080u;  // codes 1,3,5,7 + 0x80
        o[2 * i] = (__builtin_amdgcn_perm(od, ev, 0x05010400u) - zz) ^ 0x80808080u;
        o[2 * i + 1] = (__builtin_amdgcn_perm(od, ev, 0x07030602u) - zz) ^ 0x80808080u;
    }
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

template <int G, bool SYM, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void k_w4a8(const int8_t *__restrict__ xq, const float *__restrict__ sx,
                                                     int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ wp,
                                                     const float *__restrict__ sw, const uint8_t *__restrict__ zw,
                                                     void *__restrict__ y, int tiles)
{
    constexpr int DPG = G / 32;   // MFMA depths per group (1, 2 or 4: a divisor of the 4 depths of a step)
    constexpr int GPS = kBK / G;  // groups per step
    int8_t *const s0 = lds_block<kStage, 0>();
    int8_t *const s1 = lds_block<kStage, 1>();
    int8_t *const s2 = lds_block<kStage, 2>();

    const int per = (tiles + kW8Xcds - 1) / kW8Xcds;  // XCD x takes tiles [x per, (x + 1) per)
    const int t = (int)(blockIdx.x % kW8Xcds) * per + (int)(blockIdx.x / kW8Xcds);
    if (t >= tiles)
        return;
    const int m_tiles = (int)((M + kBM - 1) / kBM);
    const int n_tiles = (int)((N + kBN - 1) / kBN);
    // Tiles in groups of GM token tiles: consecutive tiles sweep GM token tiles for each channel tile in turn, so
    // the blocks an XCD runs at once (64) share 4 activation tiles and 16 weight tiles through its L2 (HBM
    // reads per launch: 166 MB against 395 MB when they swept all 16 token tiles of 4 channel tiles).
    constexpr int GM = 4;
    const int in_group = GM * n_tiles;
    const int first_m = (t / in_group) * GM;
    const int gsize = min(m_tiles - first_m, GM);
    const int64_t m0 = (int64_t)(first_m + (t % in_group) % gsize) * kBM;
    const int64_t n0 = (int64_t)((t % in_group) / gsize) * kBN;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col = lane % 32, h = lane / 32;
    const int64_t groups = K / G;
    const int nsteps = (int)(K / kBK);

    // Direct-load sources. Instruction i of wave w fills the 64 slots from S = (i * waves + w) * 64 of a stage:
    // slots [0, 1024) are activation row P / 8, physical piece P % 8; the rest weight row (P - 1024) / 4,
    // physical piece P % 4. A slot is filled from the logical piece that the swizzle puts there; rows past
    // M or N repeat the last row (computed, never stored). 32-bit offsets from the tile's first rows.
    const int8_t *const xbase = xq + m0 * K;
    const uint8_t *const wbase = wp + n0 * (K / 2);
    uint32_t offs[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int P = (i * kWaves + w) * kWave + lane;
        if (i < kXLoads) {
            const int r = P >> 3;
            offs[i] = (uint32_t)(std::min<int64_t>(r, M - 1 - m0) * K + 16 * ((P & 7) ^ xsw(r)));
        } else {
            const int q = P - kBM * 8, r = q >> 2;
            offs[i] = (uint32_t)(std::min<int64_t>(r, N - 1 - n0) * (K / 2) + 16 * ((q & 3) ^ wsw(r)));
        }
    }
    auto issue = [&](int8_t *stage, int k) __attribute__((always_inline)) {
        const int64_t kk = k < nsteps ? k : nsteps - 1;  // past the end: reload the last step
        const int8_t *xb = xbase + kk * kBK;
        const uint8_t *wb = wbase + kk * (kBK / 2);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const void *src = i < kXLoads ? (const void *)(xb + offs[i]) : (const void *)(wb + offs[i]);
            __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)(stage + (i * kWaves + w) * kWave * 16),
                                             16, 0, 0);
        }
    };

    // the lane's channel (clamped: channels past N are computed, never stored) and its group metadata
    const int64_t nrow = std::min<int64_t>(n0 + w * kWN + col, N - 1);
    const float *const swr = sw + nrow * groups;
    const uint8_t *const zwr = SYM ? nullptr : zw + nrow * groups;
    struct Meta {
        float s[GPS];
        uint32_t zz[GPS];
    };
    auto load_meta = [&](Meta &md, int k) __attribute__((always_inline)) {
        const int64_t kk = k < nsteps ? k : nsteps - 1;
#pragma unroll
        for (int gi = 0; gi < GPS; ++gi) {
            md.s[gi] = swr[kk * GPS + gi];
            md.zz[gi] = SYM ? 0u : (uint32_t)zwr[kk * GPS + gi] * 0x01010101u;
        }
    };

    v16i acc[kTM];
    float facc[kTM][16];
#pragma unroll
    for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            acc[j][e] = 0;
            facc[j][e] = 0.0f;
        }
    // Part p of np of the fold of tile j's finished group: its 16 / np accumulators converted and added to the
    // fp32 ones with the group scale.
    auto fold_part = [&](int j, float sc, int p, int np) __attribute__((always_inline)) {
#pragma unroll
        for (int e = p * (16 / np); e < (p + 1) * (16 / np); ++e)
            facc[j][e] = __builtin_fmaf(sc, (float)acc[j][e], facc[j][e]);
    };

    // Depth d = 2 q + e of a step: pair q, MFMA e. Its activation piece holds the same 16 codes per lane half
    // as its B operand.
    auto xpiece = [&](int d) __attribute__((always_inline)) {
        const int q = d / 2, e = d % 2;
        return G == 32 ? 4 * q + 2 * e + h : 4 * q + 2 * h + e;
    };
    const int wrow = w * kWN + col;  // the lane's weight row in a stage
    // Work unit u = (group gi, token tile j) of a step: the group's DPG MFMAs on tile j. The fold of unit u - L
    // is split over them, one part after each MFMA, so the VALU converts while the matrix core multiplies.
    // The lag L keeps the folded accumulators a whole unit away from the MFMA that wrote them (a fold right
    // behind its MFMA waits for it); L < 4 still folds a tile before the unit that reuses it. The last L
    // units of a step are folded by the first L units of the next step (all in the step's last group).
    constexpr int kUnits = GPS * kTM;
    constexpr int L = DPG == 1 ? 3 : 2;
    static_assert(L < kTM && L <= kTM, "pending units lie in one group");
    float pend_s = 0.0f;  // group scale of the pending folds; 0 before the first step (accumulators are 0)
    auto multiply = [&](const int8_t *st, const Meta &md) __attribute__((always_inline)) {
        const int8_t *ws = st + kXBytes;
        v4i fb[4];  // the step's four B operands
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if constexpr (G == 32) {  // depth 2 q + e is group 2 q + e: packed piece 2 q + e, its half h
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint2 pc = *reinterpret_cast<const uint2 *>(ws + woff(wrow, 2 * q + e) + 8 * h);
                    fb[2 * q + e] = SYM ? unpack_sym(pc.x, pc.y) : unpack_asym(pc.x, pc.y, md.zz[2 * q + e]);
                }
            } else {  // pair q lies in group (2 q) / DPG: packed piece 2 q + h, depth 2 q + e its half e
                const v4i pc = *reinterpret_cast<const v4i *>(ws + woff(wrow, 2 * q + h));
                const uint32_t zz = md.zz[(2 * q) / DPG];
                fb[2 * q] = SYM ? unpack_sym(pc[0], pc[1]) : unpack_asym(pc[0], pc[1], zz);
                fb[2 * q + 1] = SYM ? unpack_sym(pc[2], pc[3]) : unpack_asym(pc[2], pc[3], zz);
            }
        }
        auto read_unit = [&](v4i *f, int u) __attribute__((always_inline)) {
            const int gi = u / kTM, j = u % kTM;
#pragma unroll
            for (int dd = 0; dd < DPG; ++dd)
                f[dd] = *reinterpret_cast<const v4i *>(st + xoff(j * 32 + col, xpiece(gi * DPG + dd)));
        };
        v4i fcur[DPG], fnxt[DPG];
        read_unit(fcur, 0);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int gi = u / kTM, j = u % kTM;
            const int pu = u - L;                             // the unit folded now (< 0: previous step)
            const int pj = (pu + kUnits) % kTM;
            const float ps = pu < 0 ? pend_s : md.s[pu / kTM];
            if (u + 1 < kUnits)
                read_unit(fnxt, u + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dd = 0; dd < DPG; ++dd) {
                const v16i c = dd == 0 ? v16i{} : acc[j];
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fcur[dd], fb[gi * DPG + dd], c, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                fold_part(pj, ps, dd, DPG);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int dd = 0; dd < DPG; ++dd)
                fcur[dd] = fnxt[dd];
        }
        pend_s = md.s[GPS - 1];
    };

    Meta mcur, mnxt;
    auto step = [&](const int8_t *cur, int8_t *after_next, int k) __attribute__((always_inline)) {
        load_meta(mnxt, k + 1);    // before the direct loads: the wait below covers it
        issue(after_next, k + 2);
        multiply(cur, mcur);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));  // step k + 1 landed, fragment reads done
        __builtin_amdgcn_s_barrier();
        mcur = mnxt;
    };

    load_meta(mcur, 0);
    issue(s0, 0);
    issue(s1, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 15));
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
#pragma unroll
    for (int u = kUnits - L; u < kUnits; ++u)  // the last step's pending folds
        fold_part(u % kTM, pend_s, 0, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // no direct load may land in the stages reused below
    __syncthreads();

    // Epilogue: the unscaled fp32 tile as [token][channel] rows (512 bytes + 16 of padding, so the two lane
    // halves, 4 rows apart, write different banks) over the three stages; then each thread takes 8-channel
    // chunks of a row, applies the token scale (with 1/16 for symmetric codes), and stores them.
    constexpr int ROWB = kBN * 4 + 16, RPS = kStage / ROWB;
    static_assert(3 * RPS >= kBM, "the output tile fits in the stages");
    auto rowp = [&](int ml) __attribute__((always_inline)) -> float * {
        int8_t *p = ml < RPS ? s0 + ml * ROWB : ml < 2 * RPS ? s1 + (ml - RPS) * ROWB : s2 + (ml - 2 * RPS) * ROWB;
        return reinterpret_cast<float *>(p);
    };
#pragma unroll
    for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            rowp(j * 32 + 8 * (r / 4) + 4 * h + r % 4)[w * kWN + col] = facc[j][r];
    __syncthreads();
    constexpr float kUnit = SYM ? 0.0625f : 1.0f;
    constexpr int CPR = kBN / 8;  // 8-channel chunks per row
    const bool vec_ok = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(y) % 16) == 0;
    for (int qi = tid; qi < kBM * CPR; qi += kThreads) {
        const int ml = qi / CPR, cl = qi % CPR;
        const int64_t m = m0 + ml, nb = n0 + cl * 8;
        if (m >= M || nb >= N)
            continue;
        const float *src = rowp(ml) + cl * 8;
        const float4 a = reinterpret_cast<const float4 *>(src)[0], b = reinterpret_cast<const float4 *>(src)[1];
        const float sm = sx[m] * kUnit;
        const float v[8] = {a.x * sm, a.y * sm, a.z * sm, a.w * sm, b.x * sm, b.y * sm, b.z * sm, b.w * sm};
        if (vec_ok) {  // N % 8 == 0: a chunk never crosses N
            if (OUT_BF16)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + m * N + nb) =
                    make_uint4(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]), pack_bf16x2_rne(v[4], v[5]),
                               pack_bf16x2_rne(v[6], v[7]));
            else {
                float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(y) + m * N + nb);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (nb + e < N) {
                    if (OUT_BF16)
                        static_cast<uint16_t *>(y)[m * N + nb + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                    else
                        static_cast<float *>(y)[m * N + nb + e] = v[e];
                }
        }
    }
}

template <int G, bool SYM>
hipError_t w4a8_go(const W4A8Args &a, hipStream_t st)
{
    const int64_t tiles = ((a.N + kBN - 1) / kBN) * ((a.M + kBM - 1) / kBM);
    if (tiles > (int64_t)0x7FFFFFF0)
        return hipErrorInvalidValue;
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
