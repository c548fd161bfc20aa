// k_search.hip -- the fused alpha-grid search (steps 2-4) for gfx950.
//
// What is computed ("AWQ (activation-aware weight quantization)", "How it
// works" steps 2-4 and the awq() listing under "Source code"): for every
// candidate alpha_k, the mean squared output error
//     mse[k] = mean_{t,o} ( X Wq_k^T - X W^T )[t, o]^2,   Wq_k = Q(W diag(s_k)) / s_k,
// then the first strict minimum over k.
//
// How it is computed here (this design is ours; the pages give no GPU layout):
//  * Linearity: X Wq^T - X W^T = X D^T with D = Wq - W, so the reference
//    product X W^T is never formed and each candidate costs one contraction.
//    D = (q*scale - v) / s with v = w*s, built in registers from the group
//    statistics and converted once (round-to-nearest-even) to the MFMA
//    operand type.
//  * One block = 16 output rows x 256 tokens x up to NA = 11 candidates,
//    8 waves (two per SIMD), 32 tokens each. The error needs the full-K sum
//    of X D^T before squaring, so K cannot be split: every candidate keeps
//    its own fp32 accumulator tile (NA x 2 tiles x 4 values = 88 registers
//    per lane), which is what limits the block to 16 rows x 256 tokens x 11
//    candidates; 21 candidates take two blocks.
//  * Per group of G input columns: each wave builds the D tiles of one or
//    two candidates in the exact register layout of the MFMA B operand and
//    stores them to LDS; after a barrier every wave runs the 16x16x32 MFMAs
//    of all candidates against its own 32 tokens, whose X fragments stay in
//    registers across candidates. D is therefore generated once per (row,
//    column, candidate) and reused by all 256 tokens of the block.
//  * The group maximum (or min/max) of a row is in-lane over KS*8 values plus
//    two cross-lane steps: lanes r, r+16, r+32, r+48 hold the 4 column slices
//    of row r.
//  * Epilogue: squares summed in fp64 per lane, then a fixed butterfly per
//    wave and a fixed-order sum of the 8 waves: one fp64 partial per
//    (candidate, block); no atomics, so results are bitwise reproducible.
//  * The search may round differently from the exact quantizer (a reciprocal
//    multiply instead of the IEEE division, contracted multiply-adds, 16-bit
//    D): only the error is produced here, and its tolerance allows it. The
//    codes that get stored come from the exact kernel in k_pack.hip.
#include "awq_internal.h"

#include <math.h>

#include <type_traits>

namespace awq {

constexpr int kWaves = 8;               // two per SIMD
constexpr int kTokPerWave = kTokPerBlock / kWaves;
constexpr int kTT = kTokPerWave / 16;   // 16-token MFMA tiles per wave
constexpr int kMaxNA = 11;              // candidates per block: 16 * NA accumulator registers per lane
constexpr int kLdsBudget = 160 * 1024 - 512;   // bytes of LDS per block

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
    static __device__ __forceinline__ f32x4 run(const bf16x8 &a, const bf16x8 &b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<f16> {
    static __device__ __forceinline__ f32x4 run(const f16x8 &a, const f16x8 &b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
// fp32 inputs: eight 16x16x4 fp32 MFMAs cover the same 32 columns. Slot i of
// every lane feeds MFMA i, so A and B pair the same column in each product.
template <> struct Mfma<float> {
    static __device__ __forceinline__ f32x4 run(const f32x8 &a, const f32x8 &b, f32x4 c)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
};

// Max / min over the four lanes l, l^16, l^32, l^48 (the four 8-column
// slices of one row in the B-operand layout) with two lane-swap steps:
// permlane16_swap(x, x) hands lane l the values of lanes l and l^16, and
// permlane32_swap(x, x) those of l and l^32.
__device__ __forceinline__ float lanes4_max(float m)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(m), __float_as_int(m), false, false);
    m = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float lanes4_min(float m)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(m), __float_as_int(m), false, false);
    m = fminf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fminf(__int_as_float(b[0]), __int_as_float(b[1]));
}

// fp32(w * s) for a stored fp16 weight, the low or high half of a 32-bit
// pair, in one instruction: v_fma_mix_f32 widens an fp16 source exactly and
// rounds w * s + 0 once (the same value as widening and multiplying).
__device__ __forceinline__ float mul_f16_lo(uint32_t pair, float s)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
    return r;
}
__device__ __forceinline__ float mul_f16_hi(uint32_t pair, float s)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
    return r;
}

// MFMA instructions per 32-column step of one 16x16 tile.
template <typename T> struct MfmaCount { static constexpr int value = 1; };
template <> struct MfmaCount<float> { static constexpr int value = 8; };

template <typename T> __device__ __forceinline__ typename Vec8<T>::type narrow8(const float *d);
template <> __device__ __forceinline__ f32x8 narrow8<float>(const float *d)
{
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = d[i];
    return r;
}
template <> __device__ __forceinline__ bf16x8 narrow8<bf16>(const float *d)
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const bf16x2 p = __builtin_convertvector(f32x2{d[i], d[i + 1]}, bf16x2);
        r[i] = p[0];
        r[i + 1] = p[1];
    }
    return r;
}
template <> __device__ __forceinline__ f16x8 narrow8<f16>(const float *d)
{
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const f16x2 p = __builtin_convertvector(f32x2{d[i], d[i + 1]}, f16x2);
        r[i] = p[0];
        r[i + 1] = p[1];
    }
    return r;
}

template <typename TOp, int G>
struct SearchShape {
    static constexpr int KS = G / 32;   // 32-column MFMA steps per group
    static constexpr int kTileBytes = KS * 64 * (int)sizeof(typename Vec8<TOp>::type);
    // LDS per block for NA candidates: two buffers (this group's D tiles, the
    // next group's) of NA + 1 tiles (the extra one takes the writes of idle
    // generation slots), s and 1/s rows for two groups, the epilogue sums.
    static constexpr int lds_bytes(int na)
    {
        return 2 * (na + 1) * kTileBytes + 2 * 2 * na * G * 4 + kWaves * na * 8;
    }
    static constexpr int fit(int na) { return na > 1 && lds_bytes(na) > kLdsBudget ? fit(na - 1) : na; }
    static constexpr int NA = fit(kMaxNA);
    static constexpr int GPW = (NA + kWaves - 1) / kWaves;   // tiles each wave builds per group
};

// Stored inputs -> MFMA operand type (identity, or exact widening to fp32).
template <typename TIn, typename TOp> struct ToOp {
    static __device__ __forceinline__ typename Vec8<TOp>::type run(const typename Vec8<TIn>::type &v)
    {
        return v;
    }
};
template <typename TIn> struct ToOp<TIn, float> {
    static __device__ __forceinline__ f32x8 run(const typename Vec8<TIn>::type &v)
    {
        f32x8 r;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = static_cast<float>(v[i]);
        return r;
    }
};

// D for one candidate tile: q = rne(v / scale) (clamped to the asymmetric
// code range; the symmetric clamp of the exact quantizer can never bind,
// since |v| <= max|v| = L * scale), d = (q * scale - v) / s, rounded to the
// operand type and stored as this lane's 8-column slices of the B operand.
//
// The plain path takes the quotient as v * rcp(scale) and scale as
// max|v| * (1/L): the error sum tolerates those last-bit differences. EXACT
// reproduces the exact quantizer's arithmetic: IEEE scale and zero, and the
// correctly rounded quotient from one residual step (Markstein: with
// y = RN(1/b) and q0 = RN(a*y), RN(q0 + RN(a - b*q0)*y) = RN(a/b)). It is
// used for the candidate whose scales are all ones (alpha = 0): v then holds
// the stored 16-bit weights, which sit exactly on rounding ties often enough
// that a one-ulp quotient difference would flip codes the exact quantizer
// keeps (a systematic 2e-4 shift of the RTN error). For other candidates
// v = w * s is unstructured and such flips have probability ~1e-7 per weight.
template <typename TOp, int KS, bool ASYM, bool EXACT>
__device__ __forceinline__ void build_tile(const float (&v)[KS][8], float levels, float maxq,
                                           float inv_levels, float inv_maxq,
                                           const float *__restrict__ irow,
                                           typename Vec8<TOp>::type *dst)
{
    float scale, rs, zlo = 0.f, zhi = 0.f;
    if (!ASYM) {
        float m = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                m = fmaxf(m, fabsf(v[ks][i]));
        m = lanes4_max(m);
        if (EXACT) {
            scale = fmaxf(m / levels, 1e-8f);
            rs = 1.0f / scale;
        } else {
            scale = fmaxf(m * inv_levels, 1e-8f);
            rs = __builtin_amdgcn_rcpf(scale);
        }
    } else {
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo = fminf(lo, v[ks][i]);
                hi = fmaxf(hi, v[ks][i]);
            }
        lo = lanes4_min(lo);
        hi = lanes4_max(hi);
        float zero;
        if (EXACT) {
            scale = fmaxf((hi - lo) / maxq, 1e-8f);
            rs = 1.0f / scale;
            zero = rintf(-lo / scale);
        } else {
            scale = fmaxf((hi - lo) * inv_maxq, 1e-8f);
            rs = __builtin_amdgcn_rcpf(scale);
            zero = rintf(-lo * rs);
        }
        zlo = -zero;
        zhi = maxq - zero;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const f32x8 i8 = *reinterpret_cast<const f32x8 *>(irow + ks * 32);
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float u = v[ks][i] * rs;
            if (EXACT)
                u = fmaf(fmaf(-u, scale, v[ks][i]), rs, u);
            float q = rintf(u);
            if (ASYM)
                q = fminf(fmaxf(q, zlo), zhi);
            d[i] = fmaf(q, scale, -v[ks][i]) * i8[i];
        }
        dst[ks * 64] = narrow8<TOp>(d);
    }
}

// Logical block coordinates (row block, token block, candidate pass).
// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2. When the row blocks split evenly over the XCDs, the blocks that
// share W rows (every token block and candidate pass of one row block) get
// consecutive places in one XCD's dispatch order, so those rows come from
// HBM once and then from that XCD's L2; otherwise the grid is used as is.
constexpr int kXcds = 8;
struct BlockCoord {
    int64_t x, y, z;
};
__device__ __forceinline__ BlockCoord block_coord()
{
    const int64_t nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
    if (nx % kXcds != 0)
        return {(int64_t)blockIdx.x, (int64_t)blockIdx.y, (int64_t)blockIdx.z};
    const int64_t lin = blockIdx.x + nx * (blockIdx.y + ny * (int64_t)blockIdx.z);
    const int64_t xcd = lin % kXcds, k = lin / kXcds;
    const int64_t per = ny * nz;   // blocks per row block: passes fastest, then token blocks
    const int64_t rem = k % per;
    return {(k / per) * kXcds + xcd, rem / nz, rem % nz};
}

// One block: 16 output rows x 256 tokens x NA candidates (candidates a0 ..
// a0 + NA - 1, a0 = NA * pass), 8 waves of 32 tokens, two per SIMD.
//
// Software pipeline over groups of G input columns, one barrier per group:
// the D tiles live in two LDS buffers selected by group parity. In the
// iteration of group g every wave
//   1. issues the loads of group g+1's weights and of group g+2's s rows,
//   2. waits at the barrier (group g's tiles are complete; group g-1's have
//      been read by everyone),
//   3. runs the MFMAs of all NA candidates of group g (B fragments read one
//      candidate ahead), then issues the loads of group g+1's X fragments,
//   4. builds its share of group g+1's tiles into the other buffer and
//      stages group g+2's s rows.
// Measured on gfx950, a SIMD's MFMA and VALU time add up rather than overlap
// (also across waves, and also with waves specialised to one of the two
// roles), so the time per group is close to the MFMA time plus the tile
// generation's VALU time; the pipeline keeps LDS and memory latency out of it.
template <typename TIn, typename TOp, int G, bool ASYM>
__global__ __launch_bounds__(kWaves * 64, 1) void k_search(
    const TIn *__restrict__ W, const TIn *__restrict__ X, int64_t out, int64_t in, int64_t tokens,
    const float *__restrict__ s_tab, const float *__restrict__ inv_tab,
    const int32_t *__restrict__ unit, int n_alpha, int bits, double *__restrict__ partial)
{
    typedef typename Vec8<TOp>::type V8;
    typedef typename Vec8<TIn>::type V8in;
    constexpr int KS = SearchShape<TOp, G>::KS;
    constexpr int NA = SearchShape<TOp, G>::NA;
    constexpr int GPW = SearchShape<TOp, G>::GPW;

    __shared__ V8 dbuf[2][NA + 1][KS][64];
    // s and 1/s of this block's candidates over one group of columns, for
    // the group being built; double-buffered by group parity.
    __shared__ f32x4 stab[2][2][NA][G / 4];
    __shared__ double wsum[kWaves][NA];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;           // row inside the tile (B operand column n)
    const int c = lane >> 4;           // which 8-column slice of a 32-column step
    const BlockCoord bc = block_coord();
    const int64_t row = bc.x * 16 + r;
    const bool row_ok = row < out;
    const int64_t row_c = row_ok ? row : out - 1;
    const int64_t tok0 = bc.y * kTokPerBlock + wave * kTokPerWave;
    const int a0 = (int)bc.z * NA;
    const int na = n_alpha - a0 < NA ? n_alpha - a0 : NA;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    const int64_t blk = bc.x * gridDim.y + bc.y;

    const float levels = (float)((1 << (bits - 1)) - 1);
    const float maxq = (float)((1 << bits) - 1);
    const float inv_levels = 1.0f / levels;
    const float inv_maxq = 1.0f / maxq;

    // X rows of this wave's tokens and the W row of this lane, clamped to the
    // last token / row (always in bounds). The products of the clamped
    // duplicates land in accumulator entries of tokens or rows past the end,
    // which the epilogue leaves out; nothing is masked inside the loop.
    const TIn *xrow[kTT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
        const int64_t t = tok0 + tt * 16 + r;
        xrow[tt] = X + (t < tokens ? t : tokens - 1) * in + c * 8;
    }
    const TIn *wrow = W + row_c * in + c * 8;

    // Generation slots of this wave: slots wave + 8 i, of which the first
    // na are real. Waves 0-2 get two slots when na > 8, so SIMDs 0-2 build
    // three tiles per group and SIMD 3 (waves 3 and 7) two; slot s builds
    // candidate (s - 3) mod na, which puts candidate 0 -- the one built with
    // the slower exact path in the first pass -- on wave 3, i.e. on SIMD 3.
    // Idle slots build a valid candidate's tile into the spare slot NA.
    int gen_a[GPW], gen_slot[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int a = wave + kWaves * i;
        const bool real = a < na;
        const int cand = (a + 3 * (na - 1)) % na;   // (a - 3) mod na, a < 8 + na
        gen_a[i] = a0 + (real ? cand : na - 1);
        gen_slot[i] = real ? cand : NA;
    }
    // Slots after the first are built only when they hold a candidate (the
    // first slot of every wave is always real or the spare).
    const int gen_n = wave + kWaves < na ? (wave + 2 * kWaves < na ? 3 : 2) : 1;
    // Which tiles take the exact quotient path: the candidate whose scales
    // are all ones (alpha = 0: slot 0 of wave 0 in the first pass), or every
    // candidate when all of them are all ones (flat activations, where the
    // candidates must come out identical). Decided once per wave, outside the
    // group loop, so each loop body is free of per-tile branches.
    const bool all_unit = unit[n_alpha - 1] != 0;
    const int exm = all_unit ? 2 : (a0 == 0 && gen_slot[0] == 0 ? 1 : 0);
    V8 xa[kTT][KS];
    auto load_x = [&](int64_t k0, V8 (&xd)[kTT][KS]) {
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                xd[tt][ks] = ToOp<TIn, TOp>::run(load8(xrow[tt] + k0 + ks * 32));
    };
    auto load_w = [&](int64_t k0, V8in (&wd)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            wd[ks] = load8(wrow + k0 + ks * 32);
    };
    // s and 1/s rows of group `gi`: fetched into registers (3 float4 per
    // thread at NA = 11, G = 128), stored to LDS later so the fetch latency
    // hides behind a whole iteration.
    constexpr int kSEntries = 2 * NA * (G / 4);
    constexpr int kSPer = (kSEntries + kWaves * 64 - 1) / (kWaves * 64);
    auto fetch_s = [&](int64_t gi, f32x4 (&sv)[kSPer]) {
#pragma unroll
        for (int i = 0; i < kSPer; ++i) {
            const int e = (int)threadIdx.x + kWaves * 64 * i;
            const int ec = e < kSEntries ? e : kSEntries - 1;
            const int which = ec / (NA * (G / 4));          // 0: s, 1: 1/s
            const int a = (ec / (G / 4)) % NA;
            const int q = ec % (G / 4);
            const int ag = a0 + (a < na ? a : na - 1);
            const float *base = which ? inv_tab : s_tab;
            sv[i] = *reinterpret_cast<const f32x4 *>(base + (int64_t)ag * in + gi * G + q * 4);
        }
    };
    auto store_s = [&](int sp, const f32x4 (&sv)[kSPer]) {
#pragma unroll
        for (int i = 0; i < kSPer; ++i) {
            const int e = (int)threadIdx.x + kWaves * 64 * i;
            if (e < kSEntries)
                (&stab[sp][0][0][0])[e] = sv[i];
        }
    };
    // v = w * s of one candidate: fp16 weights straight from the loaded
    // pairs (v_fma_mix_f32), other types from the once-widened wg.
    auto build_slot = [&](auto exact_tag, const V8in (&wraw)[KS], const float (&wg)[KS][8], int par,
                          int i) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        const int sa = gen_slot[i] < NA ? gen_slot[i] : na - 1;
        const float *srow = reinterpret_cast<const float *>(&stab[par][0][sa][0]) + c * 8;
        const float *irow = reinterpret_cast<const float *>(&stab[par][1][sa][0]) + c * 8;
        float v[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const f32x8 s8 = *reinterpret_cast<const f32x8 *>(srow + ks * 32);
            if constexpr (std::is_same<TIn, f16>::value) {
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 pr = __builtin_bit_cast(u32x4, wraw[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[ks][2 * e] = mul_f16_lo(pr[e], s8[2 * e]);
                    v[ks][2 * e + 1] = mul_f16_hi(pr[e], s8[2 * e + 1]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[ks][e] = wg[ks][e] * s8[e];
            }
        }
        build_tile<TOp, KS, ASYM, EXACT>(v, levels, maxq, inv_levels, inv_maxq, irow,
                                         &dbuf[par][gen_slot[i]][0][lane]);
    };
    auto build = [&](auto exm_tag, const V8in (&wraw)[KS], int par) {
        constexpr int EXM = decltype(exm_tag)::value;
        float wg[KS][8];
        if constexpr (!std::is_same<TIn, f16>::value) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                widen8<TIn>(wraw[ks], wg[ks]);
        }
        build_slot(std::integral_constant<bool, (EXM >= 1)>{}, wraw, wg, par, 0);
#pragma unroll
        for (int i = 1; i < GPW; ++i)
            if (i < gen_n)
                build_slot(std::integral_constant<bool, (EXM == 2)>{}, wraw, wg, par, i);
    };

    f32x4 acc[NA][kTT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
            acc[a][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t ngroups = in / G;
    const int64_t glast = ngroups - 1;
    // MFMAs of all NA candidates of the group whose tiles are in buffer par.
    // Every slot, unconditionally: a branch around an MFMA would make its
    // accumulator a control-flow merge, which the compiler resolves by
    // copying all accumulators between register files. Slots past na hold
    // valid but unused tiles and are never read out. The B fragments of
    // candidate a+1 are read before the MFMAs of candidate a (pinned, so the
    // LDS latency hides under the MFMAs).
    auto mfma_group = [&](int par) {
        V8 bcur[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bcur[ks] = dbuf[par][0][ks][lane];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            V8 bnext[KS];
            if (a + 1 < NA)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    bnext[ks] = dbuf[par][a + 1][ks][lane];
            // Each accumulator's MFMAs back to back: with the column steps
            // interleaved instead, the register allocator permutes the
            // loop-carried accumulators every group.
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc[a][tt] = Mfma<TOp>::run(xa[tt][ks], bcur[ks], acc[a][tt]);
            if (a + 1 < NA)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    bcur[ks] = bnext[ks];
        }
        __builtin_amdgcn_sched_group_barrier(0x0100, KS, 0);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            if (a + 1 < NA)
                __builtin_amdgcn_sched_group_barrier(0x0100, KS, 0);
            __builtin_amdgcn_sched_group_barrier(0x0008, KS * kTT * MfmaCount<TOp>::value, 0);
        }
    };

    // One iteration per group g, one barrier each: the MFMAs of group g
    // (tiles in buffer g & 1), then the building of group g+1's tiles into
    // the other buffer.
    auto run = [&](auto exm_tag) {
        {
            f32x4 sv[kSPer];
            fetch_s(0, sv);
            store_s(0, sv);
            fetch_s(ngroups > 1 ? 1 : 0, sv);
            store_s(1, sv);
        }
        {
            V8in w0[KS];
            load_w(0, w0);
            load_x(0, xa);
            __syncthreads();
            build(exm_tag, w0, 0);
        }
        for (int64_t g = 0; g < ngroups; ++g) {
            const int par = (int)(g & 1);
            // Next group's weights and the s rows of the group after it are
            // fetched first; the next group's X fragments after this group's
            // MFMAs, so the current and next fragments are never live
            // together. (The last groups reload valid groups; what they then
            // build or store lands in buffers nobody reads again.)
            const int64_t gn = g + 1 < ngroups ? g + 1 : glast;
            V8in wn[KS];
            load_w(gn * G, wn);
            f32x4 sv[kSPer];
            fetch_s(g + 2 < ngroups ? g + 2 : glast, sv);
            __syncthreads();
            mfma_group(par);
            load_x(gn * G, xa);
            build(exm_tag, wn, par ^ 1);
            store_s(par, sv);
        }
    };
    if (exm == 0)
        run(std::integral_constant<int, 0>{});
    else if (exm == 1)
        run(std::integral_constant<int, 1>{});
    else
        run(std::integral_constant<int, 2>{});

    // Sum of squares: exact fp64 squares of the fp32 accumulators, fixed order.
    // Lane l holds, of tile tt, output row r = l & 15 for the tokens
    // tok0 + 16 tt + 4 (l >> 4) + e; entries of rows or tokens past the end
    // (products of the clamped duplicates) are left out.
    bool keep[kTT][4];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            keep[tt][e] = row_ok && tok0 + tt * 16 + 4 * c + e < tokens;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        if (a < na) {
            double sum = 0.0;
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double x = keep[tt][e] ? (double)acc[a][tt][e] : 0.0;
                    sum += x * x;
                }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1)
                sum += __shfl_xor(sum, off);
            if (lane == 0)
                wsum[wave][a] = sum;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < na) {
        const int a = threadIdx.x;
        double total = wsum[0][a];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            total += wsum[w][a];
        partial[(int64_t)(a0 + a) * nblk + blk] = total;
    }
}

// The finish as its own launch (one block; the work is a few thousand
// doubles for the layers this is meant for). Body: finish_block.
constexpr int kFinishWaves = 16;

__global__ __launch_bounds__(kFinishWaves * 64) void k_finish(const double *__restrict__ partial,
                                                            int64_t nblk, int n_alpha, double denom,
                                                            const float *__restrict__ s_tab,
                                                            int64_t in, double *__restrict__ mse,
                                                            int32_t *__restrict__ best,
                                                            float *__restrict__ s_best)
{
    __shared__ double err[AWQ_MAX_GRID + 1];
    __shared__ int sbest;
    finish_block(partial, nblk, n_alpha, denom, s_tab, in, mse, best, s_best, err, &sbest);
}

template <typename TIn, typename TOp, int G>
static hipError_t search_typed(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,
                               const float *s_tab, const float *inv_tab, const int32_t *unit,
                               int n_alpha, int bits, int mode, double *partial, hipStream_t st)
{
    constexpr int NA = SearchShape<TOp, G>::NA;
    dim3 grid((unsigned)((out + 15) / 16), (unsigned)((tokens + kTokPerBlock - 1) / kTokPerBlock),
              (unsigned)((n_alpha + NA - 1) / NA));
    if (mode == AWQ_SYM)
        hipLaunchKernelGGL((k_search<TIn, TOp, G, false>), grid, dim3(kWaves * 64), 0, st, (const TIn *)W,
                           (const TIn *)X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits,
                           partial);
    else
        hipLaunchKernelGGL((k_search<TIn, TOp, G, true>), grid, dim3(kWaves * 64), 0, st, (const TIn *)W,
                           (const TIn *)X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits,
                           partial);
    return hipGetLastError();
}

template <typename TIn, typename TOp>
static hipError_t search_group(const void *W, const void *X, int64_t out, int64_t in,
                               int64_t tokens, const float *s_tab, const float *inv_tab,
                               const int32_t *unit, int n_alpha, int bits, int group, int mode,
                               double *partial, hipStream_t st)
{
    switch (group) {
    case 32:
        return search_typed<TIn, TOp, 32>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, mode, partial, st);
    case 64:
        return search_typed<TIn, TOp, 64>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, mode, partial, st);
    default:
        return search_typed<TIn, TOp, 128>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, mode, partial, st);
    }
}

// The 16-bit operands round D to 8 (bf16) or 11 (fp16) significant bits. The
// rounding errors are unbiased; their effect on a row's squared error is
// about 2 u / sqrt(3 n) relative (u = 2^-8 for bf16, n = the number of input
// channels that dominate the row's error, as few as 1-2 when a handful of
// outlier channels carry the activation energy), and it averages down over
// independent rows: about 1e-5 at the sizes of real layers, but up to 1e-3
// on a 64-row layer with two dominant channels. Layers with fewer than 256
// rows (or 16 tokens) therefore use exact fp32 operands; they are cheap.
bool search_uses_fp32_operands(int dtype, int64_t out, int64_t tokens)
{
    return dtype == AWQ_F32 || out < kMinRows16 || tokens < kMinTokens16;
}

// The 32x32 search (k_search16.hip) takes 16-bit operands with `in` a
// multiple of 128 and passes of 9..12 candidates (n_alpha >= 9).
bool search16_applies(int dtype, int64_t out, int64_t in, int64_t tokens, int n_alpha)
{
    if (search_uses_fp32_operands(dtype, out, tokens))
        return false;
    const int npass = (n_alpha + 11) / 12;
    const int64_t nblocks = ((out + 15) / 16) * ((tokens + kTokPerBlock - 1) / kTokPerBlock);
    return in % 128 == 0 && n_alpha / npass >= 9 && nblocks * npass <= 0x7fffffffLL;
}

hipError_t launch_prepare(const void *X, int dtype, const float *xmag, int64_t out, int64_t in,
                          int64_t tokens, int grid, float *s_tab, float *inv_tab, int32_t *unit,
                          void *xfrag, hipStream_t st)
{
    if (search16_applies(dtype, out, in, tokens, grid + 1))
        return dtype == AWQ_F16 ? launch_prepare16_f16(X, xmag, in, tokens, grid, s_tab, inv_tab, unit, xfrag, st)
                                : launch_prepare16_bf16(X, xmag, in, tokens, grid, s_tab, inv_tab, unit, xfrag, st);
    return launch_s_table(xmag, in, grid, s_tab, inv_tab, unit, st);
}

hipError_t launch_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                         int64_t tokens, const float *s_tab, const float *inv_tab,
                         const int32_t *unit, int n_alpha, int bits, int group, int mode,
                         double *partial, const void *xfrag, const FinishOut *fin, hipStream_t st)
{
    hipError_t e;
    const bool wide = search_uses_fp32_operands(dtype, out, tokens);
    if (search16_applies(dtype, out, in, tokens, n_alpha)) {
#define AWQ_S16_CALL(name) name(W, xfrag, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, mode, partial, st)
        if (dtype == AWQ_F16)
            e = group == 32 ? AWQ_S16_CALL(launch_search16_f16_g32)
              : group == 64 ? AWQ_S16_CALL(launch_search16_f16_g64)
                            : AWQ_S16_CALL(launch_search16_f16_g128);
        else
            e = group == 32 ? AWQ_S16_CALL(launch_search16_bf16_g32)
              : group == 64 ? AWQ_S16_CALL(launch_search16_bf16_g64)
                            : AWQ_S16_CALL(launch_search16_bf16_g128);
#undef AWQ_S16_CALL
    } else {
        switch (dtype) {
        case AWQ_F32:
            e = search_group<float, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
            break;
        case AWQ_F16:
            e = wide ? search_group<f16, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st)
                     : search_group<f16, f16>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
            break;
        default:
            e = wide ? search_group<bf16, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st)
                     : search_group<bf16, bf16>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
            break;
        }
    }
    // single-call search: the finish follows on the same stream
    if (e == hipSuccess && fin)
        e = launch_reduce_argmin(partial, ((out + 15) / 16) * ((tokens + kTokPerBlock - 1) / kTokPerBlock),
                                 n_alpha, out, tokens, in, s_tab, fin->mse, fin->best, fin->s_best, st);
    return e;
}

hipError_t launch_reduce_argmin(const double *partial, int64_t nblk, int n_alpha, int64_t out,
                                int64_t tokens, int64_t in, const float *s_tab, double *mse,
                                int32_t *best, float *s_best, hipStream_t st)
{
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinishWaves * 64), 0, st, partial, nblk, n_alpha,
                       (double)tokens * (double)out, s_tab, in, mse, best, s_best);
    return hipGetLastError();
}

}  // namespace awq
