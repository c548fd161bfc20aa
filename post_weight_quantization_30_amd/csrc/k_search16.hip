// k_search16.hip -- the alpha-grid search (steps 2-4) for fp16 and bf16
// layers, on the 32x32x16 matrix instructions of gfx950.
//
// What is computed ("AWQ (activation-aware weight quantization)", "How it
// works" steps 2-4 and the awq() listing under "Source code"): for every
// candidate alpha_k, the mean squared output error
//     mse[k] = mean_{t,o} ( X Wq_k^T - X W^T )[t, o]^2,   Wq_k = Q(W diag(s_k)) / s_k.
// This kernel leaves one fp64 partial sum of squares per (candidate, block of
// 16 output rows x 256 tokens); k_finish sums them and takes the argmin.
//
// How (the design is ours; the pages describe no GPU layout):
//  * Linearity: X Wq^T - X W^T = X D^T with D = Wq - W, so each candidate
//    costs one contraction and X W^T is never formed. D = (q*scale - v) / s
//    with v = w*s is built in registers and rounded once to the 16-bit
//    operand type.
//  * One block: 16 output rows x 256 tokens x up to 12 candidates, 8 waves
//    (two per SIMD) of 64 tokens. The matrix instruction is
//    v_mfma_f32_32x32x16: A = 32 tokens of X (shared by every candidate),
//    B = the D rows of a PAIR of candidates (2 x 16 rows side by side in the
//    32-wide N dimension), so a block's 16 rows still fill the instruction and
//    each wave keeps 16 fp32 accumulators per candidate pair and A tile. The
//    error is squared only after the full-K sum, so K is never split.
//  * Measured on this GPU (mb_gfx950): an MFMA-only wave keeps its rate
//    next to a VALU wave on the same SIMD, which loses about 8 cycles per
//    32x32x16 instruction. So every wave both runs its MFMAs for step si and
//    builds D tiles for step si + 1, the two streams interleaved instruction
//    by instruction in fenced slots (sched_barrier), instead of all waves
//    alternating between an MFMA phase and a build phase.
//  * Per step of 128 input columns (8 k-steps of 16; any group size that
//    divides 128): the W tile (16 rows x 128) and the s and 1/s rows of the
//    block's candidates are loaded into registers two steps ahead and
//    written to LDS at the end of the step before they are built; the D
//    tiles are double-buffered in LDS in the exact lane layout of the B
//    operand; one barrier per step. X comes from a copy in matrix-fragment
//    order (written by the preparation kernel below), so each A-fragment load
//    is one contiguous 1 KB read.
//  * D-tile building: a "unit" is one candidate's 16 x 128 tile, built by one
//    wave, lane (r, c) = (lane & 15, lane >> 4) holding row r, columns
//    32c .. 32c + 31. A block of n candidates has n units over 8 waves; the
//    candidate whose scales are all ones (alpha = 0) takes the exact
//    quantizer arithmetic and is placed on the SIMD that builds fewest units.
//  * k-order: inside a 128-column step, k-step s of the lanes of half h
//    (lane >> 5) covers columns 64h + 8s .. 64h + 8s + 7 for both A and B (a
//    contraction may permute k), so every lane's X and D fragments are
//    contiguous 128-byte runs.
//  * Epilogue: each lane's squares summed in fp32 fused multiply-adds, then
//    fp64 fixed butterflies and a fixed-order sum over the waves; no
//    atomics, bitwise reproducible.
//  * The search may round differently from the exact quantizer (reciprocal
//    multiply, 16-bit D): only the error is produced here, and its tolerance
//    allows that. Stored codes come from the exact kernel in k_pack.hip.
#include "awq_internal.h"

#include <math.h>

#include <type_traits>

namespace awq {

namespace s16 {

constexpr int kWaves = 8;                 // two per SIMD
constexpr int kTokW = 32;                 // tokens per wave (the A tile)
constexpr int kRows = kRowsPerBlock;      // 16 output rows per block
constexpr int kPairs = 6;                 // candidate pairs per block (12 slots)
constexpr int kSlots = 2 * kPairs;
constexpr int kStep = 128;                // input columns per pipeline step
constexpr int kKs = kStep / 16;           // 16-column k-steps per pipeline step
constexpr int kStg = 2;                   // staging buffers (step si in si % kStg)
constexpr int kPd = 3;                    // B fragments read ahead (each serves two MFMAs)
static_assert(kWaves * kTokW == kTokPerBlock, "block token count");

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma32;
template <> struct Mfma32<f16> {
    static __device__ __forceinline__ f32x16 run(const f16x8 &a, const f16x8 &b, const f32x16 &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma32<bf16> {
    static __device__ __forceinline__ f32x16 run(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// LDS of one block.
template <typename T> struct Smem {
    typedef typename Vec8<T>::type V8;
    f32x4 st[kStg][2][kSlots][kStep / 4];     // s and 1/s rows of the slots, by step parity: 12 KB each
    u32x4 w[kStg][4][64];                     // the W tile (builder lane order): 4 KB each
    V8 d[2][kPairs][kKs][64];                 // D tiles (B operand layout), by step parity: 96 KB
    double wsum[4][kSlots];   // per token group of 64
};

// Max / min over lanes l, l^16, l^32, l^48 (the four 32-column slices of one
// row): permlane16_swap(x, x) gives lane l the values of lanes l and l^16,
// permlane32_swap(x, x) those of l and l^32.
__device__ __forceinline__ float fmax2(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float fmin2(float a, float b)
{
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float xl16_max(float m)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fmax2(__int_as_float(a[0]), __int_as_float(a[1]));
}
__device__ __forceinline__ float xl32_max(float m)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fmax2(__int_as_float(a[0]), __int_as_float(a[1]));
}
__device__ __forceinline__ float xl16_min(float m)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fmin2(__int_as_float(a[0]), __int_as_float(a[1]));
}
__device__ __forceinline__ float xl32_min(float m)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
    return fmin2(__int_as_float(a[0]), __int_as_float(a[1]));
}
// Reduction over the lanes that hold one quantization group of a row:
// the lane's own 32 columns (G = 32), with lane l^16 (G = 64), or all four
// slices (G = 128).
template <int G> __device__ __forceinline__ float group_max(float m)
{
    if (G >= 64)
        m = xl16_max(m);
    if (G >= 128)
        m = xl32_max(m);
    return m;
}
template <int G> __device__ __forceinline__ float group_min(float m)
{
    if (G >= 64)
        m = xl16_min(m);
    if (G >= 128)
        m = xl32_min(m);
    return m;
}

// fp32(w * s) for the low / high fp16 of a 32-bit pair in one instruction:
// v_fma_mix_f32 widens the fp16 source exactly and rounds w * s + 0 once
// (only the sign of a zero product differs from the plain product, which the
// error does not see). Written out because this toolchain, selecting the
// instruction from a widened element of a loaded vector, fed every element
// of the vector from its first register.
__device__ __forceinline__ float mix_lo(uint32_t pair, float s)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
    return r;
}
__device__ __forceinline__ float mix_hi(uint32_t pair, float s)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
    return r;
}

// Three-input max / min (one instruction each); amax3 takes absolute values.
// Written out because the compiler, not knowing that the v_fma_mix results
// above are ordinary numbers, would otherwise quiet each input first.
__device__ __forceinline__ float amax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float min3(float a, float b, float c)
{
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Sum of an fp64 value over the 16 lanes of each row and the two halves of
// the wave, in registers: each step adds the value of a partner lane (DPP
// quad_perm swaps of 1 and 2 lanes, row_half_mirror and row_mirror, which
// after the steps before pair lanes holding the sums of different quarters
// and halves of the row, then permlane32_swap across the halves); every
// lane ends with the same total, bitwise the xor butterfly's since each step
// adds the same two partial sums.
template <int CTRL> __device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, (uint64_t)hi << 32 | lo);
}
__device__ __forceinline__ double wave_rows_sum_f64(double x)
{
    x += dpp_f64<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_f64<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_f64<0x141>(x);   // row_half_mirror
    x += dpp_f64<0x140>(x);   // row_mirror
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    return __builtin_bit_cast(double, (uint64_t)(uint32_t)hi[0] << 32 | (uint32_t)lo[0]) +
           __builtin_bit_cast(double, (uint64_t)(uint32_t)hi[1] << 32 | (uint32_t)lo[1]);
}

template <typename T> __device__ __forceinline__ typename Vec8<T>::type pack8(const float *d);
template <> __device__ __forceinline__ f16x8 pack8<f16>(const float *d)
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
template <> __device__ __forceinline__ bf16x8 pack8<bf16>(const float *d)
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

struct QParams {
    float levels, maxq, inv_levels, inv_maxq;
};

// f(std::integral_constant<int, 0>), ..., f(std::integral_constant<int, N - 1>)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f)
{
    static_for_from<0, N>(f);
}

// One unit: the D tile of one candidate for the block's 16 rows and one
// 128-column step, built by one wave; lane (r, c) holds row r, columns
// 32c .. 32c + 31 (chunks i = 0..3 of 8 columns).
//
// q = rne(v / scale) (clamped to the asymmetric code range; the symmetric
// clamp of the exact quantizer cannot bind since |v| <= max|v| = L * scale),
// d = (q * scale - v) / s. The plain path takes v * rcp(scale) and
// max|v| * (1/L); EXACT uses IEEE scale and zero and the correctly rounded
// quotient from one residual step (Markstein: with y = RN(1/b) and
// q0 = RN(a*y), RN(q0 + RN(a - b*q0)*y) = RN(a/b)). EXACT serves the
// candidate whose scales are all ones: v then holds the stored weights,
// which sit exactly on rounding ties often enough that a one-ulp quotient
// difference would shift the rounding-to-nearest error systematically.
//
// The work is cut into pieces so the step's schedule can place them between
// matrix instructions. Every piece is one operation over a whole 8-column
// chunk (8 independent instructions):
//   0, 1     loads of chunks 0, 1: the chunk's weights (from the W tile) and
//            s values
//   2..9     per chunk i: v = w * s (8 v_fma_mix), then the chunk's max|v|
//            (or min and max) as a tree; the loads of chunks 2, 3 ride along
//   10       the group reduction across lanes, scale (and zero), 1/scale
//   11..     per chunk, one stage per piece: u = v / scale, [EXACT: the
//            quotient's residual and its correction], q = rne(u) (clamped
//            for the asymmetric codes; the 1/s load rides along), e =
//            q * scale - v, d = e / s -- converted to the operand type and
//            stored to the D tile in LDS.
template <bool EX> struct UnitPieces {
    static constexpr int kStages = EX ? 6 : 4;
    static constexpr int value = 11 + 4 * kStages;
};

template <typename T, int G, bool ASYM, bool EX>
struct Unit {
    typedef typename Vec8<T>::type V8;
    static constexpr int kStages = UnitPieces<EX>::kStages;
    const u32x4 *wrow;          // this lane's W chunks in the W tile (LDS; chunk i at +64 i)
    const float *srow, *irow;   // s and 1/s at this lane's 32 columns (LDS)
    V8 *dst;                    // the lane's slot of chunk 0 in the D tile (LDS)
    u32x4 wv[4];
    f32x8 sv[4], iv[4];
    float v[4][8], t[4][8], r_[4][8], mc[4][2];
    float scale, rs, zlo, zhi;

    __device__ __forceinline__ void init(const u32x4 *w_, const float *s_, const float *i_, V8 *d_)
    {
        wrow = w_;
        srow = s_;
        irow = i_;
        dst = d_;
    }

    __device__ __forceinline__ void ld(int i)
    {
        wv[i] = wrow[64 * i];
        sv[i] = *reinterpret_cast<const f32x8 *>(srow + 8 * i);
    }
    __device__ __forceinline__ void ldi(int i) { iv[i] = *reinterpret_cast<const f32x8 *>(irow + 8 * i); }

    __device__ __forceinline__ void vchunk(int i)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (std::is_same<T, f16>::value) {
                v[i][2 * e] = mix_lo(wv[i][e], sv[i][2 * e]);
                v[i][2 * e + 1] = mix_hi(wv[i][e], sv[i][2 * e + 1]);
            } else {
                v[i][2 * e] = __uint_as_float(wv[i][e] << 16) * sv[i][2 * e];
                v[i][2 * e + 1] = __uint_as_float(wv[i][e] & 0xffff0000u) * sv[i][2 * e + 1];
            }
        }
    }
    // max |v| of the chunk (sym), or min and max (asym), as trees of
    // three-input operations
    __device__ __forceinline__ void mchunk(int i)
    {
        const float *x = v[i];
        if (!ASYM) {
            const float a = amax3(x[0], x[1], x[2]);
            const float b = amax3(x[3], x[4], x[5]);
            mc[i][0] = amax3(x[6], x[7], max3(a, b, a));
        } else {
            const float a = min3(x[0], x[1], x[2]);
            const float b = min3(x[3], x[4], x[5]);
            mc[i][0] = min3(a, b, min3(x[6], x[7], 0.f));
            const float c = max3(x[0], x[1], x[2]);
            const float d = max3(x[3], x[4], x[5]);
            mc[i][1] = max3(c, d, max3(x[6], x[7], 0.f));
        }
    }

    __device__ __forceinline__ void reduce(const QParams &qp)
    {
        if (!ASYM) {
            const float mm = group_max<G>(max3(max3(mc[0][0], mc[1][0], mc[2][0]), mc[3][0], mc[3][0]));
            if (EX) {
                scale = fmaxf(mm / qp.levels, 1e-8f);
                rs = 1.0f / scale;
            } else {
                scale = fmaxf(mm * qp.inv_levels, 1e-8f);
                rs = __builtin_amdgcn_rcpf(scale);
            }
        } else {
            const float l = group_min<G>(min3(min3(mc[0][0], mc[1][0], mc[2][0]), mc[3][0], mc[3][0]));
            const float h = group_max<G>(max3(max3(mc[0][1], mc[1][1], mc[2][1]), mc[3][1], mc[3][1]));
            float zero;
            if (EX) {
                scale = fmaxf((h - l) / qp.maxq, 1e-8f);
                rs = 1.0f / scale;
                zero = rintf(-l / scale);
            } else {
                scale = fmaxf((h - l) * qp.inv_maxq, 1e-8f);
                rs = __builtin_amdgcn_rcpf(scale);
                zero = rintf(-l * rs);
            }
            zlo = -zero;
            zhi = qp.maxq - zero;
        }
    }

    // Stage st of chunk i.
    __device__ __forceinline__ void dstage(int i, int st)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = v[i][e];
            if (st == 0) {
                t[i][e] = x * rs;
            } else if (EX && st == 1) {
                r_[i][e] = fmaf(-t[i][e], scale, x);
            } else if (EX && st == 2) {
                t[i][e] = fmaf(r_[i][e], rs, t[i][e]);
            } else if (st == kStages - 3) {
                float q = rintf(t[i][e]);
                if (ASYM)
                    q = fminf(fmaxf(q, zlo), zhi);
                t[i][e] = q;
            } else if (st == kStages - 2) {
                t[i][e] = fmaf(t[i][e], scale, -x);
            } else {
                t[i][e] = t[i][e] * iv[i][e];
            }
        }
        if (st == kStages - 1)
            dst[i * 64] = pack8<T>(t[i]);
    }

    template <int K>
    __device__ __forceinline__ void piece(const QParams &qp)
    {
        if constexpr (K <= 1) {
            ld(K);
        } else if constexpr (K <= 9) {
            constexpr int i = (K - 2) / 2;
            if constexpr (K == 2)
                ld(2);
            if constexpr (K == 4)
                ld(3);
            if constexpr ((K - 2) % 2 == 0)
                vchunk(i);
            else
                mchunk(i);
        } else if constexpr (K == 10) {
            reduce(qp);
        } else {
            constexpr int i = (K - 11) / kStages, st = (K - 11) % kStages;
            if constexpr (st == kStages - 3)
                ldi(i);
            dstage(i, st);
        }
    }
};

// Block coordinates. The linear block id is pass-major, so the blocks of
// every pass run before those of the next one and each compute unit gets
// blocks of each pass (passes differ in candidate count). Workgroups go to
// the 8 XCDs round-robin by linear id, each with its own L2: when the row
// blocks split evenly over the XCDs, the blocks of one row block (its token
// blocks, and its other passes) land on one XCD, which then reads those W
// rows from HBM once.
struct Coord {
    int64_t rb, tb;
    int pass;
};
__device__ __forceinline__ Coord coord(int64_t nrb, int64_t ntb)
{
    const int64_t per = nrb * ntb;
    const int64_t lin = blockIdx.x;
    Coord k;
    k.pass = (int)(lin / per);
    const int64_t rem = lin % per;
    if (nrb % 8 == 0) {
        const int64_t xcd = rem % 8, j = rem / 8;
        k.rb = (j / ntb) * 8 + xcd;
        k.tb = j % ntb;
    } else {
        k.rb = rem / ntb;
        k.tb = rem % ntb;
    }
    return k;
}

template <typename T, int G, bool ASYM>
struct Search {
    typedef typename Vec8<T>::type V8;

    // The block's pipeline. Wave w covers tokens 64 g .. 64 g + 63 (g = w & 3,
    // two 32-token A tiles) of pair group h = w >> 2: pairs 3h .. 3h + NPW - 1
    // (waves w and w + 4 share a SIMD and the same tokens). U units per wave
    // (1 or 2); EX: the wave's units use the exact quantizer arithmetic.
    template <int NPW, int U, bool EX>
    static __device__ __forceinline__ void run(Smem<T> &sm, const T *__restrict__ W, const T *__restrict__ X,
                                               int64_t out, int64_t in, int64_t tokens,
                                               const float *__restrict__ s_tab,
                                               const float *__restrict__ inv_tab, int a0, int na,
                                               const int (&uslot)[2], const QParams &qp, int64_t rb,
                                               int64_t tb, int64_t nblk, int64_t blk,
                                               double *__restrict__ partial)
    {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        const int g = wave & 3, h = wave >> 2;
        const int pair0 = 3 * h;
        const int64_t nsteps = in / kStep;
        const int64_t slast = nsteps - 1;

        // MFMA side: the two A tiles of this wave in the fragment-ordered
        // copy of X (k_xfrag): tile t, step si, k-step s at
        // xp[t] + si * kXStep + s * 512 elements.
        constexpr int64_t kXStep = (int64_t)kWaves * kKs * 64 * 8;
        const int64_t tok0 = tb * kTokPerBlock + 64 * g;
        const T *xp0 = X + ((tb * nsteps * kWaves + 2 * g) * kKs * 64 + lane) * 8;
        const T *xp1 = xp0 + kKs * 64 * 8;

        // Builder side: row r, columns 32c .. 32c + 31 of each step.
        const int r = lane & 15, c = lane >> 4;

        // Staging of step `si`: 16 loads of 1 KB (64 lanes x 16 bytes) per
        // block, two per wave (load L = wave and wave + 8), fetched into
        // registers early in the step before and written to the LDS staging
        // buffer at its end, without branches. L < 4: chunk L of the W tile
        // (lane l carries chunk L of builder lane l). L >= 4: the s (L < 10)
        // or 1/s rows of slots 2m, 2m + 1 (m = (L - 4) % 6), 512 bytes
        // each; slots past na reload the last real one.
        const int64_t rowc = rb * kRows + r < out ? rb * kRows + r : out - 1;
        const T *wsrc = W + rowc * in + 32 * c;
        auto stage_src = [&](int64_t si, int j) -> const u32x4 * {
            const int L = wave + 8 * j;
            const int ld = L - 4 > 0 ? L - 4 : 0;
            const int which = ld / kPairs, m = ld % kPairs;
            const int slot = 2 * m + (lane >> 5);
            const int sl = slot < na ? slot : na - 1;
            const float *tab = which ? inv_tab : s_tab;
            const void *src_s = tab + (int64_t)(a0 + sl) * in + si * kStep + 4 * (lane & 31);
            const void *src_w = wsrc + si * kStep + 8 * (L & 3);
            return reinterpret_cast<const u32x4 *>(L < 4 ? src_w : src_s);
        };
        auto stage_dst = [&](int par, int j) -> u32x4 * {
            const int L = wave + 8 * j;
            const int ld = L - 4 > 0 ? L - 4 : 0;
            const int which = ld / kPairs, m = ld % kPairs;
            return L < 4 ? &sm.w[par][L & 3][lane]
                         : reinterpret_cast<u32x4 *>(&sm.st[par][which][2 * m][0]) + lane;
        };

        f32x16 acc[NPW][2];
#pragma unroll
        for (int p = 0; p < NPW; ++p)
            acc[p][0] = acc[p][1] = f32x16{};
        // X ring: k-step s of a step uses entry s % kXr; its two fragments
        // for k-step s + kXr are loaded as soon as k-step s retires.
        constexpr int kXr = 4;
        V8 xr[kXr][2];

        typedef Unit<T, G, ASYM, EX> UnitT;
        // unit i of this wave: staged inputs (s and 1/s rows, W tile) and
        // the D tile it writes
        auto unit_init_p = [&](UnitT &un, int i, const f32x4 *st_src, const u32x4 *w_src, V8 *d_dst) {
            const int sl = uslot[i];
            un.init(w_src + lane, reinterpret_cast<const float *>(st_src + sl * (kStep / 4)) + 32 * c,
                    reinterpret_cast<const float *>(st_src + (kSlots + sl) * (kStep / 4)) + 32 * c,
                    d_dst + ((sl >> 1) * kKs + 4 * (c & 1)) * 64 + 16 * (sl & 1) + r + 32 * (c >> 1));
        };
        auto unit_init = [&](UnitT &un, int i, int sb, int dp) {
            unit_init_p(un, i, &sm.st[sb][0][0][0], &sm.w[sb][0][0], &sm.d[dp][0][0][0]);
        };

        // Prologue: the loads staging steps 0 and 1 and those of X for the
        // first kXr k-steps go out first; the zero tiles are written while
        // they are in flight; then the staged data goes to LDS and step 0 is
        // built (plainly).
        u32x4 pre[kStg][2];
#pragma unroll
        for (int i = 0; i < kStg; ++i) {
            const int64_t si = i < nsteps ? i : slast;
            pre[i][0] = *stage_src(si, 0);
            pre[i][1] = *stage_src(si, 1);
        }
#pragma unroll
        for (int s = 0; s < kXr; ++s) {
            xr[s][0] = load8(xp0 + s * 512);
            xr[s][1] = load8(xp1 + s * 512);
        }
        // Empty slots (an odd count, or pairs past the candidates) hold zero
        // tiles in both buffers; nobody builds them. Pairs below na / 2 are
        // full, so only the pairs from there on are visited.
        {
            const int p0 = na >> 1, np = kPairs - p0;
            for (int e = threadIdx.x; e < 2 * np * kKs * 64; e += kWaves * 64) {
                const int b = e / (np * kKs * 64), p = p0 + (e / (kKs * 64)) % np;
                const int ln = e % 64;
                const int slot = 2 * p + ((ln & 31) >> 4);
                if (slot >= na)
                    sm.d[b][p][(e / 64) % kKs][ln] = V8{};
            }
        }

#pragma unroll
        for (int i = 0; i < kStg; ++i) {
            *stage_dst(i, 0) = pre[i][0];
            *stage_dst(i, 1) = pre[i][1];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < U; ++i) {
            UnitT un;
            unit_init(un, i, 0, 0);
            static_for<UnitPieces<EX>::value>([&](auto K) { un.template piece<decltype(K)::value>(qp); });
        }
        __syncthreads();

        // Step si (D and staging buffer par = si & 1), as a fixed sequence of NM slots, one
        // per matrix instruction (slot j = k-step s, pair p, A tile t; j =
        // (s * NPW + p) * 2 + t), fenced from each other so the compiler
        // keeps the order:
        //   - the B fragment of pair p, k-step s is read kPd fragments (2 kPd
        //     slots) ahead of its first MFMA and serves both A tiles,
        //   - the MFMA of slot j,
        //   - the pieces of this wave's tile building that fall on slot j
        //     (piece k of kPieces * U goes to slot k * NM / (kPieces * U)),
        //     units one after the other,
        //   - after the last MFMA of k-step s, the X fragments of the k-step
        //     kXr later (in this step or the next) go into its ring entry.
        // Before the slots, the loads staging step si + 2 are issued; at the
        // end of the step their data goes to staging buffer par (its step si
        // was built during step si - 1). One barrier per step.
        constexpr int NB = kKs * NPW;   // B fragments per step
        constexpr int NM = 2 * NB;      // MFMAs per step
        constexpr int kPieces = UnitPieces<EX>::value;
        constexpr int PT = kPieces * U;
        auto body = [&](auto build_tag, int64_t si) {
            constexpr bool BUILD = decltype(build_tag)::value;
            const int par = (int)(si & 1);
            const int64_t sn = si + 1 < nsteps ? si + 1 : slast;
            V8 b[NB];
            UnitT un[U];
            u32x4 sreg[2];
            if (BUILD) {
                // step si + 2, written to staging buffer par at the end
                const int64_t s2 = si + 2 < nsteps ? si + 2 : slast;
                sreg[0] = *stage_src(s2, 0);
                sreg[1] = *stage_src(s2, 1);
#pragma unroll
                for (int i = 0; i < U; ++i)
                    unit_init(un[i], i, par ^ 1, par ^ 1);
            }
#pragma unroll
            for (int q = 0; q < kPd; ++q)
                b[q] = sm.d[par][pair0 + q % NPW][q / NPW][lane];
            __builtin_amdgcn_sched_barrier(0);
            static_for<NM>([&](auto J) {
                constexpr int j = decltype(J)::value;
                constexpr int bi = j / 2, t = j % 2;
                constexpr int s = bi / NPW, p = bi % NPW;
                if constexpr (t == 0 && bi + kPd < NB)
                    b[bi + kPd] = sm.d[par][pair0 + (bi + kPd) % NPW][(bi + kPd) / NPW][lane];
                acc[p][t] = Mfma32<T>::run(xr[s % kXr][t], b[bi], acc[p][t]);
                if (BUILD) {
                    static_for<PT>([&](auto Kt) {
                        constexpr int k = decltype(Kt)::value;
                        if constexpr (k * NM / PT == j)
                            un[k / kPieces].template piece<k % kPieces>(qp);
                    });
                }
                if constexpr (t == 1 && p == NPW - 1) {
                    // k-step s + kXr: this step's, or the next step's s + kXr - kKs
                    const int64_t off = s + kXr < kKs ? si * kXStep + (s + kXr) * 512
                                                      : sn * kXStep + (s + kXr - kKs) * 512;
                    xr[s % kXr][0] = load8(xp0 + off);
                    xr[s % kXr][1] = load8(xp1 + off);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if (BUILD) {
                *stage_dst(par, 0) = sreg[0];
                *stage_dst(par, 1) = sreg[1];
            }
            __syncthreads();
        };
        for (int64_t si = 0; si + 1 < nsteps; ++si)
            body(std::true_type{}, si);
        body(std::false_type{}, slast);

        // Sum of squares. Lane l holds, for pair p and A tile t, column
        // n = l & 31 of the C tile -- candidate slot 2 (pair0 + p) + (n >> 4),
        // row n & 15 -- and tokens 32t + 8(e/4) + 4(l >> 5) + (e & 3),
        // e = 0..15, of the wave's 64. Entries of rows or tokens past the end
        // are left out. A lane's squares are summed in fp32, two chains of 16
        // fused multiply-adds (one per A tile, relative rounding below 1e-6),
        // added in fp64; the sums across lanes, waves and blocks are fp64.
        const int n = lane & 31;
        const bool row_ok = rb * kRows + (n & 15) < out;
        const bool full = tok0 + 2 * kTokW <= tokens;   // every token of the wave exists
#pragma unroll
        for (int p = 0; p < NPW; ++p) {
            float s2[2] = {0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (full) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        s2[t] = fmaf(acc[p][t][e], acc[p][t][e], s2[t]);
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t tk = tok0 + 32 * t + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const float x = tk < tokens ? acc[p][t][e] : 0.f;
                        s2[t] = fmaf(x, x, s2[t]);
                    }
                }
            }
            double sum = row_ok ? (double)s2[0] + (double)s2[1] : 0.0;
            // lanes with the same slot: the 16 of each row and both halves
            sum = wave_rows_sum_f64(sum);
            if (lane == 0)
                sm.wsum[g][2 * (pair0 + p)] = sum;
            if (lane == 16)
                sm.wsum[g][2 * (pair0 + p) + 1] = sum;
        }
        __syncthreads();
        if ((int)threadIdx.x < na) {
            const int a = threadIdx.x;
            double total = sm.wsum[0][a];
#pragma unroll
            for (int w = 1; w < 4; ++w)
                total += sm.wsum[w][a];
            partial[(int64_t)(a0 + a) * nblk + blk] = total;
        }
    }
};

// X in matrix-operand fragment order, so that every A-fragment load of the
// search is one contiguous 1 KB read (64 lanes x 16 bytes) instead of 64
// scattered 16-byte pieces of 32 token rows. Fragment f = (((tb * nsteps +
// si) * 8 + w) * 8 + s) * 64 + l holds, for token tb*256 + 32w + (l & 31) and
// input columns 128 si + 64 (l >> 5) + 8s .. + 7, the 8 stored values (zero
// past the last token). One thread per fragment; the writes are contiguous.
// Written by the preparation kernel below.
template <typename T>
__device__ __forceinline__ void xfrag_one(const T *__restrict__ X, int64_t tokens, int64_t in, int64_t nfrag,
                                          typename Vec8<T>::type *__restrict__ xf, int64_t f)
{
    typedef typename Vec8<T>::type V8;
    if (f >= nfrag)
        return;
    const int64_t nsteps = in / kStep;
    const int l = (int)(f & 63);
    const int s = (int)((f >> 6) & 7);
    const int w = (int)((f >> 9) & 7);
    const int64_t bs = f >> 12;   // tb * nsteps + si
    const int64_t tb = bs / nsteps, si = bs % nsteps;
    const int64_t t = tb * kTokPerBlock + w * kTokW + (l & 31);
    const int64_t col = si * kStep + 64 * (l >> 5) + 8 * s;
    xf[f] = t < tokens ? load8(X + t * in + col) : V8{};
}

// pass p covers candidates a0 = p*q + min(p, rem) .. + (q + (p < rem)).
template <typename T, int G, bool ASYM>
__global__ __launch_bounds__(kWaves * 64, 1) void k_search16(
    const T *__restrict__ W, const T *__restrict__ X, int64_t out, int64_t in, int64_t tokens,
    const float *__restrict__ s_tab, const float *__restrict__ inv_tab, const int32_t *__restrict__ unit,
    int n_alpha, int pass_q, int pass_rem, int bits, double *__restrict__ partial)
{
    // X: the fragment-ordered copy written by k_xfrag.
    __shared__ Smem<T> sm;
    const int64_t nrb = (out + kRows - 1) / kRows;
    const int64_t ntb = (tokens + kTokPerBlock - 1) / kTokPerBlock;
    const Coord k = coord(nrb, ntb);
    const int a0 = k.pass * pass_q + (k.pass < pass_rem ? k.pass : pass_rem);
    const int na = pass_q + (k.pass < pass_rem ? 1 : 0);
    const int wave = threadIdx.x >> 6;
    QParams qp;
    qp.levels = (float)((1 << (bits - 1)) - 1);
    qp.maxq = (float)((1 << bits) - 1);
    qp.inv_levels = 1.0f / qp.levels;
    qp.inv_maxq = 1.0f / qp.maxq;
    // Pairs: waves 0-3 take pairs 0-2, waves 4-7 the rest (3 or 2).
    const int npb = (na + 1) / 2;
    // Units: unit u < 8 goes to wave u; units 8.. (na > 8) go to waves
    // (u - 8 + sh2) mod 8 -- to the waves with fewer pairs (sh2 = 4) when
    // the second group has only 2 -- and unit u builds slot (u - u0) mod na,
    // where u0 = na - 8 puts slot 0 (alpha = 0 in the first pass) on a wave
    // that builds one unit.
    const int sh2 = npb == 5 ? 4 : 0;
    const int u0 = na >= 9 ? na - 8 : 0;
    const int ub = 8 + (wave - sh2 + 8) % 8;
    const int nunits = ub < na ? 2 : 1;
    int uslot[2];
    uslot[0] = (wave - u0 + na) % na;
    uslot[1] = (ub - u0 + na) % na;
    // Exact arithmetic for units whose scales are all ones. Both flags are
    // read (uslot[1] < na always), so the two loads share one round trip.
    const int32_t f0 = unit[a0 + uslot[0]], f1 = unit[a0 + uslot[1]];
    const bool ex = f0 != 0 || (nunits == 2 && f1 != 0);
    const int64_t nblk = nrb * ntb;
    const int64_t blk = k.rb * ntb + k.tb;
    typedef Search<T, G, ASYM> S;
#define AWQ_S16_RUN(NPW, U, EX)                                                                        \
    S::template run<NPW, U, EX>(sm, W, X, out, in, tokens, s_tab, inv_tab, a0, na, uslot, qp, k.rb, k.tb, \
                                nblk, blk, partial)
    if (wave < 4 || npb == 6) {
        if (nunits == 2)
            ex ? AWQ_S16_RUN(3, 2, true) : AWQ_S16_RUN(3, 2, false);
        else
            ex ? AWQ_S16_RUN(3, 1, true) : AWQ_S16_RUN(3, 1, false);
    } else {
        if (nunits == 2)
            ex ? AWQ_S16_RUN(2, 2, true) : AWQ_S16_RUN(2, 2, false);
        else
            ex ? AWQ_S16_RUN(2, 1, true) : AWQ_S16_RUN(2, 1, false);
    }
#undef AWQ_S16_RUN
}

// Preparation in one launch: blocks [0, nS) compute the s-table (one per
// 256 columns and candidate), blocks from nS on write the fragment-ordered
// copy of X (one thread per fragment).
template <typename T>
__global__ __launch_bounds__(256) void k_prepare16(const T *__restrict__ X, int64_t tokens, int64_t in,
                                                   int64_t nfrag, typename Vec8<T>::type *__restrict__ xf,
                                                   const float *__restrict__ xmag, int grid,
                                                   float *__restrict__ s_tab, float *__restrict__ inv_tab,
                                                   int32_t *__restrict__ unit, int64_t ncb)
{
    const int64_t b = blockIdx.x, nS = ncb * (grid + 1);
    if (b < nS) {
        s_table_block(xmag, in, grid, (int)(b / ncb), b % ncb, s_tab, inv_tab, unit);
        return;
    }
    xfrag_one<T>(X, tokens, in, nfrag, xf, (b - nS) * 256 + threadIdx.x);
}

template <typename T>
static hipError_t launch_prepare_typed(const void *X, const float *xmag, int64_t in, int64_t tokens,
                                       int grid, float *s_tab, float *inv_tab, int32_t *unit, void *xfrag,
                                       hipStream_t st)
{
    const int64_t ntb = (tokens + kTokPerBlock - 1) / kTokPerBlock;
    const int64_t nfrag = ntb * kTokPerBlock * in / 8;
    const int64_t ncb = (in + 255) / 256;
    const int64_t nblocks = ncb * (grid + 1) + (nfrag + 255) / 256;
    hipLaunchKernelGGL((k_prepare16<T>), dim3((unsigned)nblocks), dim3(256), 0, st, (const T *)X, tokens, in,
                       nfrag, (typename Vec8<T>::type *)xfrag, xmag, grid, s_tab, inv_tab, unit, ncb);
    return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_typed(const void *W, const void *xfrag, int64_t out, int64_t in, int64_t tokens,
                               const float *s_tab, const float *inv_tab, const int32_t *unit,
                               int n_alpha, int bits, int mode, double *partial, hipStream_t st)
{
    const int npass = (n_alpha + kSlots - 1) / kSlots;
    const int64_t nrb = (out + kRows - 1) / kRows;
    const int64_t ntb = (tokens + kTokPerBlock - 1) / kTokPerBlock;
    const dim3 grid((unsigned)(nrb * ntb * npass));
    const int q = n_alpha / npass, rem = n_alpha % npass;
    if (mode == AWQ_SYM)
        hipLaunchKernelGGL((k_search16<T, G, false>), grid, dim3(kWaves * 64), 0, st, (const T *)W,
                           (const T *)xfrag, out, in, tokens, s_tab, inv_tab, unit, n_alpha, q, rem, bits,
                           partial);
    else
        hipLaunchKernelGGL((k_search16<T, G, true>), grid, dim3(kWaves * 64), 0, st, (const T *)W,
                           (const T *)xfrag, out, in, tokens, s_tab, inv_tab, unit, n_alpha, q, rem, bits,
                           partial);
    return hipGetLastError();
}

}  // namespace s16

// One translation unit per (operand type, group size), compiled in
// parallel: AWQ_S16_T and AWQ_S16_G name the instantiation and the launcher
// it defines (declared in awq_internal.h).
#if defined(AWQ_S16_T) && defined(AWQ_S16_G)
#define AWQ_S16_CAT2(a, b, c) a##b##_g##c
#define AWQ_S16_CAT(a, b, c) AWQ_S16_CAT2(a, b, c)
hipError_t AWQ_S16_CAT(launch_search16_, AWQ_S16_T, AWQ_S16_G)(
    const void *W, const void *X, int64_t out, int64_t in, int64_t tokens, const float *s_tab,
    const float *inv_tab, const int32_t *unit, int n_alpha, int bits, int mode, double *partial,
    hipStream_t st)
{
    return s16::launch_typed<AWQ_S16_T, AWQ_S16_G>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha,
                                                   bits, mode, partial, st);
}
#if AWQ_S16_G == 128
#define AWQ_S16_CAT1(a, b) a##b
#define AWQ_S16_PREP(a, b) AWQ_S16_CAT1(a, b)
hipError_t AWQ_S16_PREP(launch_prepare16_, AWQ_S16_T)(const void *X, const float *xmag, int64_t in,
                                                       int64_t tokens, int grid, float *s_tab, float *inv_tab,
                                                       int32_t *unit, void *xfrag, hipStream_t st)
{
    return s16::launch_prepare_typed<AWQ_S16_T>(X, xmag, in, tokens, grid, s_tab, inv_tab, unit, xfrag, st);
}
#endif
#endif

}  // namespace awq
