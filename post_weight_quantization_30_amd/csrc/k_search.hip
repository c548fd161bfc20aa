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
//  * One block = 16 output rows x 256 tokens x up to NA candidates, 4 waves.
//    The error needs the full-K sum of X D^T before squaring, so K cannot be
//    split: every candidate keeps its own fp32 accumulator tile
//    (NA x 4 tiles x 4 values = 336 registers per lane at NA = 21), which is
//    what limits the block to 16 rows x 256 tokens.
//  * Per group of G input columns: each wave builds the D tiles of its share
//    of the candidates (wave w takes candidates w, w+4, ...) in the exact
//    register layout of the MFMA B operand and stores them to LDS; after a
//    barrier every wave runs the 16x16x32 MFMAs of all candidates against its
//    own 64 tokens, whose X fragments stay in registers across candidates.
//    D is therefore generated once per (row, column, candidate) and reused by
//    all 256 tokens of the block.
//  * The group maximum (or min/max) of a row is in-lane over KS*8 values plus
//    two cross-lane steps: lanes r, r+16, r+32, r+48 hold the 4 column slices
//    of row r.
//  * Epilogue: squares summed in fp64 per lane, then a fixed butterfly per
//    wave and a fixed-order sum of the 4 waves: one fp64 partial per
//    (candidate, block); no atomics, so results are bitwise reproducible.
//  * The search may round differently from the exact quantizer (a reciprocal
//    multiply instead of the IEEE division, contracted multiply-adds, 16-bit
//    D): only the error is produced here, and its tolerance allows it. The
//    codes that get stored come from the exact kernel in k_pack.hip.
#include "awq_internal.h"

#include <math.h>

namespace awq {

constexpr int kWaves = 4;
constexpr int kTokPerWave = 64;
constexpr int kTT = kTokPerWave / 16;   // 16-token MFMA tiles per wave
constexpr int kMaxNA = 21;              // accumulator budget: 16 * NA registers per lane
constexpr int kLdsBudget = 86016;       // bytes of LDS for the D tiles of one group

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

// D for one candidate tile: q = rne(v / scale) (clamped to the asymmetric
// code range; the symmetric clamp of the exact quantizer can never bind,
// since |v| <= max|v| = L * scale), d = (q * scale - v) / s, rounded to the
// operand type and stored as this lane's 8-column slices of the B operand.
// The quotient is v * (1/scale); EXACT adds one residual step that makes it
// the correctly rounded quotient (Markstein: with y = RN(1/b) and
// q0 = RN(a*y), RN(q0 + RN(a - b*q0)*y) = RN(a/b)). EXACT is used when s is
// all ones (alpha = 0 or flat activations): v then holds the stored 16-bit
// weights, which land exactly on rounding ties often enough that the
// one-ulp difference of the plain product would flip codes the exact
// quantizer keeps. For other candidates v = w * s is unstructured and such
// flips have probability ~1e-7 per weight.
template <typename TOp, int KS, bool ASYM, bool EXACT>
__device__ __forceinline__ void emit_tile(const float (&v)[KS][8], float scale, float rs, float zlo,
                                          float zhi, const float *__restrict__ irow,
                                          typename Vec8<TOp>::type *dst)
{
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

template <typename TOp, int G>
struct SearchShape {
    static constexpr int KS = G / 32;                                  // 32-column MFMA steps per group
    static constexpr int kTileBytes = KS * 64 * (int)sizeof(typename Vec8<TOp>::type);
    static constexpr int NA = kLdsBudget / kTileBytes < kMaxNA ? kLdsBudget / kTileBytes : kMaxNA;
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

// TIn: stored element type of W and X. TOp: MFMA operand type (TIn for the
// 16-bit path, float for the fp32-operand path).
template <typename TIn, typename TOp, int G>
__global__ __launch_bounds__(256, 1) void k_search(
    const TIn *__restrict__ W, const TIn *__restrict__ X, int64_t out, int64_t in, int64_t tokens,
    const float *__restrict__ s_tab, const float *__restrict__ inv_tab,
    const int32_t *__restrict__ unit, int n_alpha, int bits, int mode, double *__restrict__ partial)
{
    typedef typename Vec8<TOp>::type V8;
    constexpr int KS = SearchShape<TOp, G>::KS;
    constexpr int NA = SearchShape<TOp, G>::NA;

    __shared__ V8 dtile[NA][KS][64];
    __shared__ double wsum[kWaves][NA];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;           // row inside the tile (B operand column n)
    const int c = lane >> 4;           // which 8-column slice of a 32-column step
    const int64_t row = (int64_t)blockIdx.x * 16 + r;
    const bool row_ok = row < out;
    const int64_t row_c = row_ok ? row : out - 1;
    const int64_t tok0 = (int64_t)blockIdx.y * kTokPerBlock + wave * kTokPerWave;
    const int a0 = blockIdx.z * NA;
    const int na = n_alpha - a0 < NA ? n_alpha - a0 : NA;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.y;
    const int64_t blk = (int64_t)blockIdx.x * gridDim.y + blockIdx.y;

    const float levels = (float)((1 << (bits - 1)) - 1);
    const float maxq = (float)((1 << bits) - 1);

    f32x4 acc[NA][kTT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
            acc[a][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const V8 zero8 = {};
    for (int i = threadIdx.x; i < (NA - na) * KS * 64; i += blockDim.x)
        (&dtile[na][0][0])[i] = zero8;

    for (int64_t k0 = 0; k0 < in; k0 += G) {
        // X fragments of this wave's 64 tokens (A operand), reused by every candidate.
        // Tokens past the end read the last token's row (always in bounds)
        // and are replaced by zeros, so they add nothing to the error.
        V8 xa[kTT][KS];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) {
            const int64_t t = tok0 + tt * 16 + r;
            const int64_t tc = t < tokens ? t : tokens - 1;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const V8 x = ToOp<TIn, TOp>::run(load8(X + tc * in + k0 + ks * 32 + c * 8));
                xa[tt][ks] = t < tokens ? x : zero8;
            }
        }
        // This lane's weights: row `row`, columns k0 + 32 ks + 8 c + (0..7);
        // rows past the end are zero (their D is zero and adds nothing).
        float w[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            widen8<TIn>(load8(W + row_c * in + k0 + ks * 32 + c * 8), w[ks]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[ks][i] = row_ok ? w[ks][i] : 0.f;
        }

        // Build the D tiles of this wave's candidates.
        for (int a = wave; a < na; a += kWaves) {
            const float *srow = s_tab + (int64_t)(a0 + a) * in + k0 + c * 8;
            const float *irow = inv_tab + (int64_t)(a0 + a) * in + k0 + c * 8;
            float v[KS][8];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f32x8 s8 = *reinterpret_cast<const f32x8 *>(srow + ks * 32);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[ks][i] = w[ks][i] * s8[i];
            }
            float scale, rs, zlo = 0.f, zhi = 0.f;
            if (mode == AWQ_SYM) {
                float m = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        m = fmaxf(m, fabsf(v[ks][i]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                scale = fmaxf(m / levels, 1e-8f);
                rs = 1.0f / scale;
                zlo = -levels - 1.0f;
                zhi = levels;
            } else {
                float lo = 0.f, hi = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        lo = fminf(lo, v[ks][i]);
                        hi = fmaxf(hi, v[ks][i]);
                    }
                lo = fminf(lo, __shfl_xor(lo, 16));
                lo = fminf(lo, __shfl_xor(lo, 32));
                hi = fmaxf(hi, __shfl_xor(hi, 16));
                hi = fmaxf(hi, __shfl_xor(hi, 32));
                scale = fmaxf((hi - lo) / maxq, 1e-8f);
                rs = 1.0f / scale;
                const float zero = rintf(-lo / scale);
                zlo = -zero;
                zhi = maxq - zero;
            }
            V8 *dst = &dtile[a][0][lane];
            const bool exact = unit[a0 + a] != 0;
            if (mode == AWQ_SYM) {
                if (exact)
                    emit_tile<TOp, KS, false, true>(v, scale, rs, zlo, zhi, irow, dst);
                else
                    emit_tile<TOp, KS, false, false>(v, scale, rs, zlo, zhi, irow, dst);
            } else {
                if (exact)
                    emit_tile<TOp, KS, true, true>(v, scale, rs, zlo, zhi, irow, dst);
                else
                    emit_tile<TOp, KS, true, false>(v, scale, rs, zlo, zhi, irow, dst);
            }
        }
        __syncthreads();

        // Unconditional over all NA slots: a branch around an MFMA would make
        // its accumulator a control-flow merge, which the compiler resolves
        // by copying every accumulator out of and back into AGPRs each group.
        // Slots >= na hold zero tiles (cleared once below) and are never read out.
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const V8 b = dtile[a][ks][lane];
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt)
                    acc[a][tt] = Mfma<TOp>::run(xa[tt][ks], b, acc[a][tt]);
            }
        }
        __syncthreads();
    }

    // Sum of squares: exact fp64 squares of the fp32 accumulators, fixed order.
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        if (a < na) {
            double sum = 0.0;
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double x = (double)acc[a][tt][e];
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
        const double total = ((wsum[0][a] + wsum[1][a]) + wsum[2][a]) + wsum[3][a];
        partial[(int64_t)(a0 + a) * nblk + blk] = total;
    }
}

// Per candidate: fixed-order reduction of the block partials (each thread a
// contiguous stretch, then a fixed tree), mse = sse / (tokens * out).
__global__ __launch_bounds__(256) void k_reduce(const double *__restrict__ partial, int64_t nblk,
                                               double denom, double *__restrict__ mse)
{
    __shared__ double buf[256];
    const int a = blockIdx.x;
    const int64_t per = (nblk + 255) / 256;
    const int64_t b0 = threadIdx.x * per;
    const int64_t b1 = b0 + per < nblk ? b0 + per : nblk;
    double s = 0.0;
    for (int64_t b = b0; b < b1; ++b)
        s += partial[(int64_t)a * nblk + b];
    buf[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h)
            buf[threadIdx.x] += buf[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        mse[a] = buf[0] / denom;
}

// First strict minimum over the candidates (a NaN never compares below), then
// s_best = that row of the s-table, or all ones when nothing is finite.
__global__ __launch_bounds__(1024) void k_argmin(const double *__restrict__ mse, int n_alpha,
                                                 const float *__restrict__ s_tab, int64_t in,
                                                 int32_t *__restrict__ best, float *__restrict__ s_best)
{
    __shared__ int sbest;
    if (threadIdx.x == 0) {
        int b = -1;
        double be = INFINITY;
        for (int k = 0; k < n_alpha; ++k) {
            const double e = mse[k];
            if (e < be) {
                be = e;
                b = k;
            }
        }
        sbest = b;
        *best = b;
    }
    __syncthreads();
    const int b = sbest;
    for (int64_t j = threadIdx.x; j < in; j += blockDim.x)
        s_best[j] = b >= 0 ? s_tab[(int64_t)b * in + j] : 1.0f;
}

template <typename TIn, typename TOp, int G>
static hipError_t search_typed(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,
                               const float *s_tab, const float *inv_tab, const int32_t *unit,
                               int n_alpha, int bits, int mode, double *partial, hipStream_t st)
{
    constexpr int NA = SearchShape<TOp, G>::NA;
    dim3 grid((unsigned)((out + 15) / 16), (unsigned)((tokens + kTokPerBlock - 1) / kTokPerBlock),
              (unsigned)((n_alpha + NA - 1) / NA));
    hipLaunchKernelGGL((k_search<TIn, TOp, G>), grid, dim3(256), 0, st, (const TIn *)W,
                       (const TIn *)X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, mode,
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

hipError_t launch_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                         int64_t tokens, const float *s_tab, const float *inv_tab,
                         const int32_t *unit, int n_alpha, int bits, int group, int mode,
                         double *partial, hipStream_t st)
{
    const bool wide = search_uses_fp32_operands(dtype, out, tokens);
    switch (dtype) {
    case AWQ_F32:
        return search_group<float, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
    case AWQ_F16:
        return wide ? search_group<f16, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st)
                    : search_group<f16, f16>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
    default:
        return wide ? search_group<bf16, float>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st)
                    : search_group<bf16, bf16>(W, X, out, in, tokens, s_tab, inv_tab, unit, n_alpha, bits, group, mode, partial, st);
    }
}

hipError_t launch_reduce_argmin(const double *partial, int64_t nblk, int n_alpha, int64_t out,
                                int64_t tokens, int64_t in, const float *s_tab, double *mse,
                                int32_t *best, float *s_best, hipStream_t st)
{
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)n_alpha), dim3(256), 0, st, partial, nblk,
                       (double)tokens * (double)out, mse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_argmin, dim3(1), dim3(1024), 0, st, (const double *)mse, n_alpha, s_tab,
                       in, best, s_best);
    return hipGetLastError();
}

}  // namespace awq
