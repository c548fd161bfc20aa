// k_clip.hip -- the clipping-range search that follows the alpha search.
//
// What is computed ("AWQ (activation-aware weight quantization)",
// "Simplifications"; "AWQ vs GPTQ Quantization Architectures Compared", "AWQ:
// move the error away from what matters": a second search shrinks each
// group's clipping range a little when that lowers output error; the numbers
// are this library's readings): for every output row o, group g of G columns
// and ratio r_i = fl32(1 - i * max_shrink / n_clip), i = 0..n_clip-1, the
// group's quantizer range is scaled by r_i (symmetric [-r A, r A]; asymmetric
// [r lo, r hi] with 0 included), the scaled weights v = w * s are clamped
// into it and quantized with that range's scale (and zero), and the group's
// own squared output error
//     sse[o][g][i] = sum_t ( sum_{j in g} X[t, j] * (Q(v)_j / s_j - w_j) )^2
// is formed; clip[o][g] = r of the first strict minimum.
//
// How: one block per (16 rows, one group), 8 waves, two blocks per compute
// unit (at most 128 VGPRs per lane, so that one block's loads and barriers
// hide behind the other's work). Each wave owns whole ratios (ratio j by wave
// j % 8, in rounds of RW ratios per wave: one at G = 128, more for smaller
// groups): it builds their D tiles d = Q(v)/s - w in fp32 (the exact
// quantizer's operation order, correctly rounded quotients) and keeps them in
// registers as MFMA B operands; X passes through LDS in chunks of 256 tokens
// (128 for fp32), which stay resident across rounds when one chunk holds all
// tokens, and every wave multiplies each 16-token tile of it by its tiles and
// squares the results.
//
// Operand precision. Each choice rests on one (row, group) error with no
// averaging over rows, and adjacent ratios' errors often differ by only 1e-4
// relative, so D is carried at (near) fp32 precision:
//   * fp16 X: D (scaled by a power of two 2^k per row, chosen from a bound on
//     |d| so that 2^k |d| stays below 2^14) is split into hi = fp16(d') and
//     lo = fp16(d' - hi): 22 significant bits, relative error <= 2^-22 (plus
//     an absolute 2^-25 in d' units where lo falls below the fp16 normal
//     range); two fp16 MFMAs against the exact fp16 X;
//   * bf16 X: D = hi + mid + lo exactly, three bf16 parts cut by truncation
//     (8 + 8 + 8 bits cover fp32's 24); three bf16 MFMAs;
//   * fp32 X: fp32 MFMAs on D itself.
// Every product of 16-bit parts is exact in fp32; the tile sums accumulate in
// fp32 over the group, the four squares of a lane's tile are summed in fp32
// and then added in fp64. Sums run in a fixed order: bitwise reproducible, and
// a row's result does not depend on the block that holds it.
#include "awq_internal.h"

#include <math.h>

namespace awq {

constexpr int kClipWaves = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kClipThreads = kClipWaves * 64;

// Max / min over the four lanes l, l^16, l^32, l^48 (one row's slices).
__device__ __forceinline__ float clip_lanes4_max(float m)
{
    m = fmaxf(m, __shfl_xor(m, 16));
    return fmaxf(m, __shfl_xor(m, 32));
}
__device__ __forceinline__ float clip_lanes4_min(float m)
{
    m = fminf(m, __shfl_xor(m, 16));
    return fminf(m, __shfl_xor(m, 32));
}

// a / b correctly rounded for finite b > 0 and y = RN(1/b): q0 = a*y, then two
// fma residual steps (the first makes q faithful, the second exact).
__device__ __forceinline__ float clip_div(float a, float b, float y)
{
    float q = a * y;
    q = fmaf(fmaf(-b, q, a), y, q);
    return fmaf(fmaf(-b, q, a), y, q);
}

__device__ __forceinline__ float clip_ratio(int i, int n_clip, float max_shrink)
{
    return (float)(1.0 - (double)i * (double)max_shrink / (double)n_clip);
}

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// How D reaches the matrix cores for each input type: NP parts of 8 values
// per lane and 32-column step, and the MFMA sequence of one step.
template <typename TIn> struct ClipMma;

template <> struct ClipMma<f16> {
    static constexpr int NP = 2;
    static constexpr bool SCALED = true;
    typedef f16x8 xvec;
    typedef f16x8 dvec;
    static __device__ __forceinline__ void split(const float *d, dvec *p)
    {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            // d opaque: hi must be the one narrowing of the rounded d that
            // both the stored part and the difference use.
            const f32x2 x = {opaque(d[e]), opaque(d[e + 1])};
            const f16x2 h = __builtin_convertvector(x, f16x2);
            // x - f32(hi) in one v_fma_mix_f32 each (the fp16 half widened
            // exactly, times -1, plus x, rounded once): the difference is
            // exact in fp32, so this is the same value as widen-then-subtract
            const uint32_t hp = __builtin_bit_cast(uint32_t, h);
            const float m1 = -1.0f;
            float l0, l1;
            asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(l0) : "v"(hp), "v"(m1), "v"(x[0]));
            asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(l1)
                : "v"(hp), "v"(m1), "v"(x[1]));
            const f16x2 l = __builtin_convertvector(f32x2{l0, l1}, f16x2);
            p[0][e] = h[0];
            p[0][e + 1] = h[1];
            p[1][e] = l[0];
            p[1][e + 1] = l[1];
        }
    }
    static __device__ __forceinline__ f32x4 mma(const xvec &a, const dvec *b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[0], c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[1], c, 0, 0, 0);
    }
};

template <> struct ClipMma<bf16> {
    static constexpr int NP = 3;
    static constexpr bool SCALED = false;
    typedef bf16x8 xvec;
    typedef bf16x8 dvec;
    // hi = d with the low 16 bits cleared, mid likewise of d - hi, lo = the
    // rest: each difference is exact and lo has at most 8 significant bits,
    // so hi + mid + lo == d.
    static __device__ __forceinline__ void split(const float *d, dvec *p)
    {
        uint32_t u[3][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            uint32_t b0[3], b1[3];
            float x0 = d[e], x1 = d[e + 1];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                b0[k] = fbits(x0);
                b1[k] = fbits(x1);
                x0 -= bitsf(b0[k] & 0xffff0000u);
                x1 -= bitsf(b1[k] & 0xffff0000u);
            }
#pragma unroll
            for (int k = 0; k < 3; ++k)
                u[k][e / 2] = __builtin_amdgcn_perm(b1[k], b0[k], 0x07060302u);
        }
#pragma unroll
        for (int k = 0; k < 3; ++k)
            p[k] = __builtin_bit_cast(dvec, u[k]);
    }
    static __device__ __forceinline__ f32x4 mma(const xvec &a, const dvec *b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[2], c, 0, 0, 0);
    }
};

template <> struct ClipMma<float> {
    static constexpr int NP = 1;
    static constexpr bool SCALED = false;
    typedef f32x8 xvec;
    typedef f32x8 dvec;
    static __device__ __forceinline__ void split(const float *d, dvec *p)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            p[0][e] = d[e];
    }
    // Column c*8+e of the lane's slice is the k index of the e-th 4-deep step.
    static __device__ __forceinline__ f32x4 mma(const xvec &a, const dvec *b, f32x4 c)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[0][e], c, 0, 0, 0);
        return c;
    }
};

// Ratios a wave holds at once (D registers: RW * KS * NP * 8 values per lane).
template <typename TIn, int G>
struct ClipShape {
    static constexpr int KS = G / 32;
    static constexpr int RW = ClipMma<TIn>::NP == 3 ? (KS == 1 ? 2 : 1) : (4 / KS > 0 ? 4 / KS : 1);
    static constexpr int E = (int)sizeof(TIn);
    static constexpr int TOKC = E == 4 ? 128 : 256;            // tokens per LDS chunk
    static constexpr int ROWB = G * E + 16;                     // LDS bytes per token (16-byte pad)
    static constexpr int P16 = G * E / 16;                      // 16-byte pieces per token
    static constexpr int NPRE = TOKC * P16 / kClipThreads;      // pieces per thread per chunk
    static_assert(TOKC * P16 % kClipThreads == 0, "chunk must split evenly over the block");
};

// Calls f(std::integral_constant-like tag) with tag::value == nv, nv in [0, N].
template <int V> struct ClipNv { static constexpr int value = V; };
template <int N, typename F>
__device__ __forceinline__ void clip_with_nv(int nv, F &&f)
{
    if constexpr (N >= 0) {
        if (nv == N) {
            f(ClipNv<N>{});
            return;
        }
        clip_with_nv<N - 1>(nv, f);
    }
}

// One 16-token tile against the first NV ratios of the wave: the NV
// accumulator chains interleaved (each still summed in ks order), then the
// four squares of each lane summed in fp32 and added to the fp64 total.
template <int NV, typename M, int RW, int KS>
__device__ __forceinline__ void clip_tile(const typename M::xvec (&a)[KS],
                                          const typename M::dvec (&D)[RW][KS][M::NP], double (&sse)[RW])
{
    if constexpr (NV > 0) {
        f32x4 acc[NV];
#pragma unroll
        for (int m = 0; m < NV; ++m)
            acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int m = 0; m < NV; ++m)
                acc[m] = M::mma(a[ks], D[m][ks], acc[m]);
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            float p = acc[m][0] * acc[m][0];
            p = fmaf(acc[m][1], acc[m][1], p);
            p = fmaf(acc[m][2], acc[m][2], p);
            p = fmaf(acc[m][3], acc[m][3], p);
            sse[m] += (double)p;
        }
    }
}

template <typename TIn, int G, bool ASYM>
__global__ __launch_bounds__(kClipThreads, 2) void k_clip_search(
    const TIn *__restrict__ W, const TIn *__restrict__ X, int64_t out, int64_t in, int64_t tokens,
    const float *__restrict__ s, int bits, int n_clip, float max_shrink, float *__restrict__ clip,
    double *__restrict__ sse_out)
{
    typedef ClipMma<TIn> M;
    typedef ClipShape<TIn, G> S;
    constexpr int KS = S::KS, RW = S::RW, NP = M::NP;
    __shared__ __align__(16) unsigned char xs[S::TOKC * S::ROWB];
    __shared__ double sse_all[16][AWQ_MAX_CLIP];
    __shared__ __align__(16) float s_l[G];
    __shared__ __align__(16) float inv_l[G];
    __shared__ float ratio_l[AWQ_MAX_CLIP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;            // D: output row of the tile; X: token of the tile
    const int c = lane >> 4;            // 8-column slice of each 32-column step
    const int64_t row = (int64_t)blockIdx.x * 16 + r;
    const int64_t row_c = row < out ? row : out - 1;
    const int64_t g0 = (int64_t)blockIdx.y * G;

    // X chunks: piece p = tid + 512 i is token p / P16, bytes (p % P16) * 16 of
    // the group's columns; tokens past the end read the last token and are
    // stored as zeros (a zero row adds exactly 0 to every sum).
    u32x4 pre[S::NPRE];
#define CLIP_X_FETCH(T0)                                                                           \
    do {                                                                                           \
        _Pragma("unroll") for (int i_ = 0; i_ < S::NPRE; ++i_)                                     \
        {                                                                                          \
            const int p_ = tid + kClipThreads * i_;                                                \
            int64_t t_ = (T0) + p_ / S::P16;                                                       \
            t_ = t_ < tokens ? t_ : tokens - 1;                                                    \
            pre[i_] = *reinterpret_cast<const u32x4 *>(                                            \
                reinterpret_cast<const unsigned char *>(X + t_ * in + g0) + (p_ % S::P16) * 16);   \
        }                                                                                          \
    } while (0)
#define CLIP_X_STASH(T0)                                                                           \
    do {                                                                                           \
        _Pragma("unroll") for (int i_ = 0; i_ < S::NPRE; ++i_)                                     \
        {                                                                                          \
            const int p_ = tid + kClipThreads * i_;                                                \
            const bool live_ = (T0) + p_ / S::P16 < tokens;                                        \
            const u32x4 z_ = {0u, 0u, 0u, 0u};                                                     \
            *reinterpret_cast<u32x4 *>(xs + (p_ / S::P16) * S::ROWB + (p_ % S::P16) * 16) =        \
                live_ ? pre[i_] : z_;                                                              \
        }                                                                                          \
    } while (0)

    const TIn *wrow = W + row_c * in + g0 + c * 8;
    if (tid < G) {
        const float sv = s[g0 + tid];
        s_l[tid] = sv;
        inv_l[tid] = 1.0f / sv;
    }
    if (tid >= kClipThreads - AWQ_MAX_CLIP)
        ratio_l[tid - (kClipThreads - AWQ_MAX_CLIP)] = clip_ratio(tid - (kClipThreads - AWQ_MAX_CLIP), n_clip, max_shrink);
    __syncthreads();

    // Group statistics of the row (lanes l, l^16, l^32, l^48), and a bound on
    // |d|: |Q(v)| <= 2 |clamped v| <= 2 A, so |d| <= (3 A + |perr|) / s up to
    // a few roundings; (4 A + max |perr|) * max(1/s) covers it.
    float amax = 0.f, lo = 0.f, hi = 0.f, pmax = 0.f, imax = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float w[8];
        widen8<TIn>(load8(wrow + ks * 32), w);
        const f32x8 s8 = *reinterpret_cast<const f32x8 *>(s_l + c * 8 + ks * 32);
        const f32x8 i8 = *reinterpret_cast<const f32x8 *>(inv_l + c * 8 + ks * 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = w[e] * s8[e];
            amax = fmaxf(amax, fabsf(v));
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
            pmax = fmaxf(pmax, fabsf(fmaf(w[e], s8[e], -v)));
            imax = fmaxf(imax, i8[e]);
        }
    }
    amax = clip_lanes4_max(amax);
    lo = clip_lanes4_min(lo);
    hi = clip_lanes4_max(hi);
    pmax = clip_lanes4_max(pmax);
    imax = clip_lanes4_max(imax);
    const float levels = (float)((1 << (bits - 1)) - 1);
    const float maxq = (float)((1 << bits) - 1);
    const float qthr = 0.5f - ldexpf(1.0f, bits - 21);

    // Power-of-two scale of the row's D (fp16 parts only): 2^k |d| < 2^14,
    // and 2^k / s stays finite.
    float p2k = 1.0f;
    double back = 1.0;
    if (M::SCALED) {
        int eb, ei;
        frexpf((4.0f * amax + pmax) * imax, &eb);
        frexpf(imax, &ei);
        int k = 14 - eb;
        k = k < 126 - ei ? k : 126 - ei;
        k = k > -126 ? k : -126;
        p2k = ldexpf(1.0f, k);
        back = ldexp(1.0, -2 * k);
    }

    const int nch = (int)((tokens + S::TOKC - 1) / S::TOKC);
    for (int r0 = 0; r0 < n_clip; r0 += kClipWaves * RW) {
        // This wave's ratios j = r0 + wave + 8 m, m < nv, and their quantizer
        // parameters (per row).
        int nv = (n_clip - r0 - wave + kClipWaves - 1) / kClipWaves;
        nv = nv < 0 ? 0 : (nv > RW ? RW : nv);
        float scale[RW], y[RW], zero[RW], xlo[RW], xhi[RW];
#pragma unroll
        for (int m = 0; m < RW; ++m) {
            const int j = r0 + wave + kClipWaves * m;
            const float rt = ratio_l[j < n_clip ? j : 0];
            zero[m] = 0.f;
            if (!ASYM) {
                const float mx = rt * amax;
                scale[m] = fmaxf(mx / levels, 1e-8f);
                xlo[m] = -mx;
                xhi[m] = mx;
            } else {
                xlo[m] = rt * lo;
                xhi[m] = rt * hi;
                scale[m] = fmaxf((xhi[m] - xlo[m]) / maxq, 1e-8f);
                zero[m] = rintf(-xlo[m] / scale[m]);
            }
            y[m] = 1.0f / scale[m];
        }

        // D tiles: the dequantized value wh from the exact quantizer's
        // operation order, then d = ((wh - v) - perr) / s with perr = w s - v
        // exact (one fma): about 3 ulp of d, the cancellation of wh against
        // w s kept out of the rounding.
        typename M::dvec D[RW][KS][NP];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float w[8], v[8], perr[8], inv[8];
            widen8<TIn>(load8(wrow + ks * 32), w);
            const f32x8 s8 = *reinterpret_cast<const f32x8 *>(s_l + c * 8 + ks * 32);
            const f32x8 i8 = *reinterpret_cast<const f32x8 *>(inv_l + c * 8 + ks * 32);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[e] = w[e] * s8[e];
                perr[e] = fmaf(w[e], s8[e], -v[e]);
                inv[e] = i8[e] * p2k;
            }
#pragma unroll
            for (int m = 0; m < RW; ++m) {
                if (m < nv) {
                    // rne of the correctly rounded quotient x / scale: from
                    // x * y, unless some lane's x * y lies within
                    // 2^(bits-21) of a half-integer (|x / scale| <= 2^bits;
                    // x * y lies within 1.5 * 2^(bits-23) of the quotient),
                    // in which case the wave takes the two residual steps
                    float xq[8], qq[8], dmax = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xq[e] = __builtin_amdgcn_fmed3f(v[e], xlo[m], xhi[m]);
                        const float u = xq[e] * y[m];
                        qq[e] = rintf(u);
                        dmax = fmaxf(dmax, fabsf(u - qq[e]));
                    }
                    if (__builtin_amdgcn_ballot_w64(dmax >= qthr) != 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            qq[e] = rintf(clip_div(xq[e], scale[m], y[m]));
                    }
                    float d[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float q = qq[e];
                        float wh;
                        if (!ASYM) {
                            // |x| <= mx and scale >= RN(mx / levels) give
                            // |q| <= levels: the code clamp never binds.
                            wh = q * scale[m];
                        } else {
                            q = __builtin_amdgcn_fmed3f(q + zero[m], 0.0f, maxq);
                            wh = scale[m] * (q - zero[m]);
                        }
                        d[e] = ((wh - v[e]) - perr[e]) * inv[e];
                    }
                    M::split(d, D[m][ks]);
                }
            }
        }

        double sse[RW];
#pragma unroll
        for (int m = 0; m < RW; ++m)
            sse[m] = 0.0;
        for (int ch = 0; ch < nch; ++ch) {
            const int64_t t0 = (int64_t)ch * S::TOKC;
            if (!(nch == 1 && r0 > 0)) {          // a single chunk stays resident
                CLIP_X_FETCH(t0);
                if (r0 > 0 || ch > 0)
                    __syncthreads();              // the previous chunk is no longer read
                CLIP_X_STASH(t0);
                __syncthreads();
            }
            const int ntile = (int)((tokens - t0 + 15) / 16 < S::TOKC / 16 ? (tokens - t0 + 15) / 16 : S::TOKC / 16);
            for (int tt = 0; tt < ntile; ++tt) {
                typename M::xvec a[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    a[ks] = *reinterpret_cast<const typename M::xvec *>(
                        xs + (tt * 16 + r) * S::ROWB + (ks * 32 + c * 8) * S::E);
                clip_with_nv<RW>(nv, [&](auto tag) {
                    clip_tile<decltype(tag)::value, M, RW, KS>(a, D, sse);
                });
            }
        }
        // Lane l holds row l & 15 for tokens 4 (l >> 4) .. +3 of every tile:
        // add the four lanes of each row.
#pragma unroll
        for (int m = 0; m < RW; ++m) {
            const int j = r0 + wave + kClipWaves * m;
            if (m < nv) {
                double a = sse[m];
                a += __shfl_xor(a, 16);
                a += __shfl_xor(a, 32);
                if (lane < 16)
                    sse_all[lane][j] = a * back;
            }
        }
    }
    __syncthreads();
    // First strict minimum over the ratios of each row (a NaN never wins).
    if (tid < 16) {
        const int64_t o = (int64_t)blockIdx.x * 16 + tid;
        if (o < out) {
            const int64_t ng = in / G;
            int best = 0;
            double be = INFINITY;
            for (int i = 0; i < n_clip; ++i) {
                const double e = sse_all[tid][i];
                if (e < be) {
                    be = e;
                    best = i;
                }
                if (sse_out)
                    sse_out[(o * ng + blockIdx.y) * n_clip + i] = e;
            }
            clip[o * ng + blockIdx.y] = ratio_l[best];
        }
    }
#undef CLIP_X_FETCH
#undef CLIP_X_STASH
}

template <typename TIn, int G>
static hipError_t clip_typed(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,
                             const float *s, int bits, int mode, int n_clip, float max_shrink,
                             float *clip, double *sse, hipStream_t st)
{
    dim3 grid((unsigned)((out + 15) / 16), (unsigned)(in / G));
    if (mode == AWQ_SYM)
        hipLaunchKernelGGL((k_clip_search<TIn, G, false>), grid, dim3(kClipThreads), 0, st,
                           (const TIn *)W, (const TIn *)X, out, in, tokens, s, bits, n_clip, max_shrink,
                           clip, sse);
    else
        hipLaunchKernelGGL((k_clip_search<TIn, G, true>), grid, dim3(kClipThreads), 0, st,
                           (const TIn *)W, (const TIn *)X, out, in, tokens, s, bits, n_clip, max_shrink,
                           clip, sse);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t clip_group(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,
                             const float *s, int bits, int group, int mode, int n_clip,
                             float max_shrink, float *clip, double *sse, hipStream_t st)
{
    switch (group) {
    case 32: return clip_typed<TIn, 32>(W, X, out, in, tokens, s, bits, mode, n_clip, max_shrink, clip, sse, st);
    case 64: return clip_typed<TIn, 64>(W, X, out, in, tokens, s, bits, mode, n_clip, max_shrink, clip, sse, st);
    default: return clip_typed<TIn, 128>(W, X, out, in, tokens, s, bits, mode, n_clip, max_shrink, clip, sse, st);
    }
}

hipError_t launch_clip_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                              int64_t tokens, const float *s, int bits, int group, int mode,
                              int n_clip, float max_shrink, float *clip, double *sse, hipStream_t st)
{
    switch (dtype) {
    case AWQ_F32: return clip_group<float>(W, X, out, in, tokens, s, bits, group, mode, n_clip, max_shrink, clip, sse, st);
    case AWQ_F16: return clip_group<f16>(W, X, out, in, tokens, s, bits, group, mode, n_clip, max_shrink, clip, sse, st);
    default: return clip_group<bf16>(W, X, out, in, tokens, s, bits, group, mode, n_clip, max_shrink, clip, sse, st);
    }
}

}  // namespace awq
