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
// How: one block per (16 rows, one group), 8 waves of 32 tokens. The D tiles
// of up to 10 ratios at a time are built once (the exact quantizer's fp32
// operation order, correctly rounded quotients) into LDS in the B-operand
// layout of the fp32 MFMA, then every 256-token chunk of X multiplies them;
// each chunk's fp32 products are squared and summed in fp64. fp32 operands:
// this objective is per (row, group), with no averaging over rows to absorb
// the rounding of 16-bit operands, and matching the oracle's choices needs
// the group errors to ~1e-6. Sums run in a fixed order: bitwise reproducible.
#include "awq_internal.h"

#include <math.h>

#include <type_traits>

namespace awq {

constexpr int kClipWaves = 8;
constexpr int kClipTT = 2;                                  // 16-token tiles per wave
constexpr int kClipTok = kClipWaves * kClipTT * 16;         // tokens per chunk
constexpr int kClipChunk = 10;                              // ratios per LDS fill

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

template <typename TIn, int G, bool ASYM>
__global__ __launch_bounds__(kClipWaves * 64, 1) void k_clip_search(
    const TIn *__restrict__ W, const TIn *__restrict__ X, int64_t out, int64_t in, int64_t tokens,
    const float *__restrict__ s, int bits, int n_clip, float max_shrink, float *__restrict__ clip,
    double *__restrict__ sse_out)
{
    constexpr int KS = G / 32;
    __shared__ f32x8 tiles[kClipChunk][KS][64];
    __shared__ double red[kClipWaves][kClipChunk][16];
    __shared__ double sse_all[16][AWQ_MAX_CLIP];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;            // row inside the tile (B operand column)
    const int c = lane >> 4;            // 8-column slice of each 32-column step
    const int64_t row = (int64_t)blockIdx.x * 16 + r;
    const bool row_ok = row < out;
    const int64_t row_c = row_ok ? row : out - 1;
    const int64_t g0 = (int64_t)blockIdx.y * G;

    // This lane's scaled weights v = fp32(w s), the exact rounding error of
    // that product, perr = w s - v (an fma gives it exactly), and 1/s.
    float v[KS][8], perr[KS][8], inv[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float w[8];
        widen8<TIn>(load8(W + row_c * in + g0 + c * 8 + ks * 32), w);
        const f32x8 s8 = *reinterpret_cast<const f32x8 *>(s + g0 + c * 8 + ks * 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[ks][e] = w[e] * s8[e];
            perr[ks][e] = fmaf(w[e], s8[e], -v[ks][e]);
            inv[ks][e] = 1.0f / s8[e];
        }
    }
    // Group statistics of the row (the four lanes l, l^16, l^32, l^48).
    float amax = 0.f, lo = 0.f, hi = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            amax = fmaxf(amax, fabsf(v[ks][e]));
            lo = fminf(lo, v[ks][e]);
            hi = fmaxf(hi, v[ks][e]);
        }
    amax = clip_lanes4_max(amax);
    lo = clip_lanes4_min(lo);
    hi = clip_lanes4_max(hi);
    const float levels = (float)((1 << (bits - 1)) - 1);
    const float maxq = (float)((1 << bits) - 1);

    // D tile of ratio rt for this lane's slice: the dequantized value wh comes
    // from the exact quantizer's operation order; then
    //   d = wh / s - w = ((wh - v) - perr) / s
    // keeps the cancellation of wh against w s out of the rounding: about
    // 3 ulp of d instead of ulps of w.
    auto build = [&](float rt, f32x8 *dst) {
        float scale, zero = 0.f, xlo, xhi;
        if (!ASYM) {
            const float mx = rt * amax;
            scale = fmaxf(mx / levels, 1e-8f);
            xlo = -mx;
            xhi = mx;
        } else {
            xlo = rt * lo;
            xhi = rt * hi;
            scale = fmaxf((xhi - xlo) / maxq, 1e-8f);
            zero = rintf(-xlo / scale);
        }
        const float y = 1.0f / scale;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f32x8 d;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = fminf(fmaxf(v[ks][e], xlo), xhi);
                float q = rintf(clip_div(x, scale, y));
                float wh;
                if (!ASYM) {
                    q = fminf(fmaxf(q, -levels - 1.0f), levels);
                    wh = q * scale;
                } else {
                    q = fminf(fmaxf(q + zero, 0.0f), maxq);
                    wh = scale * (q - zero);
                }
                d[e] = ((wh - v[ks][e]) - perr[ks][e]) * inv[ks][e];
            }
            dst[ks * 64] = d;
        }
    };

    // X rows of this wave's tokens in a chunk, clamped to the last token.
    auto x_row = [&](int64_t t0, int tt) {
        int64_t t = t0 + wave * (kClipTT * 16) + tt * 16 + r;
        t = t < tokens ? t : tokens - 1;
        return X + t * in + g0 + c * 8;
    };

    for (int i0 = 0; i0 < n_clip; i0 += kClipChunk) {
        const int nc = n_clip - i0 < kClipChunk ? n_clip - i0 : kClipChunk;
        // tiles: ratio i0 + j by wave j % 8
        for (int j = wave; j < nc; j += kClipWaves)
            build(clip_ratio(i0 + j, n_clip, max_shrink), &tiles[j][0][lane]);
        __syncthreads();

        double sse[kClipChunk];
#pragma unroll
        for (int j = 0; j < kClipChunk; ++j)
            sse[j] = 0.0;
        for (int64_t t0 = 0; t0 < tokens; t0 += kClipTok) {
            f32x8 xa[kClipTT][KS];
#pragma unroll
            for (int tt = 0; tt < kClipTT; ++tt) {
                const TIn *xp = x_row(t0, tt);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    widen8<TIn>(load8(xp + ks * 32), reinterpret_cast<float *>(&xa[tt][ks]));
            }
            bool keep[kClipTT][4];
#pragma unroll
            for (int tt = 0; tt < kClipTT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    keep[tt][e] = t0 + wave * (kClipTT * 16) + tt * 16 + 4 * c + e < tokens;
#pragma unroll
            for (int j = 0; j < kClipChunk; ++j) {
                if (j < nc) {
#pragma unroll
                    for (int tt = 0; tt < kClipTT; ++tt) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const f32x8 b = tiles[j][ks][lane];
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[tt][ks][e], b[e], acc, 0, 0, 0);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const double a = keep[tt][e] ? (double)acc[e] : 0.0;
                            sse[j] += a * a;
                        }
                    }
                }
            }
        }
        // Lane l holds row l & 15: add the four lanes of each row, then the
        // waves in order.
#pragma unroll
        for (int j = 0; j < kClipChunk; ++j) {
            double a = sse[j];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            if (lane < 16)
                red[wave][j][lane] = a;
        }
        __syncthreads();
        if ((int)threadIdx.x < 16 * kClipChunk) {
            const int rr = threadIdx.x & 15, j = threadIdx.x >> 4;
            if (j < nc) {
                double tot = red[0][j][rr];
#pragma unroll
                for (int wv = 1; wv < kClipWaves; ++wv)
                    tot += red[wv][j][rr];
                sse_all[rr][i0 + j] = tot;
            }
        }
        __syncthreads();
    }
    // First strict minimum over the ratios of each row (a NaN never wins).
    if ((int)threadIdx.x < 16) {
        const int rr = threadIdx.x;
        const int64_t o = (int64_t)blockIdx.x * 16 + rr;
        if (o < out) {
            const int64_t ng = in / G;
            int best = 0;
            double be = INFINITY;
            for (int i = 0; i < n_clip; ++i) {
                const double e = sse_all[rr][i];
                if (e < be) {
                    be = e;
                    best = i;
                }
                if (sse_out)
                    sse_out[(o * ng + blockIdx.y) * n_clip + i] = e;
            }
            clip[o * ng + blockIdx.y] = clip_ratio(best, n_clip, max_shrink);
        }
    }
}

template <typename TIn, int G>
static hipError_t clip_typed(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,
                             const float *s, int bits, int mode, int n_clip, float max_shrink,
                             float *clip, double *sse, hipStream_t st)
{
    dim3 grid((unsigned)((out + 15) / 16), (unsigned)(in / G));
    if (mode == AWQ_SYM)
        hipLaunchKernelGGL((k_clip_search<TIn, G, false>), grid, dim3(kClipWaves * 64), 0, st,
                           (const TIn *)W, (const TIn *)X, out, in, tokens, s, bits, n_clip, max_shrink,
                           clip, sse);
    else
        hipLaunchKernelGGL((k_clip_search<TIn, G, true>), grid, dim3(kClipWaves * 64), 0, st,
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
