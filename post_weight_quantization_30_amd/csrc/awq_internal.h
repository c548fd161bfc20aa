// awq_internal.h -- private declarations shared by the HIP sources of libawq.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "awq.h"

namespace awq {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight consecutive elements of one row: the unit every kernel loads, and the
// per-lane operand of one 16x16x32 MFMA step.
template <typename T> struct Vec8;
template <> struct Vec8<float> { typedef f32x8 type; };
template <> struct Vec8<f16> { typedef f16x8 type; };
template <> struct Vec8<bf16> { typedef bf16x8 type; };

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type load8(const T *p)
{
    return *reinterpret_cast<const typename Vec8<T>::type *>(p);
}

// Exact widening of 8 stored elements to fp32.
template <typename T>
__device__ __forceinline__ void widen8(const typename Vec8<T>::type &v, float *f)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = static_cast<float>(v[i]);
}

// An fp32 value made opaque to instruction selection. Around a multiply the
// compiler otherwise folds an fp16 widening or narrowing into a mixed-precision
// fma with a +0 addend: that turns -0 * s into +0 and rounds the exact product
// once to fp16 instead of first to fp32 -- and it may do so for one use of a
// narrowed value and not for another, so that the "same" fp16 value differs
// between them.
__device__ __forceinline__ float opaque(float x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Workspace layout of awq_search (each part 256-byte aligned).
struct SearchWs {
    size_t s_off, inv_off, unit_off, part_off, xf_off, total;
    int64_t nblk;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kRowsPerBlock = 16;    // output rows per search block (one MFMA N tile)
constexpr int kTokPerBlock = 256;    // calibration tokens per search block (8 waves x 32)
// Below these sizes the search runs with fp32 MFMA operands (see k_search.hip).
constexpr int64_t kMinRows16 = 256;
constexpr int64_t kMinTokens16 = 16;

inline SearchWs search_ws_layout(int64_t out, int64_t in, int64_t tokens, int grid)
{
    SearchWs w;
    const int64_t na = (int64_t)grid + 1;
    w.nblk = ((out + kRowsPerBlock - 1) / kRowsPerBlock) * ((tokens + kTokPerBlock - 1) / kTokPerBlock);
    w.s_off = 0;
    w.inv_off = align256((size_t)(na * in) * sizeof(float));
    w.unit_off = w.inv_off + align256((size_t)(na * in) * sizeof(float));
    w.part_off = w.unit_off + align256((size_t)na * sizeof(int32_t));
    // X of a 16-bit layer rearranged into matrix-operand fragment order (see
    // k_search16.hip), zero-padded to whole 256-token blocks.
    w.xf_off = w.part_off + align256((size_t)(na * w.nblk) * sizeof(double));
    const int64_t tpad = ((tokens + kTokPerBlock - 1) / kTokPerBlock) * kTokPerBlock;
    w.total = w.xf_off + align256((size_t)(tpad * in) * 2);
    return w;
}

// ---------------------------------------------------------------------------
// Device bodies shared by separate kernels and the fused ones, so both give
// bitwise the same results.

// Step 2 for columns 256 cb .. 256 cb + 255 of candidate k (alpha = k / grid),
// one thread per column, 256 threads: s = fp32(xmag^alpha / sqrt(pmax *
// pmin)) with pmax, pmin the powers of max and min xmag. For alpha >= 0,
// x -> x^alpha is non-decreasing, and the fp32 inputs are at least one fp32
// ulp (2^-23 relative) apart, far more than any error of an fp64 pow, so
//   max_j pow(x_j, alpha) == pow(max_j x_j, alpha)   (and likewise for min)
// holds for the computed values too: every block finds max and min of xmag
// itself (exact, any order) and powers only those two and its own columns.
// unit[k] is set when the two powers are equal (k = 0, or flat activations):
// then every s is exactly 1 (sqrt(p * p) == p in binary floating point) and
// the search treats the candidate's scaled weights as the raw stored values.
__device__ __forceinline__ void s_table_block(const float *__restrict__ xmag, int64_t in, int grid, int k,
                                              int64_t cb, float *__restrict__ s_tab,
                                              float *__restrict__ inv_tab, int32_t *__restrict__ unit)
{
    __shared__ float smax[4], smin[4];
    __shared__ double ext[2];
    const double alpha = (double)k / (double)grid;
    const int64_t j = cb * 256 + threadIdx.x;
    const bool col_ok = j < in;
    const double p = pow((double)xmag[col_ok ? j : 0], alpha);

    // Max and min of xmag (> 0): 16 independent loads in flight per thread
    // per round (one round for in <= 4096).
    float lmax = 0.f, lmin = 3.402823466e38f;
    for (int64_t i0 = threadIdx.x; i0 < in; i0 += 256 * 16) {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t i = i0 + 256 * u;
            x[u] = xmag[i < in ? i : i0];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            lmax = fmaxf(lmax, x[u]);
            lmin = fminf(lmin, x[u]);
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        lmax = fmaxf(lmax, __shfl_xor(lmax, off));
        lmin = fminf(lmin, __shfl_xor(lmin, off));
    }
    if ((threadIdx.x & 63) == 0) {
        smax[threadIdx.x >> 6] = lmax;
        smin[threadIdx.x >> 6] = lmin;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const float xm = threadIdx.x == 0 ? fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]))
                                          : fminf(fminf(smin[0], smin[1]), fminf(smin[2], smin[3]));
        ext[threadIdx.x] = pow((double)xm, alpha);
    }
    __syncthreads();
    const double pmax = ext[0], pmin = ext[1];
    if (unit && cb == 0 && threadIdx.x == 0)
        unit[k] = pmax == pmin ? 1 : 0;
    if (!col_ok)
        return;
    const float s = (float)(p / sqrt(pmax * pmin));
    s_tab[(int64_t)k * in + j] = s;
    if (inv_tab)
        inv_tab[(int64_t)k * in + j] = 1.0f / s;
}

// The finish: fixed-order reduction of the block partials of every candidate
// (wave w takes candidates w, w + nwaves, ...; lane l sums partials l, l + 64,
// ... in order, then a fixed xor butterfly -- the same arithmetic for any
// number of waves), then the first strict minimum over the candidates (a NaN
// never compares below) and s_best = that row of the s-table, or all ones
// when nothing is finite. err: LDS of n_alpha doubles; sbest: one LDS int.
__device__ __forceinline__ void finish_block(const double *__restrict__ partial, int64_t nblk, int n_alpha,
                                             double denom, const float *__restrict__ s_tab, int64_t in,
                                             double *__restrict__ mse, int32_t *__restrict__ best,
                                             float *__restrict__ s_best, double *err, int *sbest)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    for (int a = wave; a < n_alpha; a += nwaves) {
        const double *p = partial + (int64_t)a * nblk;
        // lane l adds partials l, l + 64, l + 128, ... in that order; the
        // loads of 16 (then 4) of them go out before their adds, so a long
        // list costs one memory round trip per 16 partials of a lane
        double acc = 0.0;
        int64_t b = lane;
        for (; b + 15 * 64 < nblk; b += 16 * 64) {
            double x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                x[u] = p[b + 64 * u];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                acc += x[u];
        }
        for (; b + 192 < nblk; b += 256) {
            const double x0 = p[b], x1 = p[b + 64], x2 = p[b + 128], x3 = p[b + 192];
            acc += x0;
            acc += x1;
            acc += x2;
            acc += x3;
        }
        for (; b < nblk; b += 64)
            acc += p[b];
        for (int off = 32; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off);
        if (lane == 0) {
            const double m = acc / denom;
            err[a] = m;
            mse[a] = m;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int bi = -1;
        double be = __builtin_inf();
        for (int k = 0; k < n_alpha; ++k) {
            if (err[k] < be) {
                be = err[k];
                bi = k;
            }
        }
        *sbest = bi;
        *best = bi;
    }
    __syncthreads();
    const int bi = *sbest;
    const float *src = s_tab + (int64_t)(bi >= 0 ? bi : 0) * in;
    // sixteen independent loads in flight per thread per round
    for (int64_t j0 = threadIdx.x; j0 < in; j0 += 16 * (int64_t)blockDim.x) {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t j = j0 + u * (int64_t)blockDim.x;
            x[u] = bi >= 0 && j < in ? src[j] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t j = j0 + u * (int64_t)blockDim.x;
            if (j < in)
                s_best[j] = x[u];
        }
    }
}

// Launchers (each returns the first HIP error, hipSuccess otherwise).
hipError_t launch_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag,
                            hipStream_t st);
hipError_t launch_s_table(const float *xmag, int64_t in, int grid, float *s_tab, float *inv_tab,
                          int32_t *unit, hipStream_t st);
// The outputs of the finish, for the single-call search.
struct FinishOut {
    double *mse;
    int32_t *best;
    float *s_best;
};
hipError_t launch_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                         int64_t tokens, const float *s_tab, const float *inv_tab,
                         const int32_t *unit, int n_alpha, int bits, int group, int mode,
                         double *partial, const void *xfrag, const FinishOut *fin, hipStream_t st);
bool search_uses_fp32_operands(int dtype, int64_t out, int64_t tokens);
// Whether a layer takes the 32x32-tile search for 16-bit operands
// (k_search16.hip), which reads X from the fragment-ordered copy that the
// preparation kernel writes.
bool search16_applies(int dtype, int64_t out, int64_t in, int64_t tokens, int n_alpha);
// Preparation: the s-table, its reciprocals and the unit flags (step 2);
// for the 16-bit search also the fragment-ordered copy of X, in the same
// launch.
hipError_t launch_prepare(const void *X, int dtype, const float *xmag, int64_t out, int64_t in,
                          int64_t tokens, int grid, float *s_tab, float *inv_tab, int32_t *unit,
                          void *xfrag, hipStream_t st);
#define AWQ_S16_DECL(name)                                                                          \
    hipError_t name(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,          \
                    const float *s_tab, const float *inv_tab, const int32_t *unit, int n_alpha,     \
                    int bits, int mode, double *partial, hipStream_t st);
AWQ_S16_DECL(launch_search16_f16_g32)
AWQ_S16_DECL(launch_search16_f16_g64)
AWQ_S16_DECL(launch_search16_f16_g128)
AWQ_S16_DECL(launch_search16_bf16_g32)
AWQ_S16_DECL(launch_search16_bf16_g64)
AWQ_S16_DECL(launch_search16_bf16_g128)
#undef AWQ_S16_DECL
hipError_t launch_prepare16_f16(const void *X, const float *xmag, int64_t in, int64_t tokens, int grid,
                                float *s_tab, float *inv_tab, int32_t *unit, void *xfrag, hipStream_t st);
hipError_t launch_prepare16_bf16(const void *X, const float *xmag, int64_t in, int64_t tokens, int grid,
                                 float *s_tab, float *inv_tab, int32_t *unit, void *xfrag, hipStream_t st);
hipError_t launch_reduce_argmin(const double *partial, int64_t nblk, int n_alpha, int64_t out,
                                int64_t tokens, int64_t in, const float *s_tab, double *mse,
                                int32_t *best, float *s_best, hipStream_t st);
hipError_t launch_pack(const void *W, int dtype, int64_t out, int64_t in, const float *s,
                       const float *clip, int bits, int group, int mode, uint32_t *qweight,
                       float *scales, uint8_t *zeros, hipStream_t st);
hipError_t launch_gptq_hessian(const void *X, int dtype, int64_t tokens, int64_t in, double damp, double *H,
                               hipStream_t st);
hipError_t launch_gptq_factor(const double *H, int64_t n, double *U, double *ws, hipStream_t st);
hipError_t launch_gptq_quantize(const void *W, int dtype, int64_t out, int64_t in, const double *U, int bits,
                                int group, int mode, uint32_t *qweight, float *scales, uint8_t *zeros,
                                double *ws, hipStream_t st);
hipError_t launch_qgemm(const void *X, int dtype, int64_t M, int64_t in, const uint32_t *qweight,
                        const float *scales, const uint8_t *zeros, int64_t out, int bits, int group,
                        void *Y, bool yf32, hipStream_t st);
hipError_t launch_fold(const void *A, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                       bool scale_cols, hipStream_t st);
hipError_t launch_clip_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                              int64_t tokens, const float *s, int bits, int group, int mode,
                              int n_clip, float max_shrink, float *clip, double *sse, hipStream_t st);

}  // namespace awq
