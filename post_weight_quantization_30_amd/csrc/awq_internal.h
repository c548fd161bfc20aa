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

// Launchers (each returns the first HIP error, hipSuccess otherwise).
hipError_t launch_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag,
                            hipStream_t st);
hipError_t launch_s_table(const float *xmag, int64_t in, int grid, float *s_tab, float *inv_tab,
                          int32_t *unit, hipStream_t st);
hipError_t launch_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                         int64_t tokens, const float *s_tab, const float *inv_tab,
                         const int32_t *unit, int n_alpha, int bits, int group, int mode,
                         double *partial, void *xfrag, hipStream_t st);
bool search_uses_fp32_operands(int dtype, int64_t out, int64_t tokens);
// The 32x32-tile search for 16-bit operands (k_search16.hip): whether it
// takes this shape, and its launcher (same contract as launch_search),
// which dispatches to one launcher per operand type and group size.
bool search16_applies(int64_t in, int n_alpha, int64_t nblocks);
hipError_t launch_search16(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                           int64_t tokens, const float *s_tab, const float *inv_tab,
                           const int32_t *unit, int n_alpha, int bits, int group, int mode,
                           double *partial, void *xfrag, hipStream_t st);
#define AWQ_S16_DECL(name)                                                                          \
    hipError_t name(const void *W, const void *X, int64_t out, int64_t in, int64_t tokens,          \
                    const float *s_tab, const float *inv_tab, const int32_t *unit, int n_alpha,     \
                    int bits, int mode, double *partial, void *xfrag, hipStream_t st);
AWQ_S16_DECL(launch_search16_f16_g32)
AWQ_S16_DECL(launch_search16_f16_g64)
AWQ_S16_DECL(launch_search16_f16_g128)
AWQ_S16_DECL(launch_search16_bf16_g32)
AWQ_S16_DECL(launch_search16_bf16_g64)
AWQ_S16_DECL(launch_search16_bf16_g128)
#undef AWQ_S16_DECL
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
