// k_fold.hip -- folding the searched scales into the model.
//
// The identity W x = (W diag(s)) (diag(s)^-1 x) ("AWQ vs GPTQ Quantization
// Architectures Compared", "AWQ: move the error away from what matters") is
// applied to the stored tensors ("AWQ (activation-aware weight quantization)",
// "How it works" step 5 and the transformer paragraph after it):
//   rows mode: out[r][c] = store(A[r][c] / s[r]) -- the producer of the layer's
//              input absorbs 1/s: a norm weight or bias (cols = 1), or the
//              output rows of the previous linear layer (and its bias);
//   cols mode: out[o][j] = store(W[o][j] * s[j]) -- the searched layer's weight.
// One fp32 operation per element (IEEE division or multiplication), then one
// round-half-to-even conversion to the storage type.
//
// Streaming and HBM bound: each lane moves 8 consecutive elements with one
// vector load and one vector store (16 B for fp16/bf16, 32 B for fp32);
// grid-stride over the chunks. Rows of a multiple of 8 columns keep a chunk in
// one row; a vector (cols = 1) takes 8 divisors per chunk. Other shapes, a
// ragged tail or misaligned pointers take the one-element-per-lane kernel.
// out may be A itself (in place).
#include "awq_internal.h"

namespace awq {

template <typename T> struct StoreVec8;
template <> struct StoreVec8<float> {
    static __device__ __forceinline__ void put(float *p, const float (&v)[8])
    {
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = v[e];
        *reinterpret_cast<f32x8 *>(p) = o;
    }
};
template <> struct StoreVec8<f16> {
    static __device__ __forceinline__ void put(f16 *p, const float (&v)[8])
    {
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = static_cast<f16>(v[e]);
        *reinterpret_cast<f16x8 *>(p) = o;
    }
};
template <> struct StoreVec8<bf16> {
    static __device__ __forceinline__ void put(bf16 *p, const float (&v)[8])
    {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = static_cast<bf16>(v[e]);
        *reinterpret_cast<bf16x8 *>(p) = o;
    }
};

template <typename T, bool COLS>
__global__ __launch_bounds__(256) void k_fold_vec(const T *A, T *out, int64_t cols, const float *s,
                                                  int64_t nchunk)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < nchunk; ch += stride) {
        const int64_t i0 = ch * 8;
        float a[8], f[8];
        widen8<T>(load8(A + i0), a);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[e] = opaque(a[e]);
        if (COLS) {
            const int64_t j0 = i0 % cols;          // cols % 8 == 0: one row, columns j0..j0+7
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = a[e] * s[j0 + e];
        } else if (cols == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = a[e] / s[i0 + e];
        } else {
            const float d = s[i0 / cols];           // cols % 8 == 0: one row
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = a[e] / d;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = opaque(f[e]);
        StoreVec8<T>::put(out + i0, f);
    }
}

template <typename T, bool COLS>
__global__ __launch_bounds__(256) void k_fold_any(const T *A, T *out, int64_t cols, const float *s,
                                                  int64_t first, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float a = opaque(static_cast<float>(A[i]));
        const float f = opaque(COLS ? a * s[i % cols] : a / s[i / cols]);
        out[i] = static_cast<T>(f);
    }
}

static unsigned fold_blocks(int64_t items)
{
    const int64_t b = (items + 255) / 256;
    return (unsigned)(b < 16384 ? (b > 0 ? b : 1) : 16384);
}

template <typename T, bool COLS>
static hipError_t fold_typed(const void *A, void *out, int64_t rows, int64_t cols, const float *s,
                             hipStream_t st)
{
    const int64_t n = rows * cols;
    const bool aligned = ((uintptr_t)A % (8 * sizeof(T)) == 0) && ((uintptr_t)out % (8 * sizeof(T)) == 0);
    const bool shape_ok = COLS ? cols % 8 == 0 : (cols % 8 == 0 || cols == 1);
    int64_t done = 0;
    if (aligned && shape_ok) {
        const int64_t nchunk = n / 8;
        if (nchunk > 0)
            hipLaunchKernelGGL((k_fold_vec<T, COLS>), dim3(fold_blocks(nchunk)), dim3(256), 0, st,
                               (const T *)A, (T *)out, cols, s, nchunk);
        done = nchunk * 8;
    }
    if (done < n)
        hipLaunchKernelGGL((k_fold_any<T, COLS>), dim3(fold_blocks(n - done)), dim3(256), 0, st,
                           (const T *)A, (T *)out, cols, s, done, n);
    return hipGetLastError();
}

hipError_t launch_fold(const void *A, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                       bool scale_cols, hipStream_t st)
{
    switch (dtype) {
    case AWQ_F32:
        return scale_cols ? fold_typed<float, true>(A, out, rows, cols, s, st)
                          : fold_typed<float, false>(A, out, rows, cols, s, st);
    case AWQ_F16:
        return scale_cols ? fold_typed<f16, true>(A, out, rows, cols, s, st)
                          : fold_typed<f16, false>(A, out, rows, cols, s, st);
    default:
        return scale_cols ? fold_typed<bf16, true>(A, out, rows, cols, s, st)
                          : fold_typed<bf16, false>(A, out, rows, cols, s, st);
    }
}

}  // namespace awq
