// k_stats.hip -- per-channel activation magnitude and the candidate-scale table.
//
// Step 1 ("AWQ (activation-aware weight quantization)", "How it works" step 1;
// the 1e-8 guard from "The code, line by line"):
//   xmag[j] = fp32(mean_t |X[t, j]| + 1e-8), fp64 sums in a fixed order.
// Step 2 (same page, "The code, line by line"): alpha_k = k / grid,
//   s[k][j] = fp32(xmag[j]^alpha_k / sqrt(max_j xmag^alpha_k * min_j xmag^alpha_k)).
//
// Both are HBM/latency bound and tiny next to the search; the design goal is
// a bitwise-reproducible result, not speed: the sum order is fixed (sequential
// inside 64-token chunks, then the chunk sums in ascending order) and every
// fp64 operation is a single IEEE operation (the library is built with
// -ffp-contract=off).
#include "awq_internal.h"

#include <math.h>

namespace awq {

constexpr int kChunk = 64;   // tokens per fixed-order partial sum

// One thread owns V adjacent columns of one 64-token chunk and sums them in
// token order. Consecutive threads own consecutive columns, so every token row
// is read with contiguous, coalesced loads.
template <typename T, int V>
__global__ __launch_bounds__(256) void k_act_partial(const T *__restrict__ X, int64_t tokens,
                                                      int64_t in, double *__restrict__ partial)
{
    const int64_t j0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    const int64_t c = blockIdx.y;
    if (j0 >= in)
        return;
    const int64_t t0 = c * kChunk;
    const int64_t t1 = t0 + kChunk < tokens ? t0 + kChunk : tokens;
    double acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
        acc[v] = 0.0;
    if (j0 + V <= in) {
        struct alignas(sizeof(T) * V) Pack { T e[V]; };
        for (int64_t t = t0; t < t1; ++t) {
            const Pack p = *reinterpret_cast<const Pack *>(X + t * in + j0);
#pragma unroll
            for (int v = 0; v < V; ++v)
                acc[v] += fabs((double)static_cast<float>(p.e[v]));
        }
    } else {
        for (int64_t t = t0; t < t1; ++t)
            for (int v = 0; v < V && j0 + v < in; ++v)
                acc[v] += fabs((double)static_cast<float>(X[t * in + j0 + v]));
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
        if (j0 + v < in)
            partial[c * in + j0 + v] = acc[v];
}

__global__ __launch_bounds__(256) void k_act_finalize(const double *__restrict__ partial,
                                                       int64_t nchunk, int64_t tokens, int64_t in,
                                                       float *__restrict__ xmag)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= in)
        return;
    double total = 0.0;
    for (int64_t c = 0; c < nchunk; ++c)
        total += partial[c * in + j];
    const double mean = total / (double)tokens;
    xmag[j] = (float)(mean + 1e-8);
}

template <typename T, int V>
static hipError_t stats_typed(const T *X, int64_t tokens, int64_t in, float *xmag, double *partial,
                              hipStream_t st)
{
    const int64_t nchunk = (tokens + kChunk - 1) / kChunk;
    const int64_t threads = (in + V - 1) / V;
    dim3 grid((unsigned)((threads + 255) / 256), (unsigned)nchunk);
    hipLaunchKernelGGL((k_act_partial<T, V>), grid, dim3(256), 0, st, X, tokens, in, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_act_finalize, dim3((unsigned)((in + 255) / 256)), dim3(256), 0, st,
                       (const double *)partial, nchunk, tokens, in, xmag);
    return hipGetLastError();
}

hipError_t launch_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag,
                            double *partial, hipStream_t st)
{
    // Vector width: whole 8-byte loads when the row length keeps them aligned.
    switch (dtype) {
    case AWQ_F32:
        return in % 2 == 0 ? stats_typed<float, 2>((const float *)X, tokens, in, xmag, partial, st)
                           : stats_typed<float, 1>((const float *)X, tokens, in, xmag, partial, st);
    case AWQ_F16:
        return in % 4 == 0 ? stats_typed<f16, 4>((const f16 *)X, tokens, in, xmag, partial, st)
                           : stats_typed<f16, 1>((const f16 *)X, tokens, in, xmag, partial, st);
    default:
        return in % 4 == 0 ? stats_typed<bf16, 4>((const bf16 *)X, tokens, in, xmag, partial, st)
                           : stats_typed<bf16, 1>((const bf16 *)X, tokens, in, xmag, partial, st);
    }
}

// One block per candidate k: fp64 powers, block-wide max and min (exact, so
// the reduction order does not matter), centring, one rounding to fp32. The
// powers are recomputed in the second pass rather than stored. unit[k] is set
// when all powers are equal (k = 0, or flat activations): then every s is
// exactly 1 (sqrt(p*p) == p in binary floating point) and the search treats
// the candidate's scaled weights as the raw stored values.
__global__ __launch_bounds__(1024) void k_s_table(const float *__restrict__ xmag, int64_t in,
                                                   int grid, float *__restrict__ s_tab,
                                                   float *__restrict__ inv_tab,
                                                   int32_t *__restrict__ unit)
{
    __shared__ double smax[1024 / 64], smin[1024 / 64];
    const int k = blockIdx.x;
    const double alpha = (double)k / (double)grid;
    double lmax = -INFINITY, lmin = INFINITY;
    for (int64_t j = threadIdx.x; j < in; j += blockDim.x) {
        const double p = pow((double)xmag[j], alpha);
        lmax = p > lmax ? p : lmax;
        lmin = p < lmin ? p : lmin;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const double a = __shfl_xor(lmax, off);
        const double b = __shfl_xor(lmin, off);
        lmax = a > lmax ? a : lmax;
        lmin = b < lmin ? b : lmin;
    }
    const int wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) {
        smax[wave] = lmax;
        smin[wave] = lmin;
    }
    __syncthreads();
    double pmax = smax[0], pmin = smin[0];
    for (int w = 1; w < nw; ++w) {
        pmax = smax[w] > pmax ? smax[w] : pmax;
        pmin = smin[w] < pmin ? smin[w] : pmin;
    }
    const double centre = sqrt(pmax * pmin);
    if (unit && threadIdx.x == 0)
        unit[k] = pmax == pmin ? 1 : 0;
    for (int64_t j = threadIdx.x; j < in; j += blockDim.x) {
        const double p = pow((double)xmag[j], alpha);
        const float s = (float)(p / centre);
        s_tab[(int64_t)k * in + j] = s;
        if (inv_tab)
            inv_tab[(int64_t)k * in + j] = 1.0f / s;
    }
}

hipError_t launch_s_table(const float *xmag, int64_t in, int grid, float *s_tab, float *inv_tab,
                          int32_t *unit, hipStream_t st)
{
    hipLaunchKernelGGL(k_s_table, dim3((unsigned)(grid + 1)), dim3(1024), 0, st, xmag, in, grid,
                       s_tab, inv_tab, unit);
    return hipGetLastError();
}

}  // namespace awq
