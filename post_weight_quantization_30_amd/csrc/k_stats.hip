// k_stats.hip -- per-channel activation magnitude and the candidate-scale table.
//
// Step 1 ("AWQ (activation-aware weight quantization)", "How it works" step 1;
// the 1e-8 guard from "The code, line by line"):
//   xmag[j] = fp32(mean_t |X[t, j]| + 1e-8), fp64 sums in a fixed order.
// Step 2 (same page, "The code, line by line"): alpha_k = k / grid,
//   s[k][j] = fp32(xmag[j]^alpha_k / sqrt(max_j xmag^alpha_k * min_j xmag^alpha_k)).
//
// Both are tiny next to the search; besides speed the goal is a bitwise
// reproducible result: the sum order is fixed (sequential inside 64-token
// chunks, then the chunk sums in ascending order, starting from 0) and every
// fp64 operation is a single IEEE operation (the library is built with
// -ffp-contract=off).
#include "awq_internal.h"

#include <float.h>
#include <math.h>

namespace awq {

constexpr int kChunk = 64;        // tokens per fixed-order partial sum
constexpr int kStatWaves = 16;    // chunks summed at once by one block

// One block owns 64 adjacent columns (one per lane) and up to 16 waves; in
// round r wave w sums chunk r*waves + w of its lane's column, with all 64
// loads of a full chunk issued before the sequential adds (one memory round
// trip per chunk). Wave 0 then adds the round's chunk sums, in chunk order, to
// the running total. Rows of X are read 64 columns at a time, coalesced.
template <typename T>
__global__ __launch_bounds__(kStatWaves * 64) void k_act_stats(const T *__restrict__ X,
                                                                int64_t tokens, int64_t in,
                                                                float *__restrict__ xmag)
{
    __shared__ double csum[kStatWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + lane;
    const bool col_ok = j < in;
    const int64_t jc = col_ok ? j : in - 1;   // in-bounds column for idle lanes
    const int64_t nchunk = (tokens + kChunk - 1) / kChunk;
    double total = 0.0;
    for (int64_t c0 = 0; c0 < nchunk; c0 += waves) {
        const int64_t c = c0 + wave;
        double acc = 0.0;
        if (c < nchunk) {
            const int64_t t0 = c * kChunk;
            const T *p = X + t0 * in + jc;
            if (t0 + kChunk <= tokens) {
                float v[kChunk];
#pragma unroll
                for (int t = 0; t < kChunk; ++t)
                    v[t] = static_cast<float>(p[(int64_t)t * in]);
#pragma unroll
                for (int t = 0; t < kChunk; ++t)
                    acc += fabs((double)v[t]);
            } else {
                for (int64_t t = t0; t < tokens; ++t, p += in)
                    acc += fabs((double)static_cast<float>(*p));
            }
        }
        csum[wave][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            const int64_t nr = nchunk - c0 < waves ? nchunk - c0 : waves;
            for (int w = 0; w < nr; ++w)
                total += csum[w][lane];
        }
        __syncthreads();
    }
    if (wave == 0 && col_ok)
        xmag[j] = (float)(total / (double)tokens + 1e-8);
}

template <typename T>
static hipError_t stats_typed(const T *X, int64_t tokens, int64_t in, float *xmag, hipStream_t st)
{
    const int64_t nchunk = (tokens + kChunk - 1) / kChunk;
    const int waves = nchunk < kStatWaves ? (int)nchunk : kStatWaves;
    hipLaunchKernelGGL(k_act_stats<T>, dim3((unsigned)((in + 63) / 64)), dim3(waves * 64), 0, st, X,
                       tokens, in, xmag);
    return hipGetLastError();
}

hipError_t launch_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag,
                            hipStream_t st)
{
    switch (dtype) {
    case AWQ_F32: return stats_typed<float>((const float *)X, tokens, in, xmag, st);
    case AWQ_F16: return stats_typed<f16>((const f16 *)X, tokens, in, xmag, st);
    default: return stats_typed<bf16>((const bf16 *)X, tokens, in, xmag, st);
    }
}

// One block per (256 columns, candidate k); the body (s_table_block) is
// shared with the preparation kernel of the 16-bit search.
__global__ __launch_bounds__(256) void k_s_table(const float *__restrict__ xmag, int64_t in, int grid,
                                                  float *__restrict__ s_tab,
                                                  float *__restrict__ inv_tab,
                                                  int32_t *__restrict__ unit)
{
    s_table_block(xmag, in, grid, (int)blockIdx.y, (int64_t)blockIdx.x, s_tab, inv_tab, unit);
}

hipError_t launch_s_table(const float *xmag, int64_t in, int grid, float *s_tab, float *inv_tab,
                          int32_t *unit, hipStream_t st)
{
    hipLaunchKernelGGL(k_s_table, dim3((unsigned)((in + 255) / 256), (unsigned)(grid + 1)), dim3(256),
                       0, st, xmag, in, grid, s_tab, inv_tab, unit);
    return hipGetLastError();
}

}  // namespace awq
