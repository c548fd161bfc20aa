// k_gptq.hip -- GPTQ on the same layer inputs, in fp64 on the matrix cores.
//
// What is computed ("AWQ vs GPTQ Quantization Architectures Compared", "GPTQ:
// compensate the error you just made"; "Advanced Quantization Algorithms: AWQ
// and GPTQ Explained", section 3): H = 2 X^T X plus damp * mean(diag H) on the
// diagonal; U = the upper Cholesky factor of H^-1 (H^-1 = U^T U); then, column
// by column for all rows at once, group parameters fitted on the already
// corrected weights at each group start, the column rounded, and its error
// divided by U[i][i] and pushed into the later columns along row i of U.
// Everything is fp64, the precision of the pages' listing, so that the integer
// codes follow the same decisions.
//
// How:
//  - one fp64 MFMA GEMM kernel (v_mfma_f64_16x16x4f64, 64 x 64 tiles staged
//    through LDS) serves the Hessian, the Cholesky trailing updates, the
//    triangular-inverse products and GPTQ's lazy block updates;
//  - U without forming H^-1: with J the index reversal, the lower Cholesky
//    factor L of J H J gives H = (J L J)(J L J)^T with J L J upper, hence
//    H^-1 = (J L^-1 J)^T (J L^-1 J) and, by uniqueness, U = J L^-1 J: one
//    blocked Cholesky and one blocked triangular inverse (panels of 64);
//  - the blocked Cholesky factors each 64 x 64 diagonal block inside the
//    trailing-update GEMM that produces it (its tile-(0, 0) workgroup);
//  - the column loop in blocks of 128 columns: four rows per wave, 16 lanes
//    per row, each lane owning 8 of the block's columns; a column is
//    quantised in every row at once by its owner lanes and the scaled error
//    is shuffled to the row's other lanes, which update their later columns;
//    then one GEMM applies the block's 128 errors to all later columns (the
//    pages defer the updates of later columns and apply them 128 columns at
//    a time).
//  The serial parts (the diagonal blocks, the panel solves, the column loop)
//  are bound by the latency of their chains of dependent fp64 operations,
//  about 15 ns each on one wave.
#include "awq_internal.h"

#include <math.h>

#include <algorithm>

namespace awq {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kNb = 64;          // Cholesky / inverse panel
constexpr int kCol = 128;        // GPTQ column block

// ---------------------------------------------------------------------------
// Cholesky of the 64 x 64 diagonal block at (k0, k0), in place (lower): the
// trailing updates of earlier panels are already applied. Four waves, one per
// SIMD: lane i holds row i, wave w its columns l = 4t + w (t < 16). Step j:
// the wave owning column j forms L[i][j] (the pivot's square root broadcast
// from lane j) and publishes the column through LDS (double-buffered, so one
// barrier per step suffices); every wave then removes L[i][j] L[l][j] from
// its later columns. Entries above the diagonal are carried as scratch and
// never written back.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double bcast(double v, int src)
{
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffffLL), src);
    const int hi = __builtin_amdgcn_readlane((int)(u >> 32), src);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Needs a 256-thread workgroup.
__device__ __forceinline__ void potrf64(double *A, int64_t n, int64_t k0)
{
    __shared__ double colb[2][kNb];
    const int i = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    double a[kNb / 4];
    double *row = A + (k0 + i) * n + k0;
#pragma unroll
    for (int t = 0; t < kNb / 4; ++t)
        a[t] = 4 * t + w <= i ? row[4 * t + w] : 0.0;
#pragma unroll
    for (int j = 0; j < kNb; ++j) {
        double *cb = colb[j & 1];
        if (w == (j & 3)) {
            // 1/sqrt of the pivot once, then products (no fp64 divide on the
            // step's serial path)
            const double p = bcast(a[j >> 2], j);
            // 1/sqrt(p): the hardware estimate and two Newton steps. Each
            // step about doubles the correct bits (the estimate carries
            // about 23, one step leaves an error near 1e-14 relative); after
            // the second the result is within about an ulp of 1/sqrt(p).
            const double y0 = __builtin_amdgcn_rsq(p);
            const double e0 = fma(-(p * y0), y0, 1.0);
            const double y1 = fma(0.5 * y0, e0, y0);
            const double e1 = fma(-(p * y1), y1, 1.0);
            const double rs = fma(0.5 * y1, e1, y1);
            double v = a[j >> 2];
            v = i == j ? p * rs : (i > j ? v * rs : v);
            a[j >> 2] = v;
            cb[i] = v;                             // L[i][j] for i >= j
        }
        __syncthreads();
        const double lij = cb[i];
#pragma unroll
        for (int t = 0; t < kNb / 4; ++t)
            if (4 * t + w > j)                     // uniform per wave; one rounding
                a[t] = fma(-lij, cb[4 * t + w], a[t]);
    }
#pragma unroll
    for (int t = 0; t < kNb / 4; ++t)
        if (4 * t + w <= i)
            row[4 * t + w] = a[t];
}

__global__ __launch_bounds__(256) void k_potrf_diag(double *A, int64_t n, int64_t k0)
{
    potrf64(A, n, k0);
}

// ---------------------------------------------------------------------------
// C[m][n] = alpha * sum_k A(m, k) B(k, n) + beta * C[m][n], for each batch z
// (blockIdx.z) with A, B, C advanced by z * sA, z * sB, z * sC.
// A(m, k) = TA ? A[k lda + m] : A[m lda + k];  B(k, n) = TB ? B[n ldb + k] : B[k ldb + n].
// LOWER: tiles entirely above the diagonal are skipped (only the lower
// triangle of C is wanted). ACCC (alpha = -1, beta = 1 only): C -= A B with
// the matrix cores accumulating onto C's own values, read into the
// accumulators at the start (A's elements negated as they are staged, which
// is exact); the epilogue then only stores. Block: 32 MI x 64 of C, 4 waves
// of 16 MI x 32; k in steps of 16 through LDS (padded rows), the next step's
// elements loaded into registers while the current one is multiplied;
// out-of-range elements load as 0.
// ---------------------------------------------------------------------------
template <typename TAe, typename TBe, bool TA, bool TB, int MI>
__device__ __forceinline__ void dgemm_fetch(const TAe *A, int64_t lda, const TBe *B, int64_t ldb, int64_t M,
                                            int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t k0, int tid,
                                            double (&ra)[2 * MI], double (&rb)[4])
{
    constexpr int BM = 32 * MI;
#pragma unroll
    for (int q = 0; q < 2 * MI; ++q) {
        const int e = q * 256 + tid;
        int mm, kk;
        if (TA) { mm = e % BM; kk = e / BM; } else { kk = e & 15; mm = e >> 4; }
        const int64_t m = m0 + mm, k = k0 + kk;
        ra[q] = (m < M && k < K) ? static_cast<double>(TA ? A[k * lda + m] : A[m * lda + k]) : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = q * 256 + tid;
        int nn, kk;
        if (TB) { kk = e & 15; nn = e >> 4; } else { nn = e & 63; kk = e >> 6; }
        const int64_t n = n0 + nn, k2 = k0 + kk;
        rb[q] = (n < N && k2 < K) ? static_cast<double>(TB ? B[n * ldb + k2] : B[k2 * ldb + n]) : 0.0;
    }
}

template <typename TAe, typename TBe, bool TA, bool TB, bool LOWER, bool POTRF = false, int MI = 2,
          bool ACCC = false, int TRI = 0>
__global__ __launch_bounds__(256) void k_dgemm(int64_t M, int64_t N, int64_t K, double alpha,
                                               const TAe *__restrict__ A, int64_t lda, int64_t sA,
                                               const TBe *__restrict__ B, int64_t ldb, int64_t sB, double beta,
                                               double *__restrict__ C, int64_t ldc, int64_t sC)
{
    constexpr int BM = 32 * MI;
    __shared__ double As[16][BM + 1];
    __shared__ double Bs[16][65];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * 64;
    if (LOWER && n0 > m0 + BM - 1)
        return;                                    // uniform for the block, before any barrier
    A += (int64_t)blockIdx.z * sA;
    B += (int64_t)blockIdx.z * sB;
    C += (int64_t)blockIdx.z * sC;
    const int wm = (wave >> 1) * 16 * MI, wn = (wave & 1) * 32;
    f64x4 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm + i * 16 + (lane >> 4) + 4 * r;
                const int64_t n = n0 + wn + j * 16 + (lane & 15);
                acc[i][j][r] = (ACCC && m < M && n < N) ? C[m * ldc + n] : 0.0;
            }
    // TRI: a triangular operand's exact zeros are skipped (their products
    // add nothing): 1 = B lower (B(k, n) = 0 for k < n), 2 = A lower
    // (A(m, k) = 0 for k > m). The tile's k-range shrinks to where both can
    // be non-zero; the k-steps kept are the same, in the same order.
    const int64_t kbeg = TRI == 1 ? (n0 / 16) * 16 : 0;
    const int64_t kend = TRI == 2 ? (m0 + BM < K ? m0 + BM : K) : K;
    double ra[2 * MI], rb[4];
    dgemm_fetch<TAe, TBe, TA, TB, MI>(A, lda, B, ldb, M, N, K, m0, n0, kbeg, tid, ra, rb);
    for (int64_t k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
        for (int q = 0; q < 2 * MI; ++q) {
            const int e = q * 256 + tid;
            const double v = ACCC ? -ra[q] : ra[q];
            if (TA) As[e / BM][e % BM] = v; else As[e & 15][e >> 4] = v;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = q * 256 + tid;
            if (TB) Bs[e & 15][e >> 4] = rb[q]; else Bs[e >> 6][e & 63] = rb[q];
        }
        __syncthreads();
        if (k0 + 16 < kend)
            dgemm_fetch<TAe, TBe, TA, TB, MI>(A, lda, B, ldb, M, N, K, m0, n0, k0 + 16, tid, ra, rb);
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
            double bv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = Bs[kk + (lane >> 4)][wn + j * 16 + (lane & 15)];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const double a = As[kk + (lane >> 4)][wm + i * 16 + (lane & 15)];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv[j], acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // v_mfma_f64_16x16x4f64: element r of lane l is D[l / 16 + 4 r][l % 16]
                const int64_t m = m0 + wm + i * 16 + (lane >> 4) + 4 * r;
                const int64_t n = n0 + wn + j * 16 + (lane & 15);
                if (m < M && n < N) {
                    double *c = C + m * ldc + n;
                    if (ACCC) {
                        *c = acc[i][j][r];
                    } else {
                        const double prod = alpha * acc[i][j][r];
                        *c = beta == 0.0 ? prod : fma(beta, *c, prod);
                    }
                }
            }
    // POTRF: the workgroup of tile (0, 0) factors that tile once it is written
    // (the next diagonal block of a blocked Cholesky, whose trailing update
    // this is; the barrier makes the tile's stores visible to the workgroup).
    if (POTRF && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
        __syncthreads();
        potrf64(C, ldc, 0);
    }
}

template <typename TAe, typename TBe, bool TA, bool TB, bool LOWER, bool POTRF = false, int MI = 2,
          bool ACCC = false, int TRI = 0>
static void dgemm(int64_t M, int64_t N, int64_t K, double alpha, const TAe *A, int64_t lda, const TBe *B,
                  int64_t ldb, double beta, double *C, int64_t ldc, hipStream_t st, int64_t batch = 1,
                  int64_t sA = 0, int64_t sB = 0, int64_t sC = 0)
{
    if (M <= 0 || N <= 0 || batch <= 0)
        return;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 32 * MI - 1) / (32 * MI)), (unsigned)batch);
    hipLaunchKernelGGL((k_dgemm<TAe, TBe, TA, TB, LOWER, POTRF, MI, ACCC, TRI>), grid, dim3(256), 0, st, M, N, K, alpha, A,
                       lda, sA, B, ldb, sB, beta, C, ldc, sC);
}

// ---------------------------------------------------------------------------
// Upper triangle of a symmetric matrix from its lower one, a 64 x 64 tile per
// block through LDS (coalesced reads of tile (J, I), coalesced writes of
// tile (I, J)); tiles on and below the diagonal are left as they are.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mirror_upper(double *H, int64_t n)
{
    const int64_t ti = blockIdx.y, tj = blockIdx.x;
    if (tj <= ti)
        return;                                    // whole block
    __shared__ double t[64][65];
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;          // element (tj*64 + r, ti*64 + c)
        const int64_t gr = tj * 64 + r, gc = ti * 64 + c;
        if (gr < n && gc < n)
            t[r][c] = H[gr * n + gc];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int c = e >> 6, r = e & 63;          // element (ti*64 + c, tj*64 + r)
        const int64_t gr = ti * 64 + c, gc = tj * 64 + r;
        if (gr < n && gc < n)
            H[gr * n + gc] = t[r][c];
    }
}

// ---------------------------------------------------------------------------
// Dampening: H[i][i] += damp * mean(diag H). One block; fixed summation order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_damp(double *H, int64_t n, double damp)
{
    __shared__ double part[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256)
        s += H[i * n + i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    const double add = damp * (part[0] / (double)n);
    for (int64_t i = threadIdx.x; i < n; i += 256)
        H[i * n + i] += add;
}

// Reversing both indices of an n x n matrix, (i, j) -> (n-1-i, n-1-j), is
// reversing its flattened array: e -> n*n - 1 - e.
__global__ __launch_bounds__(256) void k_reverse_copy(const double *__restrict__ src, double *__restrict__ dst,
                                                      int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
        dst[e] = src[total - 1 - e];
}

__global__ __launch_bounds__(256) void k_reverse_inplace(double *a, int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total / 2; e += (int64_t)gridDim.x * 256) {
        const double x = a[e];
        a[e] = a[total - 1 - e];
        a[total - 1 - e] = x;
    }
}

__global__ __launch_bounds__(256) void k_fill0(double *a, int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
        a[e] = 0.0;
}

// Rows below the diagonal block: A[r][k0..k0+63] <- A[r][k0..] L_kk^-T. One
// wave per row, lane q holding entry q; step j: x_j = x_j / L[j][j] is
// broadcast from lane j and removed from the later entries (x_q -= x_j L[q][j]),
// L_kk and 1/diag in LDS.
constexpr int kTrsmRows = 8;     // rows (waves) per workgroup

__global__ __launch_bounds__(kTrsmRows * 64) void k_trsm_panel(double *A, int64_t n, int64_t k0)
{
    __shared__ double l[kNb][kNb + 1];
    __shared__ double rd[kNb];
    for (int e = threadIdx.x; e < kNb * kNb; e += kTrsmRows * 64)
        l[e / kNb][e % kNb] = A[(k0 + e / kNb) * n + k0 + e % kNb];
    __syncthreads();
    if (threadIdx.x < kNb)
        rd[threadIdx.x] = 1.0 / l[threadIdx.x][threadIdx.x];
    __syncthreads();
    const int q = threadIdx.x & 63;
    const int64_t r = k0 + kNb + (int64_t)blockIdx.x * kTrsmRows + (threadIdx.x >> 6);
    if (r >= n)
        return;                                    // whole wave, after the barriers
    double *p = A + r * n + k0 + q;
    double x = *p;
#pragma unroll
    for (int j = 0; j < kNb; ++j) {
        const double xj = bcast(x, j) * rd[j];
        x = q == j ? xj : (q > j ? fma(-xj, l[q][j], x) : x);
    }
    *p = x;
}

// Inverse of every 64 x 64 diagonal block of the lower triangular L (one block
// each; column j of the inverse by forward substitution, one thread per column).
__global__ __launch_bounds__(64) void k_trtri_diag(const double *L, double *Li, int64_t n)
{
    __shared__ double l[kNb][kNb + 1];
    const int64_t k0 = (int64_t)blockIdx.x * kNb;
    for (int e = threadIdx.x; e < kNb * kNb; e += 64)
        l[e / kNb][e % kNb] = L[(k0 + e / kNb) * n + k0 + e % kNb];
    __syncthreads();
    const int j = threadIdx.x;
    double x[kNb];
#pragma unroll
    for (int i = 0; i < kNb; ++i) {
        double s = i == j ? 1.0 : 0.0;
#pragma unroll
        for (int q = 0; q < i; ++q)
            s -= l[i][q] * x[q];
        x[i] = i < j ? 0.0 : s / l[i][i];
    }
#pragma unroll
    for (int i = 0; i < kNb; ++i)
        Li[(k0 + i) * n + k0 + j] = x[i];
}

// ---------------------------------------------------------------------------
// One block of 128 columns [b, b + 128). A wave holds four rows, 16 lanes per
// row; lane c of a row owns the row's columns b + c + 16 k (k < 8) in
// registers. Column b + 16 k0 + c0 is quantised by lane c0 of each row (its
// element k0); one shuffle hands its scaled error to the row's other lanes,
// which subtract err * U[j][col] from their own columns. U's block sits in LDS
// with its lower triangle and diagonal zeroed, so every lane updates all of
// its columns not yet passed without a mask (err * 0 leaves a weight exact).
// ---------------------------------------------------------------------------
constexpr int kRowsPerGroup = 16;   // rows per workgroup of the column loop (4 waves)
constexpr int kColRowLanes = 16;    // lanes per row
constexpr int kColPerLane = kCol / kColRowLanes;   // 8

template <bool ASYM>
__global__ __launch_bounds__(kRowsPerGroup * 16) void k_gptq_block(double *__restrict__ Wc,
                                                                    const double *__restrict__ U, int64_t out,
                                                                    int64_t in, int64_t b, int bits, int group,
                                                                    double *__restrict__ E,
                                                                    uint32_t *__restrict__ qweight,
                                                                    float *__restrict__ scales,
                                                                    uint8_t *__restrict__ zeros)
{
    // Up[j][p][c] = {U[b + j][b + c + 32 p], U[b + j][b + c + 32 p + 16]} (strict upper part only):
    // a row's 16 lanes read 256 contiguous bytes per pair of their columns
    __shared__ double2 Up[kCol][kColPerLane / 2][kColRowLanes];
    __shared__ double rdiag[kCol];       // 1 / U[j][j]: the error's scaling without a division per column
    __shared__ uint8_t cbuf[kRowsPerGroup][kCol];
    for (int e = threadIdx.x; e < kCol * kCol / 2; e += kRowsPerGroup * 16) {
        const int j = e >> 6, p = (e >> 4) & 3, c = e & 15;
        const int c0 = c + 32 * p, c1 = c0 + 16;
        const double *ur = U + (b + j) * in + b;
        Up[j][p][c] = double2{c0 > j ? ur[c0] : 0.0, c1 > j ? ur[c1] : 0.0};
    }
    if (threadIdx.x < kCol)
        rdiag[threadIdx.x] = 1.0 / U[(b + threadIdx.x) * in + b + threadIdx.x];
    const int lane = threadIdx.x & 63, c = lane & 15;
    const int r16 = (threadIdx.x >> 4);            // row within the workgroup
    const int64_t o = (int64_t)blockIdx.x * kRowsPerGroup + r16;
    const bool live = o < out;
    double w[kColPerLane], e[kColPerLane];
    uint32_t code[kColPerLane];
    const double *row = Wc + (live ? o : 0) * in + b;
#pragma unroll
    for (int k = 0; k < kColPerLane; ++k) {
        w[k] = live ? row[c + 16 * k] : 0.0;
        e[k] = 0.0;
        code[k] = 0;
    }
    __syncthreads();
    const double maxq = (double)((1 << bits) - 1);
    const double L = (double)((1 << (bits - 1)) - 1);
    const int64_t ng = in / group;
    double scale = 1.0, zero = 0.0, rscale = 1.0;
#pragma unroll
    for (int k0 = 0; k0 < kColPerLane; ++k0) {
        if ((16 * k0) % group == 0) {
            // group parameters on the current (corrected) weights of the row's
            // columns [b + 16 k0, b + 16 k0 + group); groups are 32, 64 or 128
            // wide, so a group starts at a multiple of 16
            const int kend = k0 + group / 16;
            double s64;
            if (ASYM) {
                double lo = 0.0, hi = 0.0;     // the range always contains 0
#pragma unroll
                for (int k = k0; k < kColPerLane; ++k)
                    if (k < kend) { lo = fmin(lo, w[k]); hi = fmax(hi, w[k]); }
#pragma unroll
                for (int off = 8; off > 0; off >>= 1) {
                    lo = fmin(lo, __shfl_xor(lo, off));
                    hi = fmax(hi, __shfl_xor(hi, off));
                }
                s64 = fmax((hi - lo) / maxq, 1e-8);
                scale = (double)(float)s64;
                zero = rint(-lo / scale);
            } else {
                double a = 0.0;
#pragma unroll
                for (int k = k0; k < kColPerLane; ++k)
                    if (k < kend) a = fmax(a, fabs(w[k]));
#pragma unroll
                for (int off = 8; off > 0; off >>= 1)
                    a = fmax(a, __shfl_xor(a, off));
                s64 = fmax(a / L, 1e-8);
                scale = (double)(float)s64;
                zero = (double)(1 << (bits - 1));
            }
            rscale = 1.0 / scale;
            if (live && c == 0) {
                const int64_t gi = o * ng + (b + 16 * k0) / group;
                scales[gi] = (float)scale;
                zeros[gi] = (uint8_t)(int)zero;
            }
        }
#pragma unroll 1
        for (int c0 = 0; c0 < kColRowLanes; ++c0) {
            const int jj = 16 * k0 + c0;
            double2 u[kColPerLane / 2];
#pragma unroll
            for (int p = k0 / 2; p < kColPerLane / 2; ++p)
                u[p] = Up[jj][p][c];
            const double rd = rdiag[jj];
            // every lane runs the step on its element k0; lane c0's result is the row's
            const double wv = w[k0];
            // rint(w / scale) off the division's latency: t = w * (1/scale) is
            // within 3 ulp of the quotient, so the two round to the same integer
            // unless t lies within 1e-9 of a half-integer (true for |t| < 2^20;
            // larger quotients are clamped to the code range either way); there,
            // and at exact ties, the quotient itself decides
            const double t = wv * rscale;
            // the step from rint(t); the near-tie test runs beside it and
            // its rare redo comes last, off the step's dependent chain
            auto step = [&](double r, uint32_t &cd) {
                double q, wq;
                if (ASYM) {
                    q = fmin(fmax(r + zero, 0.0), maxq);
                    wq = scale * (q - zero);
                    cd = (uint32_t)(int)q;
                } else {
                    q = fmin(fmax(r, -L - 1.0), L);
                    wq = scale * q;
                    cd = (uint32_t)((int)q + (1 << (bits - 1)));
                }
                return (wv - wq) * rd;
            };
            const double r0 = rint(t);
            uint32_t cd;
            double mine = step(r0, cd);
            if (fabs(fabs(t - r0) - 0.5) < 1e-9)
                mine = step(rint(wv / scale), cd);
            const double err = __shfl(mine, (lane & 48) | c0);
            if (c == c0) {
                e[k0] = mine;
                code[k0] = cd;
            }
#pragma unroll
            for (int k = k0; k < kColPerLane; ++k)
                w[k] -= err * (k & 1 ? u[k / 2].y : u[k / 2].x);
        }
    }
    if (live) {
        double *er = E + o * kCol;
#pragma unroll
        for (int k = 0; k < kColPerLane; ++k)
            er[c + 16 * k] = e[k];
    }
#pragma unroll
    for (int k = 0; k < kColPerLane; ++k)
        cbuf[r16][c + 16 * k] = (uint8_t)code[k];
    __syncthreads();
    // the block's 128 codes fill exactly 4 * bits words of the row's stream
    if (live) {
        const int64_t wpr = in * bits / 32;
        for (int wd = c; wd < 4 * bits; wd += kColRowLanes) {
            uint32_t word = 0;
            const int first = (32 * wd) / bits, last = (32 * wd + 31) / bits;
            for (int i = first; i <= last; ++i) {
                const uint32_t cv = cbuf[r16][i];
                const int sh = i * bits - 32 * wd;
                word |= sh >= 0 ? cv << sh : cv >> -sh;
            }
            qweight[o * wpr + (b * bits) / 32 + wd] = word;
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
static void hessian_typed(const T *X, int64_t tokens, int64_t in, double *H, hipStream_t st)
{
    // H = 2 X^T X: A(m, k) = X[k][m] (TA), B(k, n) = X[k][n]. Symmetric: the
    // tiles on and below the diagonal, then the upper ones mirrored (element
    // (j, i) is the same products summed in the same token order as (i, j))
    dgemm<T, T, true, false, true>(in, in, tokens, 2.0, X, in, X, in, 0.0, H, in, st);
    const unsigned tiles = (unsigned)((in + 63) / 64);
    hipLaunchKernelGGL(k_mirror_upper, dim3(tiles, tiles), dim3(256), 0, st, H, in);
}

hipError_t launch_gptq_hessian(const void *X, int dtype, int64_t tokens, int64_t in, double damp, double *H,
                               hipStream_t st)
{
    switch (dtype) {
    case AWQ_F32: hessian_typed((const float *)X, tokens, in, H, st); break;
    case AWQ_F16: hessian_typed((const f16 *)X, tokens, in, H, st); break;
    default: hessian_typed((const bf16 *)X, tokens, in, H, st); break;
    }
    hipLaunchKernelGGL(k_damp, dim3(1), dim3(256), 0, st, H, in, damp);
    return hipGetLastError();
}

static unsigned stream_blocks(int64_t total)
{
    const int64_t b = (total + 255) / 256;
    return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

// U = J L^-1 J, L the lower Cholesky factor of J H J. ws: n*n + n*n/4 doubles.
hipError_t launch_gptq_factor(const double *H, int64_t n, double *U, double *ws, hipStream_t st)
{
    const int64_t total = n * n;
    double *Lr = ws;                       // J H J, then (lower part) its Cholesky factor
    double *T = ws + total;                // products of the inverse's doubling steps (n*n/4)
    hipLaunchKernelGGL(k_reverse_copy, dim3(stream_blocks(total)), dim3(256), 0, st, H, Lr, total);
    // The first diagonal block on its own; every later one is factored by the
    // workgroup of the trailing update that writes it (POTRF).
    const int64_t nb = n / kNb;
    hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, st, Lr, n, (int64_t)0);
    for (int64_t k = 0; k + 1 < nb; ++k) {
        const int64_t k0 = k * kNb, rest = n - k0 - kNb;
        hipLaunchKernelGGL(k_trsm_panel, dim3((unsigned)((rest + kTrsmRows - 1) / kTrsmRows)),
                           dim3(kTrsmRows * 64), 0, st, Lr, n, k0);
        // trailing lower triangle -= P P^T, P = the panel below the diagonal
        // block; then the next diagonal block is factored in place
        const double *P = Lr + (k0 + kNb) * n + k0;
        dgemm<double, double, false, true, true, true, 2, true>(rest, rest, kNb, -1.0, P, n, P, n, 1.0,
                                                       Lr + (k0 + kNb) * n + k0 + kNb, n, st);
    }
    // Li = L^-1 in U's buffer, bottom up: invert the 64 x 64 diagonal blocks,
    // then, with the inverses of every aligned run of s blocks known, combine
    // neighbouring runs A (first) and C (second) into the inverse of their
    // union: its lower-left part is -C^-1 (L21 A^-1). Each level is two batched
    // GEMMs (T = L21 A^-1 into scratch, then -C^-1 T); a last, shorter run is
    // combined on its own.
    double *Li = U;
    double *Tb = T;
    hipLaunchKernelGGL(k_fill0, dim3(stream_blocks(total)), dim3(256), 0, st, Li, total);
    hipLaunchKernelGGL(k_trtri_diag, dim3((unsigned)nb), dim3(64), 0, st, Lr, Li, n);
    for (int64_t s = 1; s < nb; s *= 2) {
        const int64_t S = s * kNb, full = nb / (2 * s), step = 2 * S * n + 2 * S;
        // A^-1 and C^-1 are lower triangular (zeros above their diagonals)
        if (full > 0) {
            dgemm<double, double, false, false, false, false, 2, false, 1>(S, S, S, 1.0, Lr + S * n, n, Li, n, 0.0,
                                                                         Tb, S, st, full, step, step, S * S);
            dgemm<double, double, false, false, false, false, 2, false, 2>(S, S, S, -1.0, Li + S * n + S, n, Tb, S,
                                                                         0.0, Li + S * n, n, st, full, step,
                                                                         S * S, step);
        }
        const int64_t rem = nb - full * 2 * s;
        if (rem > s) {
            const int64_t base = full * 2 * S, S2 = (rem - s) * kNb;
            dgemm<double, double, false, false, false, false, 2, false, 1>(S2, S, S, 1.0, Lr + (base + S) * n + base,
                                                                         n, Li + base * n + base, n, 0.0, Tb, S,
                                                                         st);
            dgemm<double, double, false, false, false, false, 2, false, 2>(S2, S, S2, -1.0,
                                                                         Li + (base + S) * n + base + S, n, Tb, S,
                                                                         0.0, Li + (base + S) * n + base, n, st);
        }
    }
    hipLaunchKernelGGL(k_reverse_inplace, dim3(stream_blocks(total / 2)), dim3(256), 0, st, U, total);
    return hipGetLastError();
}

// The column loop. ws: out*in (corrected weights) + out*128 (block errors) doubles.
template <typename T>
__global__ __launch_bounds__(256) void k_widen(const T *__restrict__ W, double *__restrict__ Wc, int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
        Wc[e] = static_cast<double>(static_cast<float>(W[e]));
}

hipError_t launch_gptq_quantize(const void *W, int dtype, int64_t out, int64_t in, const double *U, int bits,
                                int group, int mode, uint32_t *qweight, float *scales, uint8_t *zeros,
                                double *ws, hipStream_t st)
{
    double *Wc = ws;
    double *E = ws + out * in;
    const int64_t total = out * in;
    switch (dtype) {
    case AWQ_F32:
        hipLaunchKernelGGL(k_widen<float>, dim3(stream_blocks(total)), dim3(256), 0, st, (const float *)W, Wc, total);
        break;
    case AWQ_F16:
        hipLaunchKernelGGL(k_widen<f16>, dim3(stream_blocks(total)), dim3(256), 0, st, (const f16 *)W, Wc, total);
        break;
    default:
        hipLaunchKernelGGL(k_widen<bf16>, dim3(stream_blocks(total)), dim3(256), 0, st, (const bf16 *)W, Wc, total);
        break;
    }
    for (int64_t b = 0; b < in; b += kCol) {
        hipLaunchKernelGGL(mode == AWQ_ASYM ? k_gptq_block<true> : k_gptq_block<false>,
                           dim3((unsigned)((out + kRowsPerGroup - 1) / kRowsPerGroup)),
                           dim3(kRowsPerGroup * kColRowLanes), 0, st, Wc, U, out, in, b, bits, group, E, qweight,
                           scales, zeros);
        const int64_t rest = in - b - kCol;
        if (rest > 0)   // later columns -= E U[b : b + 128][b + 128 :]
            dgemm<double, double, false, false, false, false, 2, true>(out, rest, kCol, -1.0, E, kCol,
                                                                      U + b * in + b + kCol, in, 1.0, Wc + b + kCol,
                                                                      in, st);
    }
    return hipGetLastError();
}

}  // namespace awq
