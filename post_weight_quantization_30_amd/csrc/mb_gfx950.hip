// mb_gfx950.hip -- microbenchmarks behind the kernel design choices of
// libawq.so, on the GPU they run on. Standalone program (not part of the
// library); prints one JSON object.
//
// Every test launches one 512-thread block (8 waves) per compute unit; the
// 80 KB of dynamic LDS each block asks for keeps it alone on its CU, so waves
// w and w + 4 share SIMD w (the SIMD of every wave is read from HW_ID and
// reported). Each wave times its own loop with the shader clock
// (s_memtime); a test reports the median over all waves of the chip of the
// cycles per loop iteration, and the hipEvent time of the whole launch.
//
//  overlap: one SIMD running a wave that only issues matrix instructions
//    (8 independent v_mfma_f32_16x16x32_f16 per iteration) next to a wave
//    that only issues fp32 FMAs (8 * K per iteration on 8 independent
//    chains), against each of the two alone. If the two kinds of work share
//    the SIMD's time the pair takes the sum of the two alone; if they
//    co-execute, the longer of the two. The same with the two kinds
//    interleaved inside every wave (1 MFMA then K FMAs, placed by
//    sched_group_barrier).
//  valu: cycles per wave64 fp32 FMA with one and with two waves per SIMD.
//  lds_mfma: MFMAs whose B operand is read from LDS (ds_read_b128, 1 KB per
//    wave per read), each read serving R MFMAs, 2 waves per SIMD: shows
//    where the LDS read rate, not the matrix core, sets the pace.
//  f64_latency: cycles per dependent v_fma_f64 (one chain per wave) and per
//    independent one (8 chains).
//  mfma_data: the matrix core's rate and the shader clock in the search
//    kernel's launch shape (one 8-wave block per CU, two waves per SIMD,
//    6 independent 32x32x16 f16 accumulators per wave), once with operands
//    of random N(0, 1) fp16 values cycling over 4 A and 4 B fragments (the
//    data an error contraction sees) and once with fixed small operands.
//    The clock comes from the shader cycle counter (s_memtime) against the
//    100 MHz real-time counter (s_memrealtime) over each wave's loop.
//  layouts: the LDS placement of global_load_lds_dwordx4 (lane l's 16 bytes
//    at the wave-uniform LDS address + 16 l) and the lane layouts of the A,
//    B and C operands of
//    v_mfma_f32_16x16x32_f16 and v_mfma_f32_32x32x16_f16 checked against a
//    host product with small integer operands (exact in fp32).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <math.h>

#include <algorithm>
#include <vector>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kLdsPad = 80 * 1024;   // dynamic LDS per block: one block per CU
constexpr int kRec = 4;              // per wave: cycles lo, cycles hi, simd id, flag

enum Mode { M_ONLY = 0, V_ONLY, SPLIT, M_HALF, V_HALF, INTERLEAVE, INTERLEAVE_HALF };

__device__ __forceinline__ uint32_t simd_id()
{
    // HW_ID bits [5:4] hold the SIMD the wave runs on.
    return (__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4) >> 4) & 3u;
}

__device__ __forceinline__ void record(uint32_t *rec, uint64_t cyc, int active)
{
    if ((threadIdx.x & 63) == 0) {
        const int w = (int)(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
        rec[w * kRec + 0] = (uint32_t)cyc;
        rec[w * kRec + 1] = (uint32_t)(cyc >> 32);
        rec[w * kRec + 2] = simd_id();
        rec[w * kRec + 3] = (uint32_t)active;
    }
}

template <int K>
__device__ __forceinline__ void valu_step(float (&x)[8], float m, float c)
{
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = fmaf(x[j], m, c);
}

// One matrix instruction on accumulator c of the MFMA wave. MK 0: 16x16x32
// f16 with the accumulator in VGPRs (the compiler's choice); MK 1: the same
// with the accumulator in AGPRs (inline asm; the 8 accumulators are used
// round-robin, so every read of an accumulator is 7 instructions after its
// write); MK 2: 32x32x16 f16 (two accumulators per slot: the same FLOPs
// per iteration as 16 of the 16x16x32 instruction).
template <int MK>
__device__ __forceinline__ void mfma_slot(f32x4 (&acc)[8], f32x16 (&acc32)[4], const f16x8 &a,
                                          const f16x8 &b, int c)
{
    if (MK == 0) {
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    } else if (MK == 1) {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a), "v"(b));
    } else {
        acc32[c & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc32[c & 3], 0, 0, 0);
    }
}

template <int MODE, int K, int MK = 0>
__global__ __launch_bounds__(kThreads, 1) void k_overlap(uint32_t *rec, float *sink, int iters)
{
    extern __shared__ char pad[];
    const int t = threadIdx.x, wave = t >> 6;
    f16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (t + i));
        b[i] = (_Float16)(0.002f * (t - i));
    }
    f32x4 acc[8];
    for (int c = 0; c < 8; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x16 acc32[4];
    for (int c = 0; c < 4; ++c)
        acc32[c] = f32x16{};
    float x[8];
    for (int j = 0; j < 8; ++j)
        x[j] = 1.0f + 1e-3f * (t + j);
    float m = 0.999f, cc = 1e-4f;
    asm volatile("" : "+v"(m), "+v"(cc));   // VGPR operands, as in real kernels

    const bool do_m = MODE == M_ONLY || (MODE == SPLIT && wave < 4) || (MODE == M_HALF && wave < 4);
    const bool do_v = MODE == V_ONLY || (MODE == SPLIT && wave >= 4) || (MODE == V_HALF && wave >= 4);
    const bool do_i = MODE == INTERLEAVE || (MODE == INTERLEAVE_HALF && wave < 4);
    pad[t] = 0;
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    if (do_m) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < (MK == 2 ? 4 : 8); ++c)
                mfma_slot<MK>(acc, acc32, a, b, c);
        }
    } else if (do_v) {
        for (int it = 0; it < iters; ++it)
            valu_step<K>(x, m, cc);
    } else if (do_i) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (MK != 2 || (c & 1) == 0)
                    mfma_slot<MK>(acc, acc32, a, b, c >> (MK == 2));
#pragma unroll
                for (int k = 0; k < K; ++k)
                    x[(c + k) & 7] = fmaf(x[(c + k) & 7], m, cc);
            }
#pragma unroll
            for (int c = 0; c < (MK == 2 ? 4 : 8); ++c) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0002, MK == 2 ? 2 * K : K, 0);
            }
        }
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    record(rec, t1 - t0, do_m ? 1 : do_v ? 2 : do_i ? 3 : 0);
    float s = 0.f;
    for (int c = 0; c < 8; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    for (int c = 0; c < 4; ++c)
        s += acc32[c][0] + acc32[c][15];
    for (int j = 0; j < 8; ++j)
        s += x[j];
    sink[(size_t)blockIdx.x * kThreads + t] = s + pad[t ^ 1];
}

// MFMAs fed from LDS: every wave reads 8 B fragments (ds_read_b128, distinct
// 1 KB rows of a 64 KB buffer) per iteration and runs R MFMAs on each.
// PIPE: the reads of iteration it + 1 are issued before the MFMAs of
// iteration it.
template <int R, bool PIPE = false>
__global__ __launch_bounds__(kThreads, 1) void k_lds_mfma(uint32_t *rec, float *sink, int iters)
{
    extern __shared__ f16x8 lbuf[];   // 80 KB: 5120 fragments of 16 bytes
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < kLdsPad / 16; i += kThreads)
        for (int e = 0; e < 8; ++e)
            lbuf[i][e] = (_Float16)(1e-3f * ((i + e) & 15));
    f16x8 a;
    for (int i = 0; i < 8; ++i)
        a[i] = (_Float16)(0.001f * (t + i));
    f32x4 acc[8][R];
    for (int c = 0; c < 8; ++c)
        for (int r = 0; r < R; ++r)
            acc[c][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    int base = wave * 512;
    auto loadb = [&](f16x8 (&bf)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            bf[c] = lbuf[((base + c * 64) & 4095) + lane];
        base += 8 * 64;
    };
    auto mm = [&](const f16x8 (&bf)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[c][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[c], acc[c][r], 0, 0, 0);
    };
    f16x8 b0[8], b1[8];
    if (PIPE) {
        // two fragment sets: the reads of one set are placed between the
        // MFMAs of the other (one read, then R MFMAs)
        loadb(b0);
        for (int it = 0; it < iters; it += 2) {
            loadb(b1);
            mm(b0);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0008, R, 0);
            }
            loadb(b0);
            mm(b1);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0008, R, 0);
            }
        }
    } else {
        for (int it = 0; it < iters; ++it) {
            loadb(b0);
            mm(b0);
        }
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    record(rec, t1 - t0, 1);
    float s = 0.f;
    for (int c = 0; c < 8; ++c)
        for (int r = 0; r < R; ++r)
            s += acc[c][r][0] + acc[c][r][3];
    sink[(size_t)blockIdx.x * kThreads + t] = s;
}

// Raw LDS read rate: every wave issues 8 ds_read_b128 per iteration and
// folds the data with XORs. PAT 0: 64 distinct 16-byte addresses per read
// (1 KB); PAT 1: 4 distinct addresses, each shared by 16 consecutive lanes
// (a per-column vector that 16 rows read); PAT 2: one address for the wave.
template <int PAT>
__global__ __launch_bounds__(kThreads, 1) void k_lds_raw(uint32_t *rec, float *sink, int iters)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    extern __shared__ u32x4 lraw[];   // 80 KB: 5120 entries
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < kLdsPad / 16; i += kThreads)
        lraw[i] = u32x4{(uint32_t)i, (uint32_t)(i * 3), (uint32_t)(i * 5), (uint32_t)(i * 7)};
    __syncthreads();
    const int sub = PAT == 0 ? lane : PAT == 1 ? (lane >> 4) : 0;
    int base = wave * 512;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc ^= lraw[((base + c * 64) & 4095) + sub];
        base += 8 * 64;
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    record(rec, t1 - t0, 1);
    sink[(size_t)blockIdx.x * kThreads + t] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// fp64 FMA: CHAINS independent chains of dependent operations per wave.
template <int CHAINS>
__global__ __launch_bounds__(kThreads, 1) void k_f64(uint32_t *rec, float *sink, int iters)
{
    extern __shared__ char pad[];
    const int t = threadIdx.x, wave = t >> 6;
    double x[CHAINS];
    for (int j = 0; j < CHAINS; ++j)
        x[j] = 1.0 + 1e-6 * (t + j);
    const double m = 0.9999999, c = 1e-9;
    pad[t] = 0;
    __syncthreads();
    const bool act = wave < 4;   // one wave per SIMD
    const uint64_t t0 = __builtin_readcyclecounter();
    if (act)
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int j = 0; j < CHAINS; ++j)
                    x[j] = fma(x[j], m, c);
    const uint64_t t1 = __builtin_readcyclecounter();
    record(rec, t1 - t0, act);
    double s = 0.0;
    for (int j = 0; j < CHAINS; ++j)
        s += x[j];
    sink[(size_t)blockIdx.x * kThreads + t] = (float)s + pad[t ^ 1];
}

// Layout probes: A[i][k], B[k][j] small integers, C = A B exact in fp32.
// 16x16x32: lane l holds A row l%16, k = 8(l/16)..+7; B column l%16, same k;
//           C column l%16, rows 4(l/16)..+3.
// 32x32x16: lane l holds A row l%32, k = 8(l/32)..+7; B column l%32, same k;
//           C column l%32, rows 8(e/4) + 4(l/32) + e%4 for entry e = 0..15.
__device__ __forceinline__ float aval(int i, int k) { return (float)(((i * 7 + k * 3) % 11) - 5); }
__device__ __forceinline__ float bval(int k, int j) { return (float)(((k * 5 + j * 2) % 9) - 4); }

__global__ void k_layout(float *c16, float *c32)
{
    const int l = threadIdx.x;
    f16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)aval(l % 16, 8 * (l / 16) + e);
        b[e] = (_Float16)bval(8 * (l / 16) + e, l % 16);
    }
    f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    for (int e = 0; e < 4; ++e)
        c16[(4 * (l / 16) + e) * 16 + l % 16] = c[e];
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)aval(l % 32, 8 * (l / 32) + e);
        b[e] = (_Float16)bval(8 * (l / 32) + e, l % 32);
    }
    f32x16 z = {};
    f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, z, 0, 0, 0);
    for (int e = 0; e < 16; ++e)
        c32[(8 * (e / 4) + 4 * (l / 32) + e % 4) * 32 + l % 32] = d[e];
}

// global_load_lds_dwordx4: every wave copies 1 KB; lane l reads the 16
// bytes at src + 16 * (63 - l) (reversed, so the check sees the lane order);
// the LDS copy is written back in LDS order.
// HIGH: the LDS target sits 96 KB into the block's LDS (past 64 KB).
template <bool HIGH>
__global__ void k_lds_dma(const float *src, float *dst)
{
    __shared__ float buf[(HIGH ? 24576 : 0) + 256 * 4];
    float *tgt = buf + (HIGH ? 24576 : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 1024; i += blockDim.x)
        tgt[i] = -1.0f;
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + 256 * wave + 4 * (63 - lane)),
                                     (__attribute__((address_space(3))) void *)(tgt + 256 * wave), 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += blockDim.x)
        dst[i] = tgt[i];
}

// Matrix instructions on data: 24 v_mfma_f32_32x32x16_f16 per iteration over
// 6 accumulators, A and B cycling over 4 register fragments each. RANDOM:
// fragments loaded from src (random fp16); otherwise fixed small values.
// rec per wave: shader cycles (2 words), real-time ticks (2 words).
template <bool RANDOM>
__global__ __launch_bounds__(kThreads, 1) void k_mfma_data(const f16x8 *__restrict__ src, uint32_t *rec,
                                                           float *sink, int iters)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    f16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (RANDOM) {
            a[i] = src[(w * 8 + i) * 64 + lane];
            b[i] = src[(w * 8 + 4 + i) * 64 + lane];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[i][e] = (_Float16)(0.001f * (lane + e));
                b[i][e] = (_Float16)(0.002f * (lane - e));
            }
        }
    }
    f32x16 acc[6];
#pragma unroll
    for (int c = 0; c < 6; ++c)
        acc[c] = f32x16{};
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 24; ++j)
            acc[j % 6] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j % 4], b[(j / 4 + j) % 4], acc[j % 6], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            sum += acc[c][e];
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = sum;
    if (lane == 0) {
        rec[w * kRec + 0] = (uint32_t)(t1 - t0);
        rec[w * kRec + 1] = (uint32_t)((t1 - t0) >> 32);
        rec[w * kRec + 2] = (uint32_t)(r1 - r0);
        rec[w * kRec + 3] = (uint32_t)((r1 - r0) >> 32);
    }
}

static int g_cus = 0, g_clock_khz = 0;

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "mb_gfx950: %s failed: %s\n", #x, hipGetErrorString(e_));     \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

struct Result {
    double cyc_active;   // median cycles per iteration over the active waves
    double cyc_role[4];  // the same per role (1 matrix, 2 vector, 3 interleaved)
    double ms;           // event time of the launch
    int pairs_ok;        // waves w and w+4 reported the same SIMD in every block
};

template <typename KernelFn>
static Result run(KernelFn kern, uint32_t *rec, float *sink, int iters)
{
    const int nw = g_cus * (kThreads / 64);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(kern, dim3(g_cus), dim3(kThreads), kLdsPad, 0, rec, sink, iters);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(kern, dim3(g_cus), dim3(kThreads), kLdsPad, 0, rec, sink, iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    std::vector<uint32_t> h((size_t)nw * kRec);
    CHECK(hipMemcpy(h.data(), rec, h.size() * 4, hipMemcpyDeviceToHost));
    std::vector<double> cyc, role[4];
    int pairs_ok = 1;
    for (int w = 0; w < nw; ++w) {
        const double cw = (double)(((uint64_t)h[w * kRec + 1] << 32) | h[w * kRec + 0]) / iters;
        if (h[w * kRec + 3]) {
            cyc.push_back(cw);
            role[h[w * kRec + 3] & 3].push_back(cw);
        }
        const int wl = w % 8;
        if (wl < 4 && h[w * kRec + 2] != h[(w + 4) * kRec + 2])
            pairs_ok = 0;
    }
    std::sort(cyc.begin(), cyc.end());
    Result r;
    r.cyc_active = cyc.empty() ? 0.0 : cyc[cyc.size() / 2];
    for (int k = 0; k < 4; ++k) {
        std::sort(role[k].begin(), role[k].end());
        r.cyc_role[k] = role[k].empty() ? 0.0 : role[k][role[k].size() / 2];
    }
    r.ms = ms;
    r.pairs_ok = pairs_ok;
    return r;
}

template <int K, int MK>
static void overlap_case(uint32_t *rec, float *sink, int iters, bool last)
{
    const Result m4 = run(k_overlap<M_HALF, K, MK>, rec, sink, iters);
    const Result v4 = run(k_overlap<V_HALF, K, MK>, rec, sink, iters);
    const Result sp = run(k_overlap<SPLIT, K, MK>, rec, sink, iters);
    const Result m8 = run(k_overlap<M_ONLY, K, MK>, rec, sink, iters);
    const Result il4 = run(k_overlap<INTERLEAVE_HALF, K, MK>, rec, sink, iters);
    const Result il8 = run(k_overlap<INTERLEAVE, K, MK>, rec, sink, iters);
    printf("    \"mk%d_K%d\": {\"fma_per_iter\": %d, "
           "\"mfma_wave_alone\": %.1f, \"fma_wave_alone\": %.1f, "
           "\"split_mfma_wave\": %.1f, \"split_fma_wave\": %.1f, "
           "\"two_mfma_waves\": %.1f, \"interleaved_1_wave\": %.1f, \"interleaved_2_waves\": %.1f, "
           "\"pairs_share_simd\": %s}%s\n",
           MK, K, 8 * K, m4.cyc_role[1], v4.cyc_role[2], sp.cyc_role[1], sp.cyc_role[2],
           m8.cyc_role[1], il4.cyc_role[3], il8.cyc_role[3],
           (m4.pairs_ok && sp.pairs_ok) ? "true" : "false", last ? "" : ",");
}

// One launch of k_mfma_data: median cycles per iteration, median clock,
// matrix-core busy fraction per SIMD and the chip's TFLOP/s from event time.
template <bool RANDOM>
static void mfma_data_case(const f16x8 *src, uint32_t *rec, float *sink, int iters, bool last)
{
    const int nw = g_cus * (kThreads / 64);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(k_mfma_data<RANDOM>, dim3(g_cus), dim3(kThreads), kLdsPad, 0, src, rec, sink, iters);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(k_mfma_data<RANDOM>, dim3(g_cus), dim3(kThreads), kLdsPad, 0, src, rec, sink, iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    std::vector<uint32_t> h((size_t)nw * kRec);
    CHECK(hipMemcpy(h.data(), rec, h.size() * 4, hipMemcpyDeviceToHost));
    std::vector<double> cyc, ghz;
    for (int w = 0; w < nw; ++w) {
        const double c = (double)(((uint64_t)h[w * kRec + 1] << 32) | h[w * kRec + 0]);
        const double r = (double)(((uint64_t)h[w * kRec + 3] << 32) | h[w * kRec + 2]);
        cyc.push_back(c / iters);
        if (r > 0)
            ghz.push_back(c / r * 0.1);
    }
    std::sort(cyc.begin(), cyc.end());
    std::sort(ghz.begin(), ghz.end());
    const double c_med = cyc[cyc.size() / 2], g_med = ghz.empty() ? 0.0 : ghz[ghz.size() / 2];
    // two waves per SIMD, 24 instructions of 32 cycles each per wave and iteration
    const double busy = 2.0 * 24 * 32 / c_med;
    const double flop = (double)nw * iters * 24 * (2.0 * 32 * 32 * 16);
    printf("    \"%s\": {\"cycles_per_iter\": %.1f, \"clock_ghz\": %.3f, \"clock_ghz_min\": %.3f, "
           "\"clock_ghz_max\": %.3f, \"matrix_busy\": %.3f, \"tflops\": %.1f}%s\n",
           RANDOM ? "random_fp16" : "fixed_small", c_med, g_med, ghz.empty() ? 0.0 : ghz.front(),
           ghz.empty() ? 0.0 : ghz.back(), busy, flop / (ms * 1e-3) / 1e12, last ? "" : ",");
}

int main()
{
    int dev = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&g_cus, hipDeviceAttributeMultiprocessorCount, dev));
    CHECK(hipDeviceGetAttribute(&g_clock_khz, hipDeviceAttributeClockRate, dev));
    uint32_t *rec = nullptr;
    float *sink = nullptr;
    CHECK(hipMalloc(&rec, (size_t)g_cus * 8 * kRec * sizeof(uint32_t)));
    CHECK(hipMalloc(&sink, (size_t)g_cus * kThreads * sizeof(float)));
    const int iters = 4000;

    printf("{\n  \"cus\": %d, \"clock_khz\": %d,\n", g_cus, g_clock_khz);
    printf("  \"note\": \"cycles per loop iteration, median over active waves\",\n");

    // VALU alone: K = 8 -> 64 FMAs per iteration.
    {
        const Result v1 = run(k_overlap<V_HALF, 8>, rec, sink, iters);
        const Result v2 = run(k_overlap<V_ONLY, 8>, rec, sink, iters);
        printf("  \"valu\": {\"fma_per_iter\": 64, \"one_wave_per_simd\": %.1f, \"two_waves_per_simd\": %.1f, "
               "\"cycles_per_fma_one_wave\": %.2f, \"cycles_per_fma_simd_two_waves\": %.2f},\n",
               v1.cyc_active, v2.cyc_active, v1.cyc_active / 64, v2.cyc_active / 128);
    }
    printf("  \"overlap\": {\n");
    overlap_case<2, 0>(rec, sink, iters, false);
    overlap_case<4, 0>(rec, sink, iters, false);
    overlap_case<8, 0>(rec, sink, iters, false);
    overlap_case<2, 1>(rec, sink, iters, false);
    overlap_case<4, 1>(rec, sink, iters, false);
    overlap_case<8, 1>(rec, sink, iters, false);
    overlap_case<2, 2>(rec, sink, iters, false);
    overlap_case<4, 2>(rec, sink, iters, false);
    overlap_case<8, 2>(rec, sink, iters, true);
    printf("  },\n");
    {
        const Result m8 = run(k_overlap<M_ONLY, 2>, rec, sink, iters);
        const Result l1 = run(k_lds_mfma<1>, rec, sink, iters);
        const Result l2 = run(k_lds_mfma<2>, rec, sink, iters);
        const Result l4 = run(k_lds_mfma<4>, rec, sink, iters);
        const Result p1 = run(k_lds_mfma<1, true>, rec, sink, iters);
        const Result p2 = run(k_lds_mfma<2, true>, rec, sink, iters);
        // bytes per CU per cycle: 8 waves x 8 KB per iteration / cycles per iteration
        printf("  \"lds_mfma\": {\"mfma_only_8_per_iter\": %.1f, "
               "\"R1_cycles_8reads_8mfma\": %.1f, \"R2_cycles_8reads_16mfma\": %.1f, "
               "\"R4_cycles_8reads_32mfma\": %.1f, \"R1_lds_bytes_per_cu_clk\": %.1f, "
               "\"R2_lds_bytes_per_cu_clk\": %.1f, \"R4_lds_bytes_per_cu_clk\": %.1f, "
               "\"pipelined_R1_cycles\": %.1f, \"pipelined_R2_cycles\": %.1f},\n",
               m8.cyc_active, l1.cyc_active, l2.cyc_active, l4.cyc_active,
               8 * 8192.0 / l1.cyc_active, 8 * 8192.0 / l2.cyc_active, 8 * 8192.0 / l4.cyc_active,
               p1.cyc_active, p2.cyc_active);
    }
    {
        const Result r0 = run(k_lds_raw<0>, rec, sink, iters);
        const Result r1 = run(k_lds_raw<1>, rec, sink, iters);
        const Result r2 = run(k_lds_raw<2>, rec, sink, iters);
        // 8 waves x 8 reads x 1 KB delivered to lanes per iteration
        printf("  \"lds_raw\": {\"distinct_cycles\": %.1f, \"bcast16_cycles\": %.1f, \"same_addr_cycles\": %.1f, "
               "\"distinct_bytes_per_cu_clk\": %.1f, \"bcast16_bytes_per_cu_clk\": %.1f, "
               "\"same_addr_bytes_per_cu_clk\": %.1f},\n",
               r0.cyc_active, r1.cyc_active, r2.cyc_active, 65536.0 / r0.cyc_active,
               65536.0 / r1.cyc_active, 65536.0 / r2.cyc_active);
    }
    {
        // random fp16 operands, 8 fragments of 64 lanes x 8 values per wave
        const size_t n = (size_t)g_cus * (kThreads / 64) * 8 * 64 * 8;
        std::vector<_Float16> hsrc(n);
        uint64_t x = 0x9e3779b97f4a7c15ull;
        for (size_t i = 0; i < n; i += 2) {
            // Box-Muller on a 64-bit xorshift stream
            x ^= x << 13; x ^= x >> 7; x ^= x << 17;
            const double u1 = ((x >> 11) + 1.0) / 9007199254740993.0;
            x ^= x << 13; x ^= x >> 7; x ^= x << 17;
            const double u2 = (x >> 11) / 9007199254740992.0;
            const double rr = sqrt(-2.0 * log(u1));
            hsrc[i] = (_Float16)(rr * cos(6.283185307179586 * u2));
            hsrc[i + 1] = (_Float16)(rr * sin(6.283185307179586 * u2));
        }
        f16x8 *src = nullptr;
        CHECK(hipMalloc(&src, n * sizeof(_Float16)));
        CHECK(hipMemcpy(src, hsrc.data(), n * sizeof(_Float16), hipMemcpyHostToDevice));
        printf("  \"mfma_data\": {\n");
        mfma_data_case<true>(src, rec, sink, iters, false);
        mfma_data_case<false>(src, rec, sink, iters, true);
        printf("  },\n");
        CHECK(hipFree(src));
    }
    {
        const Result d1 = run(k_f64<1>, rec, sink, iters);
        const Result d8 = run(k_f64<8>, rec, sink, iters);
        printf("  \"f64_fma\": {\"dependent_cycles_per_op\": %.2f, \"independent_8_chains_cycles_per_op\": %.2f},\n",
               d1.cyc_active / 8, d8.cyc_active / 64);
    }
    {
        float *c16 = nullptr, *c32 = nullptr;
        CHECK(hipMalloc(&c16, 256 * sizeof(float)));
        CHECK(hipMalloc(&c32, 1024 * sizeof(float)));
        hipLaunchKernelGGL(k_layout, dim3(1), dim3(64), 0, 0, c16, c32);
        CHECK(hipDeviceSynchronize());
        std::vector<float> h16(256), h32(1024);
        CHECK(hipMemcpy(h16.data(), c16, 256 * 4, hipMemcpyDeviceToHost));
        CHECK(hipMemcpy(h32.data(), c32, 1024 * 4, hipMemcpyDeviceToHost));
        auto av = [](int i, int k) { return (float)(((i * 7 + k * 3) % 11) - 5); };
        auto bv = [](int k, int j) { return (float)(((k * 5 + j * 2) % 9) - 4); };
        int bad16 = 0, bad32 = 0;
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
                float s = 0.f;
                for (int k = 0; k < 32; ++k)
                    s += av(i, k) * bv(k, j);
                bad16 += h16[i * 16 + j] != s;
            }
        for (int i = 0; i < 32; ++i)
            for (int j = 0; j < 32; ++j) {
                float s = 0.f;
                for (int k = 0; k < 16; ++k)
                    s += av(i, k) * bv(k, j);
                bad32 += h32[i * 32 + j] != s;
            }
        // LDS DMA placement: expected dst[256 w + 4 l + e] = src[256 w + 4 (63 - l) + e]
        float *gs = nullptr, *gd = nullptr;
        CHECK(hipMalloc(&gs, 1024 * sizeof(float)));
        CHECK(hipMalloc(&gd, 1024 * sizeof(float)));
        std::vector<float> hs(1024), hd(1024);
        for (int i = 0; i < 1024; ++i)
            hs[i] = (float)i;
        CHECK(hipMemcpy(gs, hs.data(), 4096, hipMemcpyHostToDevice));
        int bad_dma = 0, bad_dma_high = 0;
        for (int high = 0; high < 2; ++high) {
            if (high)
                hipLaunchKernelGGL(k_lds_dma<true>, dim3(1), dim3(256), 0, 0, gs, gd);
            else
                hipLaunchKernelGGL(k_lds_dma<false>, dim3(1), dim3(256), 0, 0, gs, gd);
            CHECK(hipDeviceSynchronize());
            CHECK(hipMemcpy(hd.data(), gd, 4096, hipMemcpyDeviceToHost));
            for (int w = 0; w < 4; ++w)
                for (int l = 0; l < 64; ++l)
                    for (int e = 0; e < 4; ++e)
                        (high ? bad_dma_high : bad_dma) += hd[256 * w + 4 * l + e] != hs[256 * w + 4 * (63 - l) + e];
        }
        CHECK(hipFree(gs));
        CHECK(hipFree(gd));
        printf("  \"layouts\": {\"mfma_16x16x32_f16_mismatches\": %d, \"mfma_32x32x16_f16_mismatches\": %d, "
               "\"global_load_lds_dwordx4_mismatches\": %d, \"global_load_lds_dwordx4_above_64k_mismatches\": %d}\n",
               bad16, bad32, bad_dma, bad_dma_high);
        CHECK(hipFree(c16));
        CHECK(hipFree(c32));
    }
    printf("}\n");
    CHECK(hipFree(rec));
    CHECK(hipFree(sink));
    return 0;
}
