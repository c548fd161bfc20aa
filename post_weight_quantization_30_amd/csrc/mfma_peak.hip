// mfma_peak.hip -- attainable dense MFMA throughput on this GPU, the second
// peak the search kernel is compared with (beside the spec sheet's).
//
// 8 waves per block, 2 or more blocks per CU, each wave cycling 8 independent
// accumulators through v_mfma_f32_16x16x32_{f16,bf16} with register operands:
// no memory traffic, no other work. Prints one JSON line with the best of 5
// timed launches per operand type. Standalone program (not part of
// libawq.so); bench.py runs it as a child process.
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAcc = 8;
constexpr int kThreads = 512;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_mfma_loop(float *out, int iters)
{
    const int t = threadIdx.x;
    f16x8 a, b;
    bf16x8 ab, bb;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (t + i));
        b[i] = (_Float16)(0.002f * (t - i));
        ab[i] = (__bf16)(0.001f * (t + i));
        bb[i] = (__bf16)(0.002f * (t - i));
    }
    f32x4 acc[kAcc];
    for (int c = 0; c < kAcc; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kAcc; ++c) {
            if (BF16)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, acc[c], 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
        }
    }
    float s = 0.f;
    for (int c = 0; c < kAcc; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(size_t)blockIdx.x * blockDim.x + t] = s;   // keeps the loop live
}

template <bool BF16>
static double measure(float *out, int blocks, int iters)
{
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
        return -1.0;
    for (int w = 0; w < 2; ++w)
        hipLaunchKernelGGL(k_mfma_loop<BF16>, dim3(blocks), dim3(kThreads), 0, 0, out, iters);
    if (hipDeviceSynchronize() != hipSuccess)
        return -1.0;
    float best = 1e30f;
    for (int r = 0; r < 5; ++r) {
        (void)hipEventRecord(e0);
        hipLaunchKernelGGL(k_mfma_loop<BF16>, dim3(blocks), dim3(kThreads), 0, 0, out, iters);
        (void)hipEventRecord(e1);
        if (hipEventSynchronize(e1) != hipSuccess)
            return -1.0;
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, e0, e1);
        best = ms < best ? ms : best;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    const double flop = (double)blocks * (kThreads / 64) * iters * kAcc * (2.0 * 16 * 16 * 32);
    return flop / (best * 1e-3) / 1e12;
}

int main()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        fprintf(stderr, "mfma_peak: no HIP device\n");
        return 1;
    }
    const int blocks = 2 * cus, iters = 20000;
    float *out = nullptr;
    if (hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)) != hipSuccess) {
        fprintf(stderr, "mfma_peak: hipMalloc failed\n");
        return 1;
    }
    const double f16 = measure<false>(out, blocks, iters);
    const double bf16 = measure<true>(out, blocks, iters);
    (void)hipFree(out);
    if (f16 < 0 || bf16 < 0) {
        fprintf(stderr, "mfma_peak: a HIP call failed\n");
        return 1;
    }
    printf("{\"mfma_16x16x32_f16_tflops\": %.1f, \"mfma_16x16x32_bf16_tflops\": %.1f, \"cus\": %d}\n", f16,
           bf16, cus);
    return 0;
}
