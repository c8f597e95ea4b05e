// Issue-rate microkernels used by the benchmark to state the VALU and transcendental rates it
// measures against: fp32 FMA and v_exp_f32 throughput of the whole GPU, as lane operations per
// second. Each thread runs 8 independent dependency chains (no memory traffic in the loop),
// 2048 threads per CU (8 waves per SIMD) so that issue, not latency, bounds the loop.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kChains = 8;
constexpr int kIters = 4096;
constexpr int kThreads = 256;
constexpr int kBlocksPerCu = 8;

__global__ __launch_bounds__(kThreads) void fma_rate_kernel(float* out, float seed) {
    float a[kChains], b[4], c[4];
#pragma unroll
    for (int j = 0; j < kChains; ++j) a[j] = seed + threadIdx.x * 1e-3f + j;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b[j] = 0.999f + j * 1e-4f + threadIdx.x * 1e-9f;
        c[j] = 1e-3f + j * 1e-4f;
    }
    for (int i = 0; i < kIters; ++i) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < kChains; ++j) a[j] = __builtin_fmaf(a[j], b[j & 3], c[j & 3]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += a[j];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void exp_rate_kernel(float* out, float seed) {
    float a[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) a[j] = seed + threadIdx.x * 1e-3f + j * 0.1f;
    for (int i = 0; i < kIters; ++i) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < kChains; ++j) a[j] = __builtin_amdgcn_exp2f(-a[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += a[j];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Measures both rates on the current device; rates[0] = fp32 FMA lane-ops/s, rates[1] =
// v_exp_f32 lane-ops/s. Allocates a small output buffer and synchronises (a benchmark helper,
// not part of the scan library). Returns 0, or -1 on any HIP error.
int mscan_measure_rates(double* rates) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    const int blocks = cus * kBlocksPerCu;
    float* out = nullptr;
    if (hipMalloc(&out, sizeof(float) * blocks * kThreads) != hipSuccess) return -1;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    const double lane_ops = double(blocks) * kThreads * kIters * 2 * kChains;
    int rc = 0;
    for (int k = 0; k < 2 && rc == 0; ++k) {
        float best = 1e30f;
        for (int rep = 0; rep < 4; ++rep) {  // first launch warms up; keep the fastest
            (void)hipEventRecord(e0, 0);
            if (k == 0) hipLaunchKernelGGL(fma_rate_kernel, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f);
            else hipLaunchKernelGGL(exp_rate_kernel, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f);
            (void)hipEventRecord(e1, 0);
            if (hipEventSynchronize(e1) != hipSuccess) { rc = -1; break; }
            float ms = 0.0f;
            (void)hipEventElapsedTime(&ms, e0, e1);
            if (rep > 0 && ms < best) best = ms;
        }
        rates[k] = lane_ops / (best * 1e-3);
    }
    if (hipGetLastError() != hipSuccess) rc = -1;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    return rc;
}

}  // extern "C"
