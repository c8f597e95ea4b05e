// Issue-rate microkernels used by the benchmark to state the VALU and transcendental rates it
// measures against, as lane operations per second of the whole GPU: fp32 FMA, v_exp_f32, an fp32
// multiply whose operand comes through a DPP row broadcast, and a 4 FMA : 1 exp mix (the ratio of
// the scan's per-element work: two multiplies and two FMAs per exp), which shows whether the
// transcendental issues alongside the FMAs or adds its own time. Each thread runs 8 independent
// dependency chains (no memory traffic in the loop), 2048 threads per CU (8 waves per SIMD) so
// that issue, not latency, bounds the loop.
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

// every lane of each 16-lane row reads lane LANE of its row (bound_ctrl: all lanes valid)
template <int LANE>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + LANE, 0xF, 0xF, true));
}

__global__ __launch_bounds__(kThreads) void dpp_mul_rate_kernel(float* out, float seed) {
    float a[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) a[j] = seed + threadIdx.x * 1e-3f + j;
    const float b = 0.999f + threadIdx.x * 1e-9f;
    for (int i = 0; i < kIters; ++i) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            a[0] = row_bcast<0>(a[0]) * b;
            a[1] = row_bcast<1>(a[1]) * b;
            a[2] = row_bcast<2>(a[2]) * b;
            a[3] = row_bcast<3>(a[3]) * b;
            a[4] = row_bcast<4>(a[4]) * b;
            a[5] = row_bcast<5>(a[5]) * b;
            a[6] = row_bcast<6>(a[6]) * b;
            a[7] = row_bcast<7>(a[7]) * b;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += a[j];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// per round: 8 FMAs on 8 chains and 2 exps on 2 more, i.e. 2 units of (4 FMA + 1 exp)
__global__ __launch_bounds__(kThreads) void mix_rate_kernel(float* out, float seed) {
    float a[kChains], e[2];
#pragma unroll
    for (int j = 0; j < kChains; ++j) a[j] = seed + threadIdx.x * 1e-3f + j;
    e[0] = seed;
    e[1] = seed * 0.5f;
    const float b = 0.999f + threadIdx.x * 1e-9f, c = 1e-3f;
    for (int i = 0; i < kIters; ++i) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int j = 0; j < kChains; ++j) a[j] = __builtin_fmaf(a[j], b, c);
            e[0] = __builtin_amdgcn_exp2f(-e[0]);
            e[1] = __builtin_amdgcn_exp2f(-e[1]);
        }
    }
    float s = e[0] + e[1];
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += a[j];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Measures the rates on the current device: rates[0] = fp32 FMA lane-ops/s, rates[1] =
// v_exp_f32 lane-ops/s, rates[2] = DPP-broadcast multiply lane-ops/s, rates[3] = units of
// (4 FMA + 1 exp) per second and lane. Allocates a small output buffer and synchronises (a
// benchmark helper, not part of the scan library). Returns 0, or -1 on any HIP error.
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
    void (*const kernels[4])(float*, float) = {fma_rate_kernel, exp_rate_kernel, dpp_mul_rate_kernel,
                                                mix_rate_kernel};
    for (int k = 0; k < 4 && rc == 0; ++k) {
        float best = 1e30f;
        for (int rep = 0; rep < 4; ++rep) {  // first launch warms up; keep the fastest
            (void)hipEventRecord(e0, 0);
            hipLaunchKernelGGL(kernels[k], dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f);
            (void)hipEventRecord(e1, 0);
            if (hipEventSynchronize(e1) != hipSuccess) { rc = -1; break; }
            float ms = 0.0f;
            (void)hipEventElapsedTime(&ms, e0, e1);
            if (rep > 0 && ms < best) best = ms;
        }
        // per iteration and lane every kernel does 2 x kChains operations; the mix does
        // 2 x (8 FMA + 2 exp), i.e. 2 x kChains / 4 units of (4 FMA + 1 exp)
        rates[k] = (k == 3 ? lane_ops / 4.0 : lane_ops) / (best * 1e-3);
    }
    if (hipGetLastError() != hipSuccess) rc = -1;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    return rc;
}

}  // extern "C"
