// Launchers of the segment-tiled backward pass (B/C widening, scan, fixed-order reduction) and of
// the reduction both backward kernels end with.
#include "launch.hpp"
#include "scan_bwd.hpp"

namespace mscan {

int launch_bwd_tiled_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                         hipStream_t stream) {
    return bf16 ? launch_bwd<bf16_t>(p, s, softplus, stream) : launch_bwd<float>(p, s, softplus, stream);
}

int launch_bwd_reduce_any(const BwdReduceParams& r, hipStream_t stream) { return launch_bwd_reduce(r, stream); }

// dst[i] = src ? src[i] : 0 for i < n (contiguous fp32): the gradients of a call with no steps or
// no rows, which are sums over nothing, or, for the initial state over no steps, the incoming
// gradient of the final state. A kernel rather than a memset or copy, so that a captured graph
// holds only kernel nodes.
__global__ __launch_bounds__(256) void bwd_fill_kernel(float* dst, const float* src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.0f;
}

int launch_bwd_fill(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (n <= 0 || !dst) return MAMBA_SCAN_OK;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    void* args[] = {&dst, &src, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_fill_kernel), dim3((unsigned)blocks), dim3(256), args,
                           0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

}  // namespace mscan
