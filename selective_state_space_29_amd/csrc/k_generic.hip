// Launcher of the generic kernel (one lane per row; any shape).
#include "launch.hpp"
#include "scan_generic.hpp"

namespace mscan {

namespace {
template <typename T>
int launch_generic(const ScanParams& q, hipStream_t stream) {
    const int64_t rows = q.batch * q.dim;
    const dim3 grid((unsigned)((rows + 63) / 64));
    const dim3 block(64);
    void* args[] = {const_cast<ScanParams*>(&q)};
    const void* fn;
    if (q.dstate <= 16)
        fn = reinterpret_cast<const void*>(&scan_generic_kernel<T, 16>);
    else if (q.dstate <= 32)
        fn = reinterpret_cast<const void*>(&scan_generic_kernel<T, 32>);
    else
        fn = reinterpret_cast<const void*>(&scan_generic_kernel<T, 64>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream) == hipSuccess ? MAMBA_SCAN_OK : MAMBA_SCAN_ERR_LAUNCH;
}
}  // namespace

int launch_generic_any(const ScanParams& q, bool bf16, hipStream_t stream) {
    return bf16 ? launch_generic<bf16_t>(q, stream) : launch_generic<float>(q, stream);
}

}  // namespace mscan
