// Launcher of the lane-per-state backward pass with B discretised by zero-order hold (its own
// translation unit: the kernel's instantiations compile in parallel with the Euler ones).
#include "launch.hpp"
#include "scan_bwd_ls.hpp"

namespace mscan {

int launch_bwd_ls_zoh_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                          hipStream_t stream) {
    return bf16 ? launch_bwd_ls<bf16_t, true>(p, s, softplus, stream) : launch_bwd_ls<float, true>(p, s, softplus, stream);
}

}  // namespace mscan
