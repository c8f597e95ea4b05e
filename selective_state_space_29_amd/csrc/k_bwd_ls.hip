// Launcher of the lane-per-state backward pass (16 states).
#include "launch.hpp"
#include "scan_bwd_ls.hpp"

namespace mscan {

int launch_bwd_ls_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                      hipStream_t stream) {
    return bf16 ? launch_bwd_ls<bf16_t, false>(p, s, softplus, stream) : launch_bwd_ls<float, false>(p, s, softplus, stream);
}

}  // namespace mscan
