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

}  // namespace mscan
