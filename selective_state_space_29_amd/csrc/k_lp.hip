// Launcher of the chunked kernel (parallel along the sequence, 16 states).
#include "launch.hpp"
#include "scan_lp.hpp"

namespace mscan {

int launch_lp_any(const ScanParams& q, bool bf16, hipStream_t stream) {
    return bf16 ? launch_lp<bf16_t>(q, stream) : launch_lp<float>(q, stream);
}

}  // namespace mscan
