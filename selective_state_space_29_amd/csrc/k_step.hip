// Launcher of the short-call kernel (decode: a few steps per call, 16 states).
#include "launch.hpp"
#include "scan_step.hpp"

namespace mscan {

int launch_step_any(const ScanParams& q, bool bf16, hipStream_t stream) {
    return bf16 ? launch_step<bf16_t>(q, stream) : launch_step<float>(q, stream);
}

}  // namespace mscan
