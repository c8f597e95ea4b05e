// Launcher of the lane-per-state kernels (16, 32, 64 states), bf16 storage.
#include "launch.hpp"
#include "scan_ls.hpp"

namespace mscan {

int launch_ls_bf16(const ScanParams& q, hipStream_t stream) { return launch_ls<bf16_t>(q, stream); }

}  // namespace mscan
