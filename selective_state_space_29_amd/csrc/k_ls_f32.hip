// Launcher of the lane-per-state kernels (16, 32, 64 states), f32 storage.
#include "launch.hpp"
#include "scan_ls.hpp"

namespace mscan {

int launch_ls_f32(const ScanParams& q, hipStream_t stream) { return launch_ls<float>(q, stream); }

}  // namespace mscan
