// Launcher of the LDS-tiled kernel (other state counts, zero-order-hold B), f32 storage.
#include "launch.hpp"
#include "scan_tiled.hpp"

namespace mscan {

int launch_tiled_f32(const ScanParams& q, hipStream_t stream) { return launch_tiled<float>(q, nullptr, 0, stream); }

bool tiled_can_run_f32(const ScanParams& q) { return tiled_can_run<float>(q); }

}  // namespace mscan
