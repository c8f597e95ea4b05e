// Launcher of the LDS-tiled kernel (other state counts, zero-order-hold B), bf16 storage.
#include "launch.hpp"
#include "scan_tiled.hpp"

namespace mscan {

int launch_tiled_bf16(const ScanParams& q, hipStream_t stream) { return launch_tiled<bf16_t>(q, nullptr, 0, stream); }

bool tiled_can_run_bf16(const ScanParams& q) { return tiled_can_run<bf16_t>(q); }

}  // namespace mscan
