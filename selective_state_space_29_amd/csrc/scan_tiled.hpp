// LDS-tiled selective-scan kernel (placeholder until the tiled path lands).
#pragma once

#include "../../include/mamba_scan.h"
#include "common.hpp"

namespace mscan {

inline int64_t tiled_workspace_bytes(const mamba_scan_shape&, uint32_t) { return 0; }

template <typename T>
int launch_tiled(const ScanParams&, const mamba_scan_ptrs*, uint32_t, hipStream_t) {
    return MAMBA_SCAN_ERR_UNSUPPORTED;
}

}  // namespace mscan
