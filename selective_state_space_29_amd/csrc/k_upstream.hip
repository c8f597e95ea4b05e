// Launcher of the block's upstream stages (conv1d + SiLU, x_proj, dt_proj on MFMA).
#include "launch.hpp"
#include "block_upstream.hpp"

namespace mscan {

int launch_upstream_any(const UpParams& q, int d_conv, hipStream_t stream) { return launch_upstream(q, d_conv, stream); }

}  // namespace mscan
