// Launchers of the kernel families, each compiled in a translation unit of its own (so that the
// library builds in parallel); the C-ABI entry points in mamba_scan.hip call only these.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/mamba_scan.h"
#include "common.hpp"

namespace mscan {

struct UpParams;

int launch_generic_any(const ScanParams& q, bool bf16, hipStream_t stream);
int launch_tiled_bf16(const ScanParams& q, hipStream_t stream);
int launch_tiled_f32(const ScanParams& q, hipStream_t stream);
bool tiled_can_run_bf16(const ScanParams& q);
bool tiled_can_run_f32(const ScanParams& q);
int launch_ls_bf16(const ScanParams& q, hipStream_t stream);
int launch_ls_f32(const ScanParams& q, hipStream_t stream);
int launch_lp_any(const ScanParams& q, bool bf16, hipStream_t stream);
int launch_step_any(const ScanParams& q, bool bf16, hipStream_t stream);

inline int launch_tiled_any(const ScanParams& q, bool bf16, hipStream_t stream) {
    return bf16 ? launch_tiled_bf16(q, stream) : launch_tiled_f32(q, stream);
}
inline bool tiled_can_run_any(const ScanParams& q, bool bf16) {
    return bf16 ? tiled_can_run_bf16(q) : tiled_can_run_f32(q);
}
inline int launch_ls_any(const ScanParams& q, bool bf16, hipStream_t stream) {
    return bf16 ? launch_ls_bf16(q, stream) : launch_ls_f32(q, stream);
}
// the forward that saves the segment states (q.ck), on the kernel a forward call would choose
int launch_fwd_checkpoints(const ScanParams& q, bool bf16, hipStream_t stream);
struct BwdReduceParams;
// the backward: the segment-tiled kernel (any dstate) or the lane-per-state one (16 states), each
// finished by the fixed-order reduction
int launch_bwd_tiled_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                         hipStream_t stream);
int launch_bwd_tiled_zoh_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                             hipStream_t stream);
int launch_bwd_ls_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                      hipStream_t stream);
int launch_bwd_ls_zoh_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                          hipStream_t stream);
int launch_bwd_reduce_any(const BwdReduceParams& r, hipStream_t stream);
// dst[i] = src ? src[i] : 0 for i < n, contiguous fp32 (the gradients of empty backward calls)
int launch_bwd_fill(float* dst, const float* src, int64_t n, hipStream_t stream);
int launch_upstream_any(const UpParams& q, int d_conv, hipStream_t stream);

}  // namespace mscan
