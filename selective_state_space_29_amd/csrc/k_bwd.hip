// Launchers of the segment-tiled backward pass (B/C widening, scan, fixed-order reduction) and of
// the reduction both backward kernels end with.
#include "launch.hpp"
#include "scan_bwd.hpp"

namespace mscan {

int launch_bwd_tiled_any(const mamba_scan_bwd_ptrs* p, const mamba_scan_shape& s, bool bf16, bool softplus,
                         hipStream_t stream) {
    return bf16 ? launch_bwd<bf16_t, false>(p, s, softplus, stream) : launch_bwd<float, false>(p, s, softplus, stream);
}

// Fixed-order sums of the partials: dB, dC over channel groups (4 steps per thread, 16-byte loads
// of the partials, groups added in order); dA, dD, dbias over the batch.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdReduceParams p) {
    const int64_t lp4 = p.lp / 4;
    const int64_t nbc4 = p.batch * p.dstate * lp4;  // 4-step columns per output tensor
    const int64_t na = p.dim * p.dstate;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < 2 * nbc4) {
        const int64_t q = i / nbc4, j = i - q * nbc4;
        const int64_t row = j / lp4;  // b * dstate + n
        const int64_t t = (j - row * lp4) * 4;
        const int64_t b = row / p.dstate, n = row - b * p.dstate;
        const float* src = p.bcpart + ((b * 2 + q) * p.dstate + n) * p.lp + t;
        const int64_t gs = p.batch * 2 * p.dstate * p.lp;  // floats between channel groups
        // the partials are read once: nontemporal loads (461 -> 455 us per backward call at the
        // Mamba-130m shape, with the full-row float4 stores below)
        typedef float nt_f4 __attribute__((ext_vector_type(4)));
        const nt_f4 a0 = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(src));
        float4 acc = make_float4(a0.x, a0.y, a0.z, a0.w);
#pragma unroll 8
        for (int64_t g = 1; g < p.groups; ++g) {
            const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(src + g * gs));
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        float* dst = (q ? p.dC : p.dB) + row * p.len + t;
        const float a[4] = {acc.x, acc.y, acc.z, acc.w};
        if (t + 4 <= p.len && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            *reinterpret_cast<float4*>(dst) = acc;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (t + k < p.len) dst[k] = a[k];
        }
    } else if (i < 2 * nbc4 + na) {
        // over the batch, and within a batch over the sequence parts in order
        const int64_t j = i - 2 * nbc4;
        float acc = 0.0f;
        for (int64_t b = 0; b < p.batch; ++b)
            for (int64_t q = 0; q < p.parts; ++q) acc += p.apart[(q * p.batch + b) * na + j];
        p.dA[j] = acc;
    } else if (i < 2 * nbc4 + na + p.dim) {
        const int64_t d = i - 2 * nbc4 - na;
        float accd = 0.0f, accb = 0.0f;
        for (int64_t b = 0; b < p.batch; ++b)
            for (int64_t q = 0; q < p.parts; ++q) {
                accd += p.dpart[(q * p.batch + b) * p.dim + d];
                accb += p.bpart[(q * p.batch + b) * p.dim + d];
            }
        if (p.dD) p.dD[d] = accd;
        if (p.dbias) p.dbias[d] = accb;
    }
}

int launch_bwd_reduce_any(const BwdReduceParams& r, hipStream_t stream) {
    const int64_t nred = 2 * r.batch * r.dstate * (r.lp / 4) + r.dim * r.dstate + r.dim;
    void* rargs[] = {const_cast<BwdReduceParams*>(&r)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_reduce_kernel), dim3((unsigned)((nred + 255) / 256)),
                           dim3(256), rargs, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}


// dst[i] = src ? src[i] : 0 for i < n (contiguous fp32): the gradients of a call with no steps or
// no rows, which are sums over nothing, or, for the initial state over no steps, the incoming
// gradient of the final state. A kernel rather than a memset or copy, so that a captured graph
// holds only kernel nodes.
__global__ __launch_bounds__(256) void bwd_fill_kernel(float* dst, const float* src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.0f;
}

int launch_bwd_fill(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (n <= 0 || !dst) return MAMBA_SCAN_OK;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    void* args[] = {&dst, &src, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_fill_kernel), dim3((unsigned)blocks), dim3(256), args,
                           0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

}  // namespace mscan
