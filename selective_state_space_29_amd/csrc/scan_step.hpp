// Short-call kernel: calls of a few steps, such as recurrent decode (one step per call from the
// previous call's last_state), 16 states (gfx950).
//
// The same operation as the other kernels (the recurrence of "Mamba代码实战…" §3.1-§3.3, the
// contraction of "Mamba-minimal项目解析…" 关键技术点 1, started from the given state as the scan of
// "手把手用PyTorch实现Mamba的SSM层…" §3.1 takes it; the single-step inference "告别'炼丹'…" §2.1 times),
// laid out for a call whose cost is latency rather than work: one lane per (channel, state), a
// wave = 4 channels x 16 states, and every step done in registers with no LDS, no staging and no
// barrier. Each lane loads its own step inputs, 4 steps at a time before any is used (the 16 lanes
// of a channel read the same u / delta / z address, the 4 channels the same B / C), computes dt
// itself (the 16 lanes of a channel compute
// the same value), advances its state with exactly the arithmetic of the sequential kernels (so the
// state it returns is the same bits), and the channel's 16 C h terms are added by a DPP prefix sum
// across the row; the row's last lane finishes and stores y.
#pragma once

#include "common.hpp"

namespace mscan {

constexpr int kStepMaxLen = 4;  // the default for calls of at most this many steps
constexpr int kStepGroup = 4;   // steps whose inputs are loaded together before any is used
// Waves per workgroup (4 channels each). One-step calls take workgroups of 16 waves: few large
// workgroups dispatch faster, which is most of such a call (at the Mamba-130m width 3.34 us per
// call with 16 waves, 3.63 with 4 or 8). Longer calls take 4-wave workgroups, which spread the
// channels over every CU (with 16-wave ones, 2 steps per call took 4.46 us against 4.19).
constexpr int kStepWavesOne = 16;
constexpr int kStepWaves = 4;

// ZOH: B discretised by zero-order hold, the lane-per-state kernels' term (zoh_coef2_f times u,
// times B), so that the states are their bits in either mode.
template <typename T, int W, bool SOFTPLUS, bool HAS_Z, bool ZOH>
__global__ __launch_bounds__(64 * W) void scan_step_kernel(ScanParams p) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t blocks = (p.dim + 4 * W - 1) / (4 * W);
    const int64_t b = blockIdx.x / blocks;
    const int64_t d0 = (blockIdx.x - b * blocks) * (4 * W) + wave * 4;
    const int c = lane >> 4, n = lane & 15;
    const bool valid = d0 + c < p.dim;
    const int64_t d = valid ? d0 + c : p.dim - 1;

    const float an = p.A[d * p.sA_d + n];
    const float a2 = an * kLog2e;
    const float ia = an != 0.0f ? 1.0f / an : 0.0f;  // zero-order hold only
    float h = p.h0 ? p.h0[b * p.sh0_b + d * p.sh0_d + n] : 0.0f;
    const float bias = p.bias ? p.bias[d * p.sbias] : 0.0f;
    const float Dv = p.D ? p.D[d * p.sD] : 0.0f;  // no skip term: D = 0
    const T* ur = static_cast<const T*>(p.u) + b * p.su_b + d * p.su_d;
    const T* xr = static_cast<const T*>(p.delta) + b * p.sdt_b + d * p.sdt_d;
    const T* zr = HAS_Z ? static_cast<const T*>(p.z) + b * p.sz_b + d * p.sz_d : nullptr;
    const T* Br = static_cast<const T*>(p.B) + b * p.sB_b + n * p.sB_n;
    const T* Cr = static_cast<const T*>(p.C) + b * p.sC_b + n * p.sC_n;
    float* yr = p.y + b * p.sy_b + d * p.sy_d;
    const int64_t L = p.len;

    if (L == 1) {
        // one step (recurrent decode): each input loaded once, the same arithmetic as below
        const float xb = to_f32(xr[0]) + bias;
        const float dt = SOFTPLUS ? softplus_f(xb) : hw_exp2(xb * kLog2e);
        const float u0 = to_f32(ur[0]);
        const float x2 = dt * a2;
        const float dA = hw_exp2(x2);
        h = __builtin_fmaf(dA, h, (ZOH ? zoh_coef2_f(dt, x2, dA, ia) : dt) * u0 * to_f32(Br[0]));
        float s = to_f32(Cr[0]) * h;
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x111, 0xF, 0xF, false));
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x112, 0xF, 0xF, false));
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x114, 0xF, 0xF, false));
        s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x118, 0xF, 0xF, false));
        if (n == 15 && valid) {
            float o = __builtin_fmaf(Dv, u0, s);
            if constexpr (HAS_Z) o *= silu_f(to_f32(zr[0]));
            yr[0] = o;
        }
        if (p.last_state && valid) p.last_state[b * p.sls_b + d * p.sls_d + n] = h;
        return;
    }
    for (int64_t t0 = 0; t0 < L; t0 += kStepGroup) {
        // the group's inputs first (steps past len read step t0, whose values are not used), so
        // that one memory latency covers the group
        float xv[kStepGroup], uv[kStepGroup], zv[kStepGroup], bv[kStepGroup], cv[kStepGroup];
#pragma unroll
        for (int i = 0; i < kStepGroup; ++i) {
            const int64_t t = t0 + i < L ? t0 + i : t0;
            xv[i] = to_f32(xr[t]);
            uv[i] = to_f32(ur[t]);
            zv[i] = HAS_Z ? to_f32(zr[t]) : 0.0f;
            bv[i] = to_f32(Br[t]);
            cv[i] = to_f32(Cr[t]);
        }
#pragma unroll
        for (int i = 0; i < kStepGroup; ++i) {
            if (t0 + i >= L) break;  // uniform across the grid
            const float xb = xv[i] + bias;
            const float dt = SOFTPLUS ? softplus_f(xb) : hw_exp2(xb * kLog2e);
            const float x2 = dt * a2;
            const float dA = hw_exp2(x2);
            const float dtu = (ZOH ? zoh_coef2_f(dt, x2, dA, ia) : dt) * uv[i];
            h = __builtin_fmaf(dA, h, dtu * bv[i]);
            // sum over the row's 16 states: inclusive prefix sum, lane 15 ends with the total
            float s = cv[i] * h;
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x111, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x112, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x114, 0xF, 0xF, false));
            s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x118, 0xF, 0xF, false));
            if (n == 15 && valid) {
                float o = __builtin_fmaf(Dv, uv[i], s);
                if constexpr (HAS_Z) o *= silu_f(zv[i]);
                yr[t0 + i] = o;
            }
        }
    }
    if (p.last_state && valid) p.last_state[b * p.sls_b + d * p.sls_d + n] = h;
}

// ---------------------------------------------------------------------------------------------
// host side

constexpr int64_t kStepLimitLen = 64;  // the longest call it takes when forced

// 16 states, either input term, no saved states, at most kStepLimitLen steps (the default picks
// it for calls of at most kStepMaxLen steps).
inline bool step_eligible(const ScanParams& q) {
    return q.dstate == 16 && !q.ck && q.len <= kStepLimitLen &&
           q.batch * ((q.dim + 4 * kStepWaves - 1) / (4 * kStepWaves)) <= 0x7fffffff;  // the most workgroups
}

template <typename T, bool SP, bool HZ, bool ZOH>
int launch_step_cfg(const ScanParams& q, hipStream_t stream) {
    void* args[] = {const_cast<ScanParams*>(&q)};
    const bool one = q.len == 1;
    const int W = one ? kStepWavesOne : kStepWaves;
    const int64_t groups = q.batch * ((q.dim + 4 * W - 1) / (4 * W));
    const void* fn = one ? reinterpret_cast<const void*>(&scan_step_kernel<T, kStepWavesOne, SP, HZ, ZOH>)
                         : reinterpret_cast<const void*>(&scan_step_kernel<T, kStepWaves, SP, HZ, ZOH>);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * W), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T>
int launch_step(const ScanParams& q, hipStream_t stream) {
    if (!step_eligible(q)) return MAMBA_SCAN_ERR_UNSUPPORTED;
    const bool sp = q.softplus != 0, hz = q.z != nullptr;
    if (q.zoh_b) {
        if (sp && hz) return launch_step_cfg<T, true, true, true>(q, stream);
        if (sp) return launch_step_cfg<T, true, false, true>(q, stream);
        if (hz) return launch_step_cfg<T, false, true, true>(q, stream);
        return launch_step_cfg<T, false, false, true>(q, stream);
    }
    if (sp && hz) return launch_step_cfg<T, true, true, false>(q, stream);
    if (sp) return launch_step_cfg<T, true, false, false>(q, stream);
    if (hz) return launch_step_cfg<T, false, true, false>(q, stream);
    return launch_step_cfg<T, false, false, false>(q, stream);
}

}  // namespace mscan
