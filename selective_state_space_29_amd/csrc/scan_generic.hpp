// Generic selective-scan kernel: one lane per (batch, channel) row, the whole sequence in order.
//
// It accepts every shape, stride and alignment the ABI allows (dstate up to 256, any len), so it
// is the fallback behind the tiled kernel. Each lane keeps up to NB states in registers; for
// dstate > NB it sweeps the sequence once per block of NB states, accumulating y in place (the
// same lane writes and re-reads its own outputs, so no synchronisation is involved) and applying
// the skip and gate on the last sweep.
//
// Per step and state it evaluates the recurrence of "Mamba代码实战…" §3.1-§3.2 as
//   dA = 2^(dt * A*log2(e)),  h = dA * h + (dt*u) * B,  y += C * h
// followed by the skip and silu gate of §3.3; with zoh_b the input term is the zero-order-hold
// one, (e^{dt A} - 1)/A * u * B.
#pragma once

#include "common.hpp"

namespace mscan {

template <typename T, int NB>
__global__ __launch_bounds__(64) void scan_generic_kernel(ScanParams p) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= p.batch * p.dim) return;
    const int64_t b = row / p.dim;
    const int64_t d = row - b * p.dim;
    const T* u = static_cast<const T*>(p.u) + b * p.su_b + d * p.su_d;
    const T* dl = static_cast<const T*>(p.delta) + b * p.sdt_b + d * p.sdt_d;
    const T* z = p.z ? static_cast<const T*>(p.z) + b * p.sz_b + d * p.sz_d : nullptr;
    const T* Bb = static_cast<const T*>(p.B) + b * p.sB_b;
    const T* Cb = static_cast<const T*>(p.C) + b * p.sC_b;
    float* y = p.y + b * p.sy_b + d * p.sy_d;
    const float bias = p.bias ? p.bias[d * p.sbias] : 0.0f;
    const float dskip = p.D ? p.D[d * p.sD] : 0.0f;
    const int64_t L = p.len;

    for (int64_t n0 = 0; n0 < p.dstate; n0 += NB) {
        const int nb = (int)((p.dstate - n0) < NB ? (p.dstate - n0) : NB);
        const bool first = (n0 == 0);
        const bool last = (n0 + NB >= p.dstate);
        float h[NB], a2[NB], an[NB], ian[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            h[j] = 0.0f;
            a2[j] = an[j] = ian[j] = 0.0f;
            if (j < nb) {
                an[j] = p.A[d * p.sA_d + n0 + j];
                a2[j] = an[j] * kLog2e;
                ian[j] = an[j] != 0.0f ? 1.0f / an[j] : 0.0f;
                if (p.h0) h[j] = p.h0[b * p.sh0_b + d * p.sh0_d + n0 + j];
            }
        }
        for (int64_t t = 0; t < L; ++t) {
            const float dt = delta_to_dt(to_f32(dl[t]) + bias, p.softplus);
            const float uu = to_f32(u[t]);
            const float dtu = dt * uu;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (j < nb) {
                    const float bv = to_f32(Bb[(n0 + j) * p.sB_n + t]);
                    const float cv = to_f32(Cb[(n0 + j) * p.sC_n + t]);
                    const float dA = hw_exp2(dt * a2[j]);
                    const float inc = p.zoh_b ? zoh_coef_f(dt, dt * an[j], dA, ian[j]) * uu * bv : dtu * bv;
                    h[j] = __builtin_fmaf(dA, h[j], inc);
                    acc = __builtin_fmaf(cv, h[j], acc);
                }
            }
            float yv = first ? acc : y[t] + acc;
            if (last) {
                yv = __builtin_fmaf(dskip, uu, yv);
                if (z) yv *= silu_f(to_f32(z[t]));
            }
            y[t] = yv;
        }
        if (p.last_state) {
            float* ls = p.last_state + b * p.sls_b + d * p.sls_d + n0;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (j < nb) ls[j] = h[j];
        }
    }
}

}  // namespace mscan
