// LDS-tiled selective-scan kernel for gfx950.
//
// Work decomposition. A workgroup owns 64 consecutive channels d of one batch b (one channel per
// lane) and walks the sequence in chunks of TC steps. Its W waves split the N states: wave w
// carries states n = w*S .. w*S+S-1 for all 64 channels, in registers, across the whole sequence.
//   * B[b, n, t] and C[b, n, t] are then the same for every lane of a wave: they are read with
//     scalar loads into SGPRs and enter the VALU as scalar operands at no per-lane cost.
//   * The per-(channel, step) work that does not depend on n - the biased softplus/exp of delta,
//     dt*u, the skip D*u and the silu gate - is done once per chunk by the whole workgroup
//     (each thread takes 4 consecutive steps of one channel, so global accesses are 8/16-byte
//     vectors along L) and shared through LDS.
// Per element (b, d, t, n) the inner loop is then the minimum the recurrence needs:
//   v_mul (dt * A*log2e), v_exp (2^x), v_mul (dt*u * B), v_fma (h = dA*h + dBu), v_fma (y += C*h)
// with fp32 state kept in VGPRs. The W partial outputs of a step are summed in LDS in wave order
// (deterministic), then skip and gate are applied and y is stored as 16-byte vectors.
// This is the recurrence of "Mamba代码实战…" §3.1-§3.3 with the output contraction of
// "Mamba-minimal项目解析…" 关键技术点 1, fused so that no (B, D, L, N) tensor is ever formed (the
// page itself materialises dA and dB, §3.1).
//
// Per chunk: prologue (chunk c) -> barrier -> main loop -> barrier -> epilogue (chunk c).
// The raw inputs of chunk c+1 are loaded into registers before chunk c's main loop, so their
// latency hides behind it.
#pragma once

#include "../../include/mamba_scan.h"
#include "common.hpp"

namespace mscan {

typedef const __attribute__((address_space(4))) uint32_t* cptr32;  // scalar-load pointer
typedef const __attribute__((address_space(4))) float* cptrf;

template <typename T>
struct Quad;  // 4 consecutive steps of one tensor row, as loaded

template <>
struct Quad<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ void load_tail(const float* p, int n) {
        v.x = n > 0 ? p[0] : 0.0f;
        v.y = n > 1 ? p[1] : 0.0f;
        v.z = n > 2 ? p[2] : 0.0f;
        v.w = n > 3 ? p[3] : 0.0f;
    }
    __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ float4 f32() const { return v; }
};

template <>
struct Quad<bf16_t> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ void load_tail(const bf16_t* p, int n) {
        const uint32_t e0 = n > 0 ? p[0].bits : 0u, e1 = n > 1 ? p[1].bits : 0u;
        const uint32_t e2 = n > 2 ? p[2].bits : 0u, e3 = n > 3 ? p[3].bits : 0u;
        v.x = e0 | (e1 << 16);
        v.y = e2 | (e3 << 16);
    }
    __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
    __device__ __forceinline__ float4 f32() const {
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// Four consecutive B (or C) values of one state, wave-uniform, through the scalar cache.
// `off` is the element offset of the first one; it is even for bf16 (checked on the host).
__device__ __forceinline__ float4 uniform_quad(const float* base, int64_t off) {
    const cptrf p = (cptrf)(base + off);
    return make_float4(p[0], p[1], p[2], p[3]);
}
__device__ __forceinline__ float4 uniform_quad(const bf16_t* base, int64_t off) {
    const cptr32 p = (cptr32)(base + off);
    const uint32_t w0 = p[0], w1 = p[1];
    return make_float4(__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                       __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u));
}
// One value, per lane (same address in every lane); used in the tail chunk only.
__device__ __forceinline__ float lane_load(const float* base, int64_t off) { return base[off]; }
__device__ __forceinline__ float lane_load(const bf16_t* base, int64_t off) { return to_f32(base[off]); }

__device__ __forceinline__ float f4get(const float4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}
__device__ __forceinline__ void f4set(float4& v, int j, float x) {
    if (j == 0) v.x = x; else if (j == 1) v.y = x; else if (j == 2) v.z = x; else v.w = x;
}

template <typename T, int S, int W, int TC>
__global__ __launch_bounds__(64 * W) void scan_tiled_kernel(ScanParams p) {
    constexpr int NQ = TC / 4;          // step quads per chunk
    constexpr int ROWP = TC + 4;        // padded LDS row (floats) of one channel
    constexpr int PAIRS = 64 * NQ;      // (channel, quad) pairs per chunk
    constexpr int PPT = PAIRS / (64 * W);
    static_assert(TC % 4 == 0 && PAIRS % (64 * W) == 0 && PPT >= 1, "chunk/waves mismatch");

    __shared__ float s_dt[64 * ROWP];
    __shared__ float s_dtu[64 * ROWP];
    __shared__ float s_yp[W * 64 * ROWP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ngroups = (p.dim + 63) / 64;
    const int64_t b = blockIdx.x / ngroups;
    const int64_t d0 = (blockIdx.x - b * ngroups) * 64;
    const int64_t L = p.len;
    const int N = (int)p.dstate;
    const int nbase = wave * S;
    const bool wave_live = nbase < N;            // the host guarantees N % S == 0
    const int w_live = (N + S - 1) / S;          // waves that carry states

    const T* __restrict__ u = static_cast<const T*>(p.u);
    const T* __restrict__ dl = static_cast<const T*>(p.delta);
    const T* __restrict__ z = static_cast<const T*>(p.z);
    const T* __restrict__ Bm = static_cast<const T*>(p.B);
    const T* __restrict__ Cm = static_cast<const T*>(p.C);

    // ---- prologue/epilogue roles: PPT (channel, quad) pairs per thread, fixed channel ----
    int pr[PPT], pq[PPT];
    bool pvalid[PPT];
    float pbias[PPT], pskip[PPT];
    int64_t off_u[PPT], off_dl[PPT], off_z[PPT], off_y[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int pidx = tid + k * 64 * W;
        pr[k] = pidx / NQ;
        pq[k] = pidx - pr[k] * NQ;
        const int64_t d = d0 + pr[k];
        pvalid[k] = d < p.dim;
        const int64_t dc = pvalid[k] ? d : 0;
        pbias[k] = p.bias ? p.bias[dc * p.sbias] : 0.0f;
        pskip[k] = p.D ? p.D[dc * p.sD] : 0.0f;
        off_u[k] = b * p.su_b + dc * p.su_d + 4 * pq[k];
        off_dl[k] = b * p.sdt_b + dc * p.sdt_d + 4 * pq[k];
        off_z[k] = b * p.sz_b + dc * p.sz_d + 4 * pq[k];
        off_y[k] = b * p.sy_b + dc * p.sy_d + 4 * pq[k];
    }

    // ---- main-loop role: this lane's channel, this wave's states ----
    const int64_t dm = d0 + lane;
    const bool mvalid = dm < p.dim;
    float a2[S], h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = nbase + s;
        a2[s] = 0.0f;
        h[s] = 0.0f;
        if (wave_live && mvalid) {
            a2[s] = p.A[dm * p.sA_d + n] * kLog2e;
            if (p.h0) h[s] = p.h0[b * p.sh0_b + dm * p.sh0_d + n];
        }
    }
    const int64_t offB = b * p.sB_b + (int64_t)nbase * p.sB_n;
    const int64_t offC = b * p.sC_b + (int64_t)nbase * p.sC_n;

    const int64_t nchunks = (L + TC - 1) / TC;
    Quad<T> rq_u[PPT], rq_dl[PPT], rq_z[PPT];  // raw inputs of the next chunk

    auto fetch = [&](int64_t c) {
        const int64_t t0 = c * TC;
        const bool full = t0 + TC <= L;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int64_t t = t0 + 4 * pq[k];
            const int nleft = (int)((L - t) < 4 ? (L - t) : 4);
            if (pvalid[k] && full) {
                rq_u[k].load(u + off_u[k] + t0);
                rq_dl[k].load(dl + off_dl[k] + t0);
                if (z) rq_z[k].load(z + off_z[k] + t0);
                else rq_z[k].zero();
            } else if (pvalid[k] && nleft > 0) {
                rq_u[k].load_tail(u + off_u[k] + t0, nleft);
                rq_dl[k].load_tail(dl + off_dl[k] + t0, nleft);
                if (z) rq_z[k].load_tail(z + off_z[k] + t0, nleft);
                else rq_z[k].zero();
            } else {
                rq_u[k].zero();
                rq_dl[k].zero();
                rq_z[k].zero();
            }
        }
    };

    fetch(0);
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * TC;
        const int steps = (int)((L - t0) < TC ? (L - t0) : TC);

        // prologue: dt and dt*u of this chunk into LDS; keep u and z for the epilogue
        float4 cu[PPT], cz[PPT];
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const float4 x = rq_dl[k].f32();
            cu[k] = rq_u[k].f32();
            cz[k] = rq_z[k].f32();
            float4 dt, dtu;
            dt.x = delta_to_dt(x.x + pbias[k], p.softplus);
            dt.y = delta_to_dt(x.y + pbias[k], p.softplus);
            dt.z = delta_to_dt(x.z + pbias[k], p.softplus);
            dt.w = delta_to_dt(x.w + pbias[k], p.softplus);
            if (4 * pq[k] >= steps) dt = make_float4(0.f, 0.f, 0.f, 0.f);  // beyond L: inert
            dtu = make_float4(dt.x * cu[k].x, dt.y * cu[k].y, dt.z * cu[k].z, dt.w * cu[k].w);
            *reinterpret_cast<float4*>(&s_dt[pr[k] * ROWP + 4 * pq[k]]) = dt;
            *reinterpret_cast<float4*>(&s_dtu[pr[k] * ROWP + 4 * pq[k]]) = dtu;
        }
        __syncthreads();
        if (c + 1 < nchunks) fetch(c + 1);

        // main loop: the recurrence for this wave's states over the chunk
        if (wave_live) {
            float* yrow = &s_yp[(wave * 64 + lane) * ROWP];
            const float* dtrow = &s_dt[lane * ROWP];
            const float* dturow = &s_dtu[lane * ROWP];
            if (steps == TC) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const float4 dt4 = *reinterpret_cast<const float4*>(dtrow + 4 * q);
                    const float4 dtu4 = *reinterpret_cast<const float4*>(dturow + 4 * q);
                    float4 y4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const float4 bq = uniform_quad(Bm, offB + s * p.sB_n + t0 + 4 * q);
                        const float4 cq = uniform_quad(Cm, offC + s * p.sC_n + t0 + 4 * q);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float dA = hw_exp2(f4get(dt4, j) * a2[s]);
                            h[s] = __builtin_fmaf(dA, h[s], f4get(dtu4, j) * f4get(bq, j));
                            f4set(y4, j, __builtin_fmaf(f4get(cq, j), h[s], f4get(y4, j)));
                        }
                    }
                    *reinterpret_cast<float4*>(yrow + 4 * q) = y4;
                }
            } else {
                for (int i = 0; i < steps; ++i) {
                    const float dt = dtrow[i], dtu = dturow[i];
                    float yv = 0.0f;
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const float bv = lane_load(Bm, offB + s * p.sB_n + t0 + i);
                        const float cv = lane_load(Cm, offC + s * p.sC_n + t0 + i);
                        const float dA = hw_exp2(dt * a2[s]);
                        h[s] = __builtin_fmaf(dA, h[s], dtu * bv);
                        yv = __builtin_fmaf(cv, h[s], yv);
                    }
                    yrow[i] = yv;
                }
            }
        }
        __syncthreads();

        // epilogue: sum the waves' partial outputs, skip, gate, store
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int tq = 4 * pq[k];
            if (!pvalid[k] || tq >= steps) continue;
            float4 acc = *reinterpret_cast<const float4*>(&s_yp[pr[k] * ROWP + tq]);
            for (int w = 1; w < w_live; ++w) {
                const float4 v = *reinterpret_cast<const float4*>(&s_yp[(w * 64 + pr[k]) * ROWP + tq]);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            acc.x = __builtin_fmaf(pskip[k], cu[k].x, acc.x);
            acc.y = __builtin_fmaf(pskip[k], cu[k].y, acc.y);
            acc.z = __builtin_fmaf(pskip[k], cu[k].z, acc.z);
            acc.w = __builtin_fmaf(pskip[k], cu[k].w, acc.w);
            if (z) {
                acc.x *= silu_f(cz[k].x);
                acc.y *= silu_f(cz[k].y);
                acc.z *= silu_f(cz[k].z);
                acc.w *= silu_f(cz[k].w);
            }
            float* yp = p.y + off_y[k] + t0;
            if (tq + 4 <= steps) {
                *reinterpret_cast<float4*>(yp) = acc;
            } else {
                const int nleft = steps - tq;
                yp[0] = acc.x;
                if (nleft > 1) yp[1] = acc.y;
                if (nleft > 2) yp[2] = acc.z;
            }
        }
    }

    if (p.last_state && wave_live && mvalid) {
        float* ls = p.last_state + b * p.sls_b + dm * p.sls_d + nbase;
#pragma unroll
        for (int s = 0; s < S; ++s) ls[s] = h[s];
    }
}

// ---------------------------------------------------------------------------------------------
// host side

inline int64_t tiled_workspace_bytes(const mamba_scan_shape&, uint32_t) { return 0; }

inline int tiled_states_per_wave(int64_t N) {
    if (N <= 8) return 1;
    if (N <= 16) return 2;
    if (N <= 32) return 4;
    if (N <= 64) return 8;
    return 0;
}

inline bool aligned(const void* ptr, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0; }

template <typename T>
bool tiled_eligible(const ScanParams& q) {
    const int S = tiled_states_per_wave(q.dstate);
    if (S == 0 || q.dstate % S != 0) return false;
    const uintptr_t vec = sizeof(T) * 4;  // one step quad
    const auto quad_ok = [&](const void* ptr, int64_t sb, int64_t sd) {
        return ptr == nullptr || (aligned(ptr, vec) && sb % 4 == 0 && sd % 4 == 0);
    };
    if (!quad_ok(q.u, q.su_b, q.su_d) || !quad_ok(q.delta, q.sdt_b, q.sdt_d) || !quad_ok(q.z, q.sz_b, q.sz_d))
        return false;
    if (!aligned(q.y, 16) || q.sy_b % 4 != 0 || q.sy_d % 4 != 0) return false;
    // B/C are read as aligned dwords through the scalar cache
    if (!aligned(q.B, 4) || !aligned(q.C, 4)) return false;
    if (sizeof(T) == 2 && (q.sB_b % 2 || q.sB_n % 2 || q.sC_b % 2 || q.sC_n % 2)) return false;
    if (q.batch * ((q.dim + 63) / 64) > 0x7fffffff) return false;
    return true;
}

template <typename T, int S>
int launch_tiled_s(const ScanParams& q, hipStream_t stream) {
    constexpr int W = 8, TC = 32;
    const int64_t groups = q.batch * ((q.dim + 63) / 64);
    void* args[] = {const_cast<ScanParams*>(&q)};
    const void* fn = reinterpret_cast<const void*>(&scan_tiled_kernel<T, S, W, TC>);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * W), args, 0, stream) == hipSuccess
               ? MAMBA_SCAN_OK
               : MAMBA_SCAN_ERR_LAUNCH;
}

template <typename T>
int launch_tiled(const ScanParams& q, const mamba_scan_ptrs*, uint32_t, hipStream_t stream) {
    if (!tiled_eligible<T>(q)) return MAMBA_SCAN_ERR_UNSUPPORTED;
    switch (tiled_states_per_wave(q.dstate)) {
        case 1: return launch_tiled_s<T, 1>(q, stream);
        case 2: return launch_tiled_s<T, 2>(q, stream);
        case 4: return launch_tiled_s<T, 4>(q, stream);
        case 8: return launch_tiled_s<T, 8>(q, stream);
        default: return MAMBA_SCAN_ERR_UNSUPPORTED;
    }
}

}  // namespace mscan
